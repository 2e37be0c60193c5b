"""moe_ffn_forward_noalloc (the layer with the library's fixed scratch area
as its workspace) against moe_ffn_forward with a caller's workspace, through
the C ABI: the same kernels on the same inputs, so the outputs must be
identical bit for bit.  Two calls in a row, the second smaller than the
first (the area keeps the first call's contents), on the MFMA path, at
decode sizes and with the router on the device."""
import ctypes

import pytest
import torch

from quantized_moe_top_amd import _lib, api, synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(big, small):
    out = []
    for cfg in (big, small):
        lay = api.pack_layer(synth.make_custom(**cfg).to(DEV))
        ref = api.ffn_forward(lay).clone()
        y = torch.full_like(ref, float("nan"))
        api.ffn_forward_noalloc(lay, y=y)
        torch.cuda.synchronize()
        out.append((ref, y))
    return out


@pytest.mark.parametrize("kind", ["mfma", "decode", "router"])
def test_noalloc_matches_workspace_entry(kind):
    cfgs = {
        "mfma": (dict(T=300, H=512, I=256, E=16, k=4, G=64, seed=201),
                 dict(T=40, H=512, I=256, E=16, k=4, G=64, seed=202)),
        "decode": (dict(T=8, H=2048, I=512, E=128, k=8, G=64, seed=203),
                   dict(T=1, H=2048, I=512, E=128, k=8, G=64, seed=204)),
        "router": (dict(T=512, H=2048, I=512, E=128, k=8, G=64, seed=205, router="weight"),
                   dict(T=96, H=1024, I=256, E=32, k=4, G=32, seed=206, router="weight")),
    }[kind]
    for ref, y in _pair(*cfgs):
        assert torch.equal(y, ref)


def test_noalloc_rejects_a_layer_beyond_the_area():
    """A layer whose workspace exceeds the fixed area is refused before
    anything is enqueued: y keeps its contents."""
    L = _lib.load()
    lay = api.pack_layer(synth.make_custom(T=4096, H=2048, I=512, E=16, k=8, G=64, seed=207).to(DEV))
    assert api.ffn_workspace_bytes(lay) > L.moe_ffn_noalloc_max_bytes()
    y = torch.full((lay.T, lay.H), 7.0, device=DEV)
    st = L.moe_ffn_forward_noalloc(ctypes.byref(api.make_layer_struct(lay, lay.T)), lay.x.data_ptr(),
                                   lay.logits.data_ptr(), y.data_ptr(), None, api._stream())
    assert st == -3  # MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
