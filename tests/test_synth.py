"""The seeded input generator: determinism and the stated distributions."""
import numpy as np
import torch

from quantized_moe_top_amd import synth
from oracle_pins import unpack_codes_bytewise


def test_deterministic():
    a, b = synth.make_layer("tiny_t16"), synth.make_layer("tiny_t16")
    for name in ("x", "logits"):
        assert torch.equal(getattr(a, name), getattr(b, name))
    for bank in ("gate", "up", "down"):
        for f in ("qweight", "scales", "biases"):
            assert torch.equal(getattr(getattr(a, bank), f), getattr(getattr(b, bank), f))


def test_shapes_and_distributions():
    lay = synth.make_layer("tiny_t16")
    assert lay.x.shape == (16, 256) and lay.x.dtype == torch.bfloat16
    assert lay.logits.shape == (16, 8) and lay.logits.dtype == torch.float32
    assert lay.gate.qweight.shape == (8, 128, 32) and lay.down.qweight.shape == (8, 256, 16)
    assert lay.gate.scales.shape == (8, 128, 8)
    q = unpack_codes_bytewise(lay.gate.qweight.numpy())
    hist = np.bincount(q.ravel(), minlength=16)
    assert hist.size == 16 and hist.min() > 0.8 * hist.mean()
    s = lay.up.scales.float()
    assert float(s.min()) >= 0.005 * 0.99 and float(s.max()) <= 0.02 * 1.01
    # bias is -8 * scale exactly
    assert torch.equal(lay.up.biases.float(), -8.0 * lay.up.scales.float())


def test_pack_roundtrip():
    rng = np.random.default_rng(0)
    q = rng.integers(0, 16, size=(3, 5, 64), dtype=np.uint8)
    assert np.array_equal(unpack_codes_bytewise(synth.pack_codes(q)), q)


def test_heavy_rows_and_imbalance():
    lay = synth.make_custom(T=1000, H=64, I=32, E=8, k=2, G=32, seed=3, router="weight",
                            heavy_frac=0.01, heavy_mul=30.0)
    assert lay.logits is None and lay.router_weight.shape == (8, 64)
    big = (lay.x.float().abs().amax(1) > 20).sum().item()
    assert 5 <= big <= 10  # 10 rows scaled x30; a N(0,1)*30 row almost surely exceeds 20
    lay = synth.make_custom(T=64, H=64, I=32, E=16, k=4, G=32, seed=4, zipf=True, empty_mod4=True)
    assert torch.isinf(lay.logits[:, 3::4]).all() and torch.isfinite(lay.logits[:, 0::4]).all()
    m = lay.logits[:, 0::4].mean(0)
    assert m[0] > m[-1] + 3.0  # -2.2 ln(e+1) bias
