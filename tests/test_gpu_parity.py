"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer outputs (routing ids, counts, offsets, scatter permutation, block
map) must be bit-exact; floating-point outputs must meet relative L2 <= 5e-3
and max abs <= 2e-2 * rms(oracle).  Small layers are compared element by
element everywhere; the full-size workloads are compared on every routing
structure and on sampled output rows the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (MAX_ABS_OVER_RMS, REL_L2_MAX, assert_fp_close, assert_weights_close, cpu, f32_ulp,
                         h_natural, h_values, router_error_bound, say)
from oracle_pins import check_blocks_invariants
from quantized_moe_top_amd import api, synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def on_dev(layer):
    return layer.to(DEV)


def compare_blocks(gpu: dict, ref: dict, tag: str):
    for key in ("counts", "offsets", "sorted_pairs", "pair_slot"):
        got = cpu(gpu[key])
        assert np.array_equal(got, ref[key]), f"{tag}: {key} differs"
    nb = int(cpu(gpu["num_blocks"])[0])
    assert nb == ref["num_blocks"], f"{tag}: num_blocks {nb} != {ref['num_blocks']}"
    assert np.array_equal(cpu(gpu["blocks"])[:nb], ref["blocks"]), f"{tag}: block map differs"


# -------------------------------------------------------------- weight pack --
def packed_sb_reference(scales: torch.Tensor, biases: torch.Tensor, G: int) -> np.ndarray:
    """The packed (scale, bias) words and tail of include/moe_w4.h, derived
    with NumPy: per expert the power of two 2^c that puts the largest
    |bias| + 32 |scale| in [2^13, 2^14); each word fp16(2^c s) | fp16(2^c b -
    32 2^c s) << 16 when that offset is an fp16 value for every group of the
    expert, else fp16(2^c s) | fp16(2^c b) << 16; tail float 2^-c [E], then
    the general flags [E], padded to 16 bytes."""
    E, N, gpr = scales.shape
    s = scales.float().numpy().astype(np.float64)
    b = biases.float().numpy().astype(np.float64)
    words = np.empty((E, N, gpr), np.uint32)
    unscale = np.empty(E, np.float32)
    general = np.empty(E, np.uint32)
    for e in range(E):
        m = float(np.max(np.abs(b[e]) + 32.0 * np.abs(s[e])))
        c = 0 if m == 0 else int(np.clip(14 - np.frexp(m)[1], -100, 100))
        se, be = np.ldexp(s[e], c), np.ldexp(b[e], c)
        off = be - 32.0 * se
        exact = bool(np.all(off.astype(np.float16).astype(np.float64) == off))
        hs = se.astype(np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
        hi = (off if exact else be).astype(np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
        words[e] = hs | (hi << 16)
        unscale[e] = np.float32(np.ldexp(1.0, -c))
        general[e] = 0 if exact else 1
    body = words.reshape(E, N // 128, 128, gpr).transpose(0, 1, 3, 2).reshape(-1)
    tail = np.concatenate([unscale.view(np.uint32), general])
    pad = (-len(tail)) % 4
    return np.concatenate([body, tail, np.zeros(pad, np.uint32)])


@pytest.mark.parametrize("E,N,K,G,bias", [(3, 128, 256, 32, "free"), (2, 384, 384, 128, "free"),
                                          (4, 256, 128, 64, "m8"), (3, 128, 256, 64, "mixed")])
def test_pack_layout(E, N, K, G, bias):
    """moe_w4_pack against the packed layout's definition (include/moe_w4.h),
    rearranged independently with NumPy: codes, (scale, bias) words, each
    expert's power of two and dequantisation form."""
    g = torch.Generator().manual_seed(E * 1000 + N + K + G)
    scales = (torch.randn((E, N, K // G), generator=g) * 0.01).to(torch.bfloat16)
    if bias == "m8":
        biases = (-8.0 * scales.float()).to(torch.bfloat16)
    else:
        biases = torch.randn((E, N, K // G), generator=g).to(torch.bfloat16)
        if bias == "mixed":  # expert 0 exact (bias = -8 scale), the others general
            biases[0] = (-8.0 * scales[0].float()).to(torch.bfloat16)
    bank = synth.W4Bank(torch.randint(-2**31, 2**31 - 1, (E, N, K // 8), generator=g, dtype=torch.int64).to(torch.int32),
                        scales, biases)
    pb = api.pack_bank(bank.to(DEV), G)
    torch.cuda.synchronize()
    q = bank.qweight.numpy().view(np.uint32)
    # words [E][N/128][K/64][4][32][2][4] from q [E][N][K/8]: column 128c + 32u + cc, half h,
    # word w -> q[.., 8s + 4h + w]
    want = q.reshape(E, N // 128, 4, 32, K // 64, 2, 4).transpose(0, 1, 4, 2, 3, 5, 6).reshape(-1)
    want = (want << np.uint32(5)) | (want >> np.uint32(27))  # each word rotated left by 5 bits
    assert np.array_equal(cpu(pb.words).view(np.uint32), want)
    ref = packed_sb_reference(scales, biases, G)
    got = cpu(pb.sb).view(np.uint32)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)
    tail = ref[E * N * (K // G):]
    if bias == "m8":
        assert np.all(tail[E:2 * E] == 0)  # every expert exact
    if bias == "mixed":
        assert tail[E] == 0 and np.all(tail[E + 1:2 * E] == 1)


# ------------------------------------------------------------------ routing --
@pytest.mark.parametrize("name", ["tiny_t16", "decode_t1", "decode_t8", "imbalanced_t8192"])
def test_route_given_logits(orc, name):
    lay = synth.make_layer(name)
    logits = lay.logits.to(DEV)
    ids, w, _ = api.route(lay.k, logits=logits)
    torch.cuda.synchronize()
    rid, rw = orc.route(lay.logits, lay.k)
    assert np.array_equal(cpu(ids), rid)
    assert_weights_close(cpu(w), rw)


def test_route_hand_cases():
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "route_hand.json")
    import math
    for case in json.load(open(path))["cases"]:
        l = torch.tensor([[float(v) for v in r] for r in case["logits"]], dtype=torch.float32)
        ids, w, _ = api.route(case["k"], logits=l.to(DEV))
        assert cpu(ids).tolist() == case["ids"], case["note"]
        exp_w = np.array([[eval(e, {"__builtins__": {}}, {"exp": math.exp}) for e in r]
                          for r in case["weights_closed_form"]])
        assert np.all(np.abs(cpu(w) - exp_w) <= 4 * f32_ulp(exp_w)), case["note"]


# T = 257, 6000 and 20000 give routing chunks of 8, 24 and 80 tokens: the
# top-k runs with 64, 16 and 8 lanes per token (20000: a full pass of 64
# tokens and a partial one).
@pytest.mark.parametrize("T", [257, 6000, 20000])
@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (256, 16), (16, 16), (5, 1), (200, 3)])
def test_route_ties_and_inf(orc, E, k, T):
    g = torch.Generator().manual_seed(E * 31 + k + T)
    l = torch.randn((T, E), generator=g)
    l[::2, : E // 2] = torch.round(l[::2, : E // 2])          # many exact ties
    l[1::3] = 0.25                                           # whole rows equal
    if E > k + 4:
        l[::5, k + 1:] = float("-inf")
    ids, w, _ = api.route(k, logits=l.to(DEV))
    rid, rw = orc.route(l, k)
    assert np.array_equal(cpu(ids), rid)
    assert_weights_close(cpu(w), rw)


def check_router_chain(orc, x, wr, k):
    """Router logits on the device: within the fp32 summation bound of the
    oracle's; routing of the device logits is bit-exact with the oracle's
    routing of those same logits; tokens whose top-k set changes between
    the two logit sets sit on a near tie."""
    ids, w, logits = api.route(k, x=x.to(DEV), router_weight=wr.to(DEV))
    torch.cuda.synchronize()
    l_gpu = cpu(logits)
    l_ref = orc.router_logits(x, wr)
    bound = router_error_bound(x, wr) + f32_ulp(l_ref)
    err = np.abs(l_gpu.astype(np.float64) - l_ref)
    say(f"  logits max err {err.max():.3e}, max bound {bound.max():.3e}")
    assert np.all(err <= bound)
    rid, rw = orc.route(l_gpu, k)
    assert np.array_equal(cpu(ids), rid)
    assert_weights_close(cpu(w), rw)
    oid, _ = orc.route(l_ref, k)
    changed = np.nonzero(np.any(np.sort(oid, 1) != np.sort(rid, 1), axis=1))[0]
    srt = -np.sort(-l_ref, axis=1)
    for t in changed:
        assert srt[t, k - 1] - srt[t, k] <= 2 * bound[t].max()
    say(f"  tokens whose top-k set differs: {len(changed)}")


@pytest.mark.parametrize("name", ["prefill_t512"])
def test_router_gemm_chain(orc, name):
    lay = synth.make_layer(name)
    check_router_chain(orc, lay.x, lay.router_weight, lay.k)


# The router tile follows T (32x32 with the k steps split over the waves,
# 64x64, 64x128, 128x128); ragged T and E, E not a multiple of 32, small H.
@pytest.mark.parametrize("T,E,H,k", [(3, 256, 128, 16), (40, 33, 384, 3), (1000, 100, 256, 8),
                                     (8192, 128, 2048, 8), (16384, 128, 1024, 8),
                                     (32768, 128, 2048, 8), (20001, 200, 640, 4)])
def test_router_tiles(orc, T, E, H, k):
    g = torch.Generator().manual_seed(T + E + H)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16)
    wr = (0.02 * torch.randn((E, H), generator=g)).to(torch.bfloat16)
    check_router_chain(orc, x, wr, k)


# ------------------------------------------- histogram / scan / scatter ---
@pytest.mark.parametrize("T,k,E,BM", [(16, 2, 8, 32), (1, 8, 128, 8), (8, 8, 128, 8), (512, 8, 128, 64),
                                      (300, 4, 16, 16), (8192, 8, 128, 128), (2500, 3, 7, 1),
                                      (1025, 8, 256, 128), (4097, 16, 64, 32),
                                      # chunks of 2,240 and 2,560 pairs: each wave ranks 5 rounds of 64,
                                      # past the 4 whose ids are read up front
                                      (70000, 8, 128, 128), (40000, 16, 64, 64)])
def test_build_blocks(orc, T, k, E, BM):
    g = torch.Generator().manual_seed(T + 7 * E + BM)
    l = torch.randn((T, E), generator=g)
    if E > 8:
        l[:, 3::4] = float("-inf")                          # empty experts
    l[:, 0] += 3.0                                           # a hot expert: several tiles
    rid, _ = orc.route(l, k)
    ids = torch.from_numpy(rid).to(DEV)
    bb = api.build_blocks(ids, E, BM)
    bb2 = api.build_blocks(ids, E, BM)
    torch.cuda.synchronize()
    ref = orc.build_blocks(rid, E, BM)
    compare_blocks(bb, ref, f"T={T} E={E} BM={BM}")
    for key in bb:                                           # deterministic
        if key != "blocks":
            assert torch.equal(bb[key], bb2[key]), key
    nb = ref["num_blocks"]
    assert torch.equal(bb["blocks"][:nb], bb2["blocks"][:nb])


# ------------------------------------------------------ grouped W4 GEMMs ---
GEMM_CASES = {
    "tiny_t16": lambda: synth.make_layer("tiny_t16"),
    "decode_t1": lambda: synth.make_layer("decode_t1"),
    "decode_t8": lambda: synth.make_layer("decode_t8"),
    "ragged_t300_g64": lambda: synth.make_custom(T=300, H=512, I=256, E=16, k=4, G=64, seed=21),
    "ragged_t100_g128": lambda: synth.make_custom(T=100, H=1024, I=256, E=32, k=6, G=128, seed=22),
    "ragged_t77_g32": lambda: synth.make_custom(T=77, H=512, I=384, E=8, k=2, G=32, seed=23),
    "gemv_t5_g32": lambda: synth.make_custom(T=5, H=768, I=384, E=16, k=4, G=32, seed=24),
    "mfma_t9": lambda: synth.make_custom(T=9, H=512, I=256, E=4, k=2, G=64, seed=25),
    # general affine weights (the general dequantisation): zero points m ~ U(2, 14), free biases
    "zeropoint_t300_g64": lambda: synth.make_custom(T=300, H=512, I=256, E=16, k=4, G=64, seed=26,
                                                    bias="zeropoint"),
    "free_t100_g128": lambda: synth.make_custom(T=100, H=1024, I=256, E=32, k=6, G=128, seed=27,
                                                bias="free"),
    "zeropoint_gemv_t5_g32": lambda: synth.make_custom(T=5, H=768, I=384, E=16, k=4, G=32, seed=28,
                                                       bias="zeropoint"),
    # |h| past the fp16 range on the x30 rows (scaled h blocks, the down
    # kernels' scaled path), and h far below fp16's normal range
    "large_h_t300": lambda: synth.make_custom(T=300, H=512, I=256, E=16, k=4, G=64, seed=29,
                                              scale=(0.1, 0.4), heavy_frac=0.05, heavy_mul=30.0),
    "tiny_h_gemv_t5": lambda: synth.make_custom(T=5, H=768, I=384, E=16, k=4, G=32, seed=30,
                                                scale=(5e-6, 2e-5)),
}


def block_m_for(T, k, E):
    avg = T * k // E
    if T <= 8:
        return 8
    return 32 if avg <= 16 else 64 if avg <= 64 else 128


@pytest.mark.parametrize("name", list(GEMM_CASES))
def test_grouped_gemms(orc, name):
    lay = GEMM_CASES[name]()
    d = on_dev(lay)
    rid, rw = orc.route(lay.logits, lay.k)
    ids, w = torch.from_numpy(rid).to(DEV), torch.from_numpy(rw).to(DEV)
    for BM in sorted({block_m_for(lay.T, lay.k, lay.E)} | ({32, 64, 128} if lay.T > 8 else {1, 8})):
        say(f"  {name}: block_m {BM}")
        bb = api.build_blocks(ids, lay.E, BM)
        kw = dict(T=lay.T, top_k=lay.k, E=lay.E, group_size=lay.G, block_m=BM)
        h, hx = api.w4_grouped_gemm(api.MOE_GEMM_GATE_UP_SWIGLU, d.x, d.gate, d.up, bb["sorted_pairs"],
                                    bb["blocks"], bb["num_blocks"], **kw)
        ys = api.w4_grouped_gemm(api.MOE_GEMM_DOWN, h, d.down, None, bb["sorted_pairs"],
                                 bb["blocks"], bb["num_blocks"], topk_weights=w.reshape(-1), h_exp=hx, **kw)
        torch.cuda.synchronize()
        sp = cpu(bb["sorted_pairs"])
        tokens = (sp // lay.k).astype(np.int32)
        experts = rid.reshape(-1)[sp].astype(np.int32)
        h_ref = orc.expert_hidden(lay.x, tokens, experts, lay.gate, lay.up, lay.G)
        P = lay.T * lay.k
        h_gpu = h_values(cpu(h), cpu(hx)[:P * (lay.I // 16)].view(np.int8).reshape(P, lay.I // 16))
        assert_fp_close(h_gpu, h_ref, f"{name} BM={BM} h")
        # down projection fed with the device's own h (isolates S7)
        o_ref = orc.expert_down(h_gpu, experts, lay.down, lay.G) * rw.reshape(-1)[sp][:, None]
        assert_fp_close(cpu(ys), o_ref, f"{name} BM={BM} y_sorted")


# ---------------------------------------------------------- whole layer ---
def layer_output_check(orc, lay, y, info, tokens=None, strata=None):
    """Routing structures bit-exact, then y against the oracle on `tokens`
    (all when None).  With `strata` = [(token list, population share)], the
    rms of the full oracle output is estimated per stratum."""
    l_used = cpu(info["logits"]).astype(np.float32)
    if lay.router_weight is not None:
        # the device logits within the fp32 summation bound of the oracle's,
        # on every row (or, for large T, on the rows whose output is checked)
        rows = np.arange(lay.T) if lay.T <= 4096 or tokens is None else np.asarray(tokens)
        xr = lay.x[torch.from_numpy(rows.astype(np.int64))]
        l_ref = orc.router_logits(xr, lay.router_weight)
        bound = router_error_bound(xr, lay.router_weight) + f32_ulp(l_ref)
        assert np.all(np.abs(l_used[rows].astype(np.float64) - l_ref) <= bound)
    else:
        assert np.array_equal(l_used, cpu(lay.logits))
    rid, rw = orc.route(l_used, lay.k)
    assert np.array_equal(cpu(info["topk_ids"]), rid)
    assert_weights_close(cpu(info["topk_weights"]), rw)
    ref = orc.build_blocks(rid, lay.E, info["block_m"])
    compare_blocks(info, ref, lay.name)
    check_blocks_invariants(rid, lay.E, info["block_m"], {
        **ref, "sorted_pairs": cpu(info["sorted_pairs"]), "pair_slot": cpu(info["pair_slot"])})
    yg = cpu(y)
    if tokens is None:
        y_ref = orc.ffn(lay.x, rid, rw, lay.gate, lay.up, lay.down, lay.G)
        assert_fp_close(yg, y_ref, f"{lay.name} y")
        return
    tokens = np.asarray(tokens, np.int32)
    y_ref = orc.ffn(lay.x, rid, rw, lay.gate, lay.up, lay.down, lay.G, tokens=tokens)
    rms = None
    if strata:
        ms, pos = 0.0, 0
        for toks, share in strata:
            n = len(toks)
            ms += share * float(np.mean(y_ref[pos:pos + n].astype(np.float64) ** 2))
            pos += n
        rms = float(np.sqrt(ms))
    assert_fp_close(yg[tokens], y_ref, f"{lay.name} y (sampled {len(tokens)} rows)", rms_ref=rms)


@pytest.mark.parametrize("name", ["tiny_t16", "decode_t1", "decode_t8", "prefill_t512"])
def test_ffn_forward_full(orc, name):
    lay = synth.make_layer(name)
    y, info = api.ffn_forward(on_dev(lay), info=True)
    torch.cuda.synchronize()
    assert info["path"] == (1 if lay.T <= 8 else 0)
    layer_output_check(orc, lay, y, info)
    # the combine is exactly the fp32 sum, in choice order, of the weighted
    # expert outputs at each token's slots (block floating point on the MFMA
    # path: its values are exact in fp32)
    ys = info["y_sorted"]
    ys = cpu(ys if ys.dtype == torch.float32 else api.unpack_y16e(ys, info["y_sorted_exp"]))
    ps = cpu(info["pair_slot"]).reshape(lay.T, lay.k)
    acc = np.zeros((lay.T, lay.H), np.float32)
    for j in range(lay.k):
        acc = acc + ys[ps[:, j]]
    assert np.array_equal(cpu(y), acc)


def test_ffn_forward_imbalanced_t8192(orc):
    """Zipf load with a quarter of the experts empty: routing structures
    bit-exact and every one of the 8192 output rows against the oracle."""
    lay = synth.make_layer("imbalanced_t8192")
    y, info = api.ffn_forward(on_dev(lay), info=True)
    torch.cuda.synchronize()
    counts = cpu(info["counts"])
    assert np.all(counts[3::4] == 0) and counts.sum() == lay.T * lay.k
    layer_output_check(orc, lay, y, info)


@pytest.mark.parametrize("layer_index", [0, 1, 2, 3])
def test_ffn_forward_longctx_t32768(orc, layer_index):
    """Each of the four independently seeded long-context layers.  The 1% of
    rows scaled x30 are the precision canary: every one of them (328) is
    checked against the oracle, with 64 of the other rows.  The max abs error
    is taken over every checked row; the rms of the whole oracle output
    combines the exact mean square of the heavy rows with an estimate of the
    normal rows' from the 64 checked (the heavy rows carry more than 99.9% of
    the mean square, so the estimate moves the bound by well under 0.1%)."""
    lay = synth.make_layer("longctx_t32768", layer_index)
    y, info = api.ffn_forward(on_dev(lay), info=True)
    torch.cuda.synchronize()
    x = lay.x.float()
    heavy = torch.nonzero(x.abs().amax(1) > 12.0).flatten().numpy()  # the x30 rows
    assert len(heavy) == round(0.01 * lay.T)
    normal = np.setdiff1d(np.arange(lay.T), heavy)
    g = np.random.default_rng(32768 + layer_index)
    tn = np.sort(g.choice(normal, 64, replace=False))
    share_h = len(heavy) / lay.T
    layer_output_check(orc, lay, y, info, tokens=np.concatenate([heavy, tn]),
                       strata=[(heavy, share_h), (tn, 1 - share_h)])


# ------------------------------------------------- general affine weights ---
# Banks whose bias is not -8 * scale: zero points m ~ U(2, 14) per group
# (bias = -m * scale) or biases drawn independently of the scale, at the
# prefill workload's shape, at group sizes 32 and 128, at decode sizes, and
# with x30 rows.  The library takes the general dequantisation for them.
GENERAL_CASES = {
    "prefill_t512_zeropoint": dict(T=512, H=2048, I=512, E=128, k=8, G=64, seed=101, router="weight",
                                   bias="zeropoint"),
    "g32_zeropoint": dict(T=300, H=512, I=256, E=16, k=4, G=32, seed=102, bias="zeropoint"),
    "g128_free": dict(T=100, H=1024, I=256, E=32, k=6, G=128, seed=103, bias="free"),
    "g32_free_t77": dict(T=77, H=512, I=384, E=8, k=2, G=32, seed=104, bias="free"),
    "decode_t1_zeropoint": dict(T=1, H=2048, I=512, E=128, k=8, G=64, seed=105, bias="zeropoint"),
    "decode_t8_free_g128": dict(T=8, H=1024, I=256, E=32, k=4, G=128, seed=106, bias="free"),
    "zeropoint_t2000": dict(T=2000, H=2048, I=512, E=32, k=4, G=64, seed=107, router="weight",
                            bias="zeropoint"),
}


@pytest.mark.parametrize("case", list(GENERAL_CASES))
def test_ffn_general_bias(orc, case):
    lay = synth.make_custom(**GENERAL_CASES[case])
    y, info = api.ffn_forward(on_dev(lay), info=True)
    torch.cuda.synchronize()
    layer_output_check(orc, lay, y, info)


# --------------------------------------------------- ranges of h and weights --
# Scales far from the workloads' (2e-3 .. 1e-2): tiny ones put h far below
# fp16's normal range, large ones with x30 rows put |h| far beyond 65504
# (up to about 1e9 here); the packed weights are rescaled per expert and h
# carries exponents per 16 columns, so both stay within the bar, on the
# MFMA path (T = 300, 512) and at decode sizes (T = 1, 8).
RANGE_CASES = {
    "tiny_scales_t300": dict(T=300, H=512, I=256, E=16, k=4, G=64, seed=111, scale=(5e-6, 2e-5)),
    "tiny_scales_decode_t1": dict(T=1, H=2048, I=512, E=128, k=8, G=64, seed=112, scale=(5e-6, 2e-5)),
    "large_h_t512": dict(T=512, H=2048, I=512, E=128, k=8, G=64, seed=113, router="weight",
                         scale=(0.1, 0.4), heavy_frac=0.01, heavy_mul=30.0),
    "large_h_decode_t8": dict(T=8, H=2048, I=512, E=128, k=8, G=64, seed=114, scale=(0.1, 0.4),
                              heavy_frac=0.25, heavy_mul=30.0),
    "huge_scales_t300": dict(T=300, H=512, I=256, E=16, k=4, G=32, seed=115, scale=(200.0, 800.0),
                             bias="zeropoint"),
}


@pytest.mark.parametrize("case", list(RANGE_CASES))
def test_ffn_scale_range(orc, case):
    lay = synth.make_custom(**RANGE_CASES[case])
    y, info = api.ffn_forward(on_dev(lay), info=True)
    torch.cuda.synchronize()
    hx = cpu(info["h_exp"])
    say(f"  {case}: h exponents in [{hx.min()}, {hx.max()}], {np.mean(hx != 0) * 100:.1f}% nonzero")
    layer_output_check(orc, lay, y, info)


# ------------------------------------------------------------ edge cases ---
def test_ffn_all_tokens_one_expert(orc):
    """Every token picks expert 0 first: one expert with T rows (many tiles,
    ragged tail) next to near-empty ones."""
    lay = synth.make_custom(T=333, H=512, I=256, E=16, k=2, G=64, seed=31)
    lay.logits[:, 0] += 100.0
    y, info = api.ffn_forward(on_dev(lay), info=True)
    torch.cuda.synchronize()
    assert int(cpu(info["counts"])[0]) == 333
    layer_output_check(orc, lay, y, info)


def test_ffn_k_equals_e_and_k1(orc):
    for lay in (synth.make_custom(T=40, H=256, I=128, E=4, k=4, G=32, seed=32),
                synth.make_custom(T=40, H=256, I=128, E=4, k=1, G=32, seed=33)):
        y, info = api.ffn_forward(on_dev(lay), info=True)
        torch.cuda.synchronize()
        layer_output_check(orc, lay, y, info)


def test_ffn_router_split(orc):
    """Router weight at small T: the router sums ranges of H separately (8 or
    4 ranges here) and the routing kernel adds them; decode sizes take the
    path whose gate/up launch also routes and builds the block map."""
    for (T, H, E, k) in [(5, 2048, 128, 8), (100, 1024, 64, 4), (3, 512, 200, 6)]:
        lay = synth.make_custom(T=T, H=H, I=256, E=E, k=k, G=64, seed=40 + T, router="weight")
        y, info = api.ffn_forward(on_dev(lay), info=True)
        torch.cuda.synchronize()
        layer_output_check(orc, lay, y, info)


def test_ffn_decode_edges(orc):
    """Decode sizes (routing and block map inside the gate/up launch): the most pairs it
    takes (T = 8, k = 16), one expert chosen of two, and an odd E."""
    for (T, E, k) in [(8, 256, 16), (1, 2, 1), (7, 5, 3)]:
        lay = synth.make_custom(T=T, H=256, I=128, E=E, k=k, G=32, seed=50 + T + E)
        y, info = api.ffn_forward(on_dev(lay), info=True)
        torch.cuda.synchronize()
        assert info["path"] == 1
        layer_output_check(orc, lay, y, info)


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_ffn_decode_ties(orc, T):
    """Decode-size routing inside the gate/up launch on logits with exact
    ties, a row of equal values, signed zeros and -inf entries, at E = 128,
    256, 5 and k = E = 16: ids bit-exact with the oracle, and ids and weights
    identical, bit for bit, to moe_route's top-k on the same logits."""
    import dataclasses
    for (E, k) in [(128, 8), (256, 16), (5, 3), (16, 16)]:
        if T * k > 128:
            continue
        lay = synth.make_custom(T=T, H=256, I=128, E=E, k=k, G=32, seed=80 + T + E)
        g = torch.Generator().manual_seed(7 * E + T)
        l = torch.randn((T, E), generator=g)
        l[::2, : E // 2] = torch.round(l[::2, : E // 2])       # exact ties, signed zeros
        l[T - 1, E // 3:] = 0.25                                # equal values
        if E > k + 4:
            l[0, k + 1::2] = float("-inf")
        lay = dataclasses.replace(lay, logits=l)
        y, info = api.ffn_forward(on_dev(lay), info=True)
        torch.cuda.synchronize()
        assert info["path"] == 1
        layer_output_check(orc, lay, y, info)
        ids, w, _ = api.route(k, logits=l.to(DEV))
        assert torch.equal(info["topk_ids"], ids), (E, k)
        assert torch.equal(info["topk_weights"], w), (E, k)


def test_ffn_decode_two_slabs_per_wave(orc):
    """Decode sizes whose down launch takes two slabs per wave (more
    workgroups than three 8-wave ones per CU hold): T = 7 and 8 at H = 2048,
    and H = 4096 with I = 256 (two 2-slab waves per workgroup), against the
    oracle."""
    for (T, H, I, E, k) in [(7, 2048, 512, 64, 8), (8, 4096, 256, 32, 4)]:
        lay = synth.make_custom(T=T, H=H, I=I, E=E, k=k, G=64, seed=70 + T + H // 1024)
        y, info = api.ffn_forward(on_dev(lay), info=True)
        torch.cuda.synchronize()
        assert info["path"] == 1
        layer_output_check(orc, lay, y, info)


def test_ffn_decode_wide_shapes(orc):
    """Decode sizes at shapes that leave the one-pass kernels: a reduction
    of 8192 in the gate/up launch (more than one pass per item, no
    prefetch), and I = 1152 (more than 16 slabs: the down projection falls
    back to the per-tile GEMV and the combine kernel)."""
    for (T, H, I, E, k) in [(3, 8192, 128, 6, 2), (5, 256, 1152, 8, 3)]:
        lay = synth.make_custom(T=T, H=H, I=I, E=E, k=k, G=64, seed=60 + T)
        y, info = api.ffn_forward(on_dev(lay), info=True)
        torch.cuda.synchronize()
        assert info["path"] == 1
        layer_output_check(orc, lay, y, info)


# ---------------------------------------------- single-launch decode layer --
def _single_vs_two(lay_dev, logits, sync, tag):
    """One call of each path on the same inputs: every output and routing
    structure identical, bit for bit; the counters back at zero, no wait
    given up.  Returns the single-launch y and info."""
    y2, i2 = api.ffn_forward(lay_dev, logits=logits, info=True)
    y1, i1 = api.ffn_forward(lay_dev, logits=logits, info=True, sync=sync)
    torch.cuda.synchronize()
    assert i1["path"] == 1
    assert torch.equal(y1, y2), f"{tag}: y differs"
    for key in ("topk_ids", "topk_weights", "counts", "offsets", "sorted_pairs", "pair_slot"):
        assert torch.equal(i1[key], i2[key]), f"{tag}: {key} differs"
    nb = int(cpu(i1["num_blocks"])[0])
    assert nb == int(cpu(i2["num_blocks"])[0])
    assert torch.equal(i1["blocks"][:nb], i2["blocks"][:nb]), f"{tag}: block map differs"
    assert torch.equal(i1["h"], i2["h"]) and torch.equal(i1["h_exp"], i2["h_exp"]), f"{tag}: h differs"
    assert torch.equal(i1["y_sorted"], i2["y_sorted"]), f"{tag}: y_sorted differs"
    s = cpu(sync)
    assert not s.any(), f"{tag}: counters left {s[np.nonzero(s)]} at {np.nonzero(s)}"
    return y1, i1


@pytest.mark.parametrize("name", ["decode_t1", "decode_t8"])
def test_ffn_single_launch_decode(orc, name):
    """moe_ffn_forward_single (gate/up and down halves in one grid, down
    workgroups waiting on per-expert counters): identical to the two-launch
    layer on every output, on the oracle's bar, and on eight calls in a row
    with fresh logits each (the counters return to zero; h is never read
    before it is stored)."""
    lay = synth.make_layer(name)
    d = on_dev(lay)
    sync = torch.zeros(api.single_sync_ints(), dtype=torch.int32, device=DEV)
    y, info = _single_vs_two(d, d.logits, sync, name)
    layer_output_check(orc, lay, y, info)
    g = torch.Generator().manual_seed(97)
    for i in range(8):
        lg = torch.randn((lay.T, lay.E), generator=g).to(DEV)
        _single_vs_two(d, lg, sync, f"{name} call {i}")


def test_ffn_single_launch_shapes(orc):
    """The single-launch layer at other decode shapes (the most pairs, one
    expert of two, an odd E, a router weight with partial sums), against the
    oracle and the two-launch path; shapes whose halves need workgroups of
    different sizes are refused."""
    sync = torch.zeros(api.single_sync_ints(), dtype=torch.int32, device=DEV)
    cases = [dict(T=8, H=256, I=128, E=256, k=16, G=32, seed=91), dict(T=1, H=256, I=128, E=2, k=1, G=32, seed=92),
             dict(T=7, H=512, I=256, E=5, k=3, G=64, seed=93),
             dict(T=3, H=2048, I=512, E=64, k=4, G=64, seed=94, router="weight")]
    for cfg in cases:
        lay = synth.make_custom(**cfg)
        d = on_dev(lay)
        y, info = _single_vs_two(d, None if lay.router_weight is not None else d.logits, sync, str(cfg))
        layer_output_check(orc, lay, y, info)
    lay = on_dev(synth.make_custom(T=3, H=8192, I=128, E=6, k=2, G=64, seed=95))
    with pytest.raises(RuntimeError, match="workgroups of one size"):
        api.ffn_forward(lay, sync=sync)


# ------------------------------------------------- either side of the layer --
def _bf16_ulp(bits: np.ndarray) -> np.ndarray:
    v = np.abs((bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    return np.where(v > 0, np.ldexp(1.0, np.frexp(v)[1] - 8), 0.0)


def test_rmsnorm(orc):
    """moe_rmsnorm against the oracle (fp64, one rounding): every value
    within one bf16 unit, and almost all identical (fp32 arithmetic moves a
    rounding only for values within ~1e-7 of a rounding boundary)."""
    g = torch.Generator().manual_seed(80)
    for T, H in [(1, 2048), (37, 2048), (300, 256), (5, 8)]:
        x = torch.randn(T, H, generator=g)
        x[::7] *= 30.0
        xb = x.to(torch.bfloat16)
        gamma = (torch.rand(H, generator=g) * 1.5 + 0.25).to(torch.bfloat16)
        got = cpu(api.rmsnorm(xb.to(DEV), gamma.to(DEV), 1e-6).view(torch.int16)).view(np.uint16)
        ref = orc.rmsnorm(xb, gamma, 1e-6)
        gv = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rv = (ref.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.all(np.abs(gv - rv) <= _bf16_ulp(ref)), (T, H)
        same = float(np.mean(got == ref))
        say(f"  rmsnorm T={T} H={H}: {same * 100:.3f}% bit-identical")
        assert same >= 0.999, (T, H, same)


@pytest.mark.parametrize("case", ["mfma_t300", "decode_t5", "router_t40", "decode_router_t3", "router_t9000",
                                  "mfma_t20001", "decode_t1_full", "decode_t8_full"])
def test_ffn_io(orc, case):
    """moe_ffn_forward_io: RMSNorm in front and out = bf16(residual + y)
    behind, against the oracle's normalisation, layer and residual sum.
    Logits given: the routing does not depend on the normalised rows and is
    compared bit-exactly; with a router weight the GPU's logits are routed by
    the oracle and compared bit-exactly, and checked against the oracle's
    logits.  At prefill sizes the router sums r * bf16(x * gamma) * wr (the
    row's factor r applied after the sum): each term's normalised input is
    within 1.5 bf16 units of the oracle's bf16(x * gamma * r) (half a unit of
    x * gamma, scaled by r, is at most one unit of the product; plus the
    oracle's own half unit), and r carries a few fp32 roundings; at decode
    sizes the rows are normalised first (within one unit)."""
    cfg = {"mfma_t300": dict(T=300, H=512, I=256, E=16, k=4, G=64, seed=81),
           "decode_t5": dict(T=5, H=512, I=256, E=16, k=4, G=64, seed=82),
           "router_t40": dict(T=40, H=512, I=256, E=32, k=4, G=64, seed=83, router="weight"),
           "decode_router_t3": dict(T=3, H=256, I=128, E=8, k=2, G=32, seed=84, router="weight"),
           # routing chunks of 40 and 80 tokens: passes of 64 rows, several
           # row pairs per wave in the folded normalisation, a partial pass
           "router_t9000": dict(T=9000, H=256, I=128, E=16, k=4, G=64, seed=85, router="weight"),
           "mfma_t20001": dict(T=20001, H=256, I=128, E=8, k=2, G=32, seed=86),
           # the decode workloads' shape: the normalisation folded into the
           # gate/up launch's staging of x
           "decode_t1_full": dict(T=1, H=2048, I=512, E=128, k=8, G=64, seed=87),
           "decode_t8_full": dict(T=8, H=2048, I=512, E=128, k=8, G=64, seed=88)}[case]
    lay = synth.make_custom(**cfg)
    g = torch.Generator().manual_seed(cfg["seed"] + 100)
    gamma = (torch.rand(lay.H, generator=g) * 1.5 + 0.25).to(torch.bfloat16)
    res = torch.randn(lay.T, lay.H, generator=g).to(torch.bfloat16)
    d = on_dev(lay)
    out = torch.empty((lay.T, lay.H), dtype=torch.bfloat16, device=DEV)
    y, info = api.ffn_forward(d, info=True, norm_weight=gamma.to(DEV), norm_eps=1e-5,
                              residual=res.to(DEV), out=out)
    torch.cuda.synchronize()
    xn = orc.rmsnorm(lay.x, gamma, 1e-5)
    l_used = cpu(info["logits"]).astype(np.float32)
    if lay.router_weight is None:
        assert np.array_equal(l_used, cpu(lay.logits))
    else:
        l_ref = orc.router_logits(xn, lay.router_weight)
        # each normalised input may differ by one bf16 unit: bound the effect
        wr = np.abs(lay.router_weight.float().numpy().astype(np.float64))
        xv = (xn.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        bound = router_error_bound(torch.from_numpy(xv).to(torch.bfloat16), lay.router_weight) + \
            1.5 * (_bf16_ulp(xn) @ wr.T) + 4 * f32_ulp(np.abs(xv) @ wr.T)
        assert np.all(np.abs(l_used.astype(np.float64) - l_ref) <= bound)
    rid, rw = orc.route(l_used, lay.k)
    assert np.array_equal(cpu(info["topk_ids"]), rid)
    assert_weights_close(cpu(info["topk_weights"]), rw)
    y_ref = orc.ffn(xn, rid, rw, lay.gate, lay.up, lay.down, lay.G)
    assert_fp_close(cpu(y), y_ref, f"{case} y")
    out_ref = orc.residual_out(res, y_ref)
    ov = (cpu(out.view(torch.int16)).view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    rv = (out_ref.astype(np.uint32) << 16).view(np.float32)
    # out is rounded to bf16 on both sides: any difference in y can move a
    # sum across a rounding boundary, so each element may also differ by one
    # bf16 unit of out (2^-5 where |out| is in [4, 8))
    ovd, rvd = ov.astype(np.float64), rv.astype(np.float64)
    rms_out = float(np.sqrt(np.mean(rvd ** 2)))
    assert np.linalg.norm(ovd - rvd) <= REL_L2_MAX * np.linalg.norm(rvd), f"{case} out rel L2"
    assert np.all(np.abs(ovd - rvd) <= MAX_ABS_OVER_RMS * rms_out + _bf16_ulp(out_ref)), f"{case} out max abs"
    # out is bf16(residual + y) of the y returned beside it: the fp32 sum
    # rounded to bf16 can differ from the once-rounded exact sum by one unit
    # (double rounding), rarely
    got, exact = cpu(out.view(torch.int16)).view(np.uint16), orc.residual_out(res, cpu(y))
    gv = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ev = (exact.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(gv - ev) <= _bf16_ulp(exact))
    assert np.mean(got == exact) >= 0.999


@pytest.mark.parametrize("T", [8192, 16384, 32768])
def test_ffn_io_router_tiles(orc, T):
    """RMSNorm folded into the router at its larger tile shapes (64x64,
    64x128 and 128x128 blocks of tokens x experts at E = 128, where gamma
    multiplies the A fragments of every k step a wave reads): the logits
    within the bound of test_ffn_io, the routing of the GPU's logits
    bit-exact with the oracle's, and y on 96 sampled tokens."""
    lay = synth.make_custom(T=T, H=256, I=128, E=128, k=8, G=64, seed=T + 7, router="weight")
    g = torch.Generator().manual_seed(T + 8)
    gamma = (torch.rand(lay.H, generator=g) * 1.5 + 0.25).to(torch.bfloat16)
    y, info = api.ffn_forward(on_dev(lay), info=True, norm_weight=gamma.to(DEV), norm_eps=1e-5)
    torch.cuda.synchronize()
    xn = orc.rmsnorm(lay.x, gamma, 1e-5)
    l_used = cpu(info["logits"]).astype(np.float32)
    l_ref = orc.router_logits(xn, lay.router_weight)
    wr = np.abs(lay.router_weight.float().numpy().astype(np.float64))
    xv = (xn.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bound = router_error_bound(torch.from_numpy(xv).to(torch.bfloat16), lay.router_weight) + \
        1.5 * (_bf16_ulp(xn) @ wr.T) + 4 * f32_ulp(np.abs(xv) @ wr.T)
    err = np.abs(l_used.astype(np.float64) - l_ref)
    say(f"  T={T}: logits max err {err.max():.3e}, min slack {(bound - err).min():.3e}")
    assert np.all(err <= bound)
    rid, rw = orc.route(l_used, lay.k)
    assert np.array_equal(cpu(info["topk_ids"]), rid)
    assert_weights_close(cpu(info["topk_weights"]), rw)
    tokens = np.sort(np.random.default_rng(T).choice(T, 96, replace=False)).astype(np.int32)
    y_ref = orc.ffn(xn, rid, rw, lay.gate, lay.up, lay.down, lay.G, tokens=tokens)
    assert_fp_close(cpu(y)[tokens], y_ref, f"T={T} y (96 sampled rows)")


# ---------------------------------------------------- decode attention --
# fp32 arithmetic over at most 131072 positions (products of bf16 values are
# exact in fp32; the sums and the rescaling by exp2 differences carry about
# 1e-6 relative error each; the probabilities enter the value sums as a bf16
# pair hi + lo, within 2^-16 of the fp32 value): relative L2 <= 1e-4, max
# abs <= 1e-3 * rms.
ATTN_REL_L2, ATTN_MAX_ABS = 1e-4, 1e-3


def _attn_check(got, ref, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = got - ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    mx = float(np.abs(err).max()) if err.size else 0.0
    say(f"  {what}: relL2 {rel:.3e} maxabs {mx:.3e} (rms {rms:.3e})")
    assert rel <= ATTN_REL_L2 and mx <= ATTN_MAX_ABS * rms + 1e-30, what


@pytest.mark.parametrize("Hq,Hkv", [(32, 4), (4, 4), (8, 4), (16, 4)])
def test_decode_attention(orc, Hq, Hkv):
    """Ragged lengths (empty, one position, partial blocks, a block's last
    position, several ranges of a workgroup), scattered blocks, every
    grouped-query factor; element by element against the oracle."""
    case = synth.make_attention([150, 0, 1, 64, 4097, 200, 63], Hq=Hq, Hkv=Hkv, D=128, block=64,
                                seed=97 + Hq)
    out = api.decode_attention(case.to(DEV))
    torch.cuda.synchronize()
    ref = orc.decode_attention(case.q, case.kcache, case.vcache, case.table, case.lens)
    got = cpu(out)
    assert np.all(got[1] == 0)
    _attn_check(got, ref, f"attention Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("block", [8, 24])
def test_decode_attention_block_sizes(orc, block):
    """Blocks shorter than a step of 32 positions and of a length that is no
    power of two: runs of 8 positions found through the table."""
    case = synth.make_attention([150, 1, 300, 63, 1000], Hq=32, Hkv=4, D=128, block=block, seed=71 + block)
    out = api.decode_attention(case.to(DEV))
    torch.cuda.synchronize()
    ref = orc.decode_attention(case.q, case.kcache, case.vcache, case.table, case.lens)
    _attn_check(cpu(out), ref, f"attention block={block}")


def test_decode_attention_skipped_blocks(orc):
    """Table entries outside [0, num_blocks) are skipped: a sequence whose
    second and fourth blocks are -1 and num_blocks gives the attention over
    its first and third blocks alone (the oracle on those 128 positions)."""
    import dataclasses
    full = synth.make_attention([256], Hq=32, Hkv=4, D=128, block=64, seed=57)
    NB = full.kcache.shape[0]
    bad = full.table.clone()
    bad[0, 1], bad[0, 3] = -1, NB
    case = dataclasses.replace(full, table=bad)
    out = api.decode_attention(case.to(DEV))
    torch.cuda.synchronize()
    kept = dataclasses.replace(full, table=full.table[:, [0, 2]].contiguous(),
                               lens=torch.tensor([128], dtype=torch.int32))
    ref = orc.decode_attention(kept.q, kept.kcache, kept.vcache, kept.table, kept.lens)
    _attn_check(cpu(out), ref, "attention with skipped blocks")


def test_decode_attention_max_len_clamp(orc):
    """A sequence length above max_len is taken as max_len: with lengths
    (300, 90) and max_len 200 the first sequence is attended over its first
    200 positions only (the oracle on lengths (200, 90)), the second in
    full."""
    import dataclasses
    case = synth.make_attention([300, 90], Hq=8, Hkv=4, D=128, block=16, seed=58)
    out = api.decode_attention(case.to(DEV), max_len=200)
    torch.cuda.synchronize()
    clamped = dataclasses.replace(case, lens=torch.tensor([200, 90], dtype=torch.int32))
    ref = orc.decode_attention(clamped.q, clamped.kcache, clamped.vcache, clamped.table, clamped.lens)
    _attn_check(cpu(out), ref, "attention with a length above max_len")


def test_decode_attention_graph_replay():
    """Both launches captured in a HIP graph (no allocation, no memset)
    replay to the eager result, bit for bit, with other attention work on the
    same workspace between replays."""
    a = synth.make_attention([3000, 17, 900], seed=58).to(DEV)
    b = synth.make_attention([700, 5000, 1], seed=59).to(DEV)
    B, Hq, D = a.q.shape
    Hkv = a.kcache.shape[1]
    ws = torch.empty(int(api._L().moe_decode_attention_workspace_bytes(B, Hq, Hkv, 5000)),
                     dtype=torch.uint8, device=DEV)
    eager = api.decode_attention(a, workspace=ws, max_len=3000).clone()
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.decode_attention(a, out=out, workspace=ws, max_len=3000)
    for r in range(4):
        out.fill_(float("nan"))
        api.decode_attention(b, workspace=ws, max_len=5000)  # rewrites the shared workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"


@pytest.mark.parametrize("name", ["attn_decode_32k", "attn_decode_128k", "attn_decode_b8_32k"])
def test_decode_attention_workloads(orc, name):
    """The benchmark workloads at full size, every output against the
    oracle, and the output identical on a second call (fixed merge order)."""
    case = synth.make_attention_workload(name)
    d = case.to(DEV)
    out = api.decode_attention(d)
    out2 = api.decode_attention(d)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    ref = orc.decode_attention(case.q, case.kcache, case.vcache, case.table, case.lens)
    _attn_check(cpu(out), ref, name)


@pytest.mark.parametrize("case", ["prefill_t512", "ragged", "imbalanced_t8192"])
def test_ffn_host_blockmap_identical(case):
    """The host-round-trip ablation runs the same kernels on a block map the
    host builds: routing structures and output bit-identical to the
    single-submission layer."""
    if case == "ragged":
        lay = synth.make_custom(T=333, H=512, I=256, E=16, k=2, G=64, seed=61)
    else:
        lay = synth.make_layer(case)
    lay = api.pack_layer(on_dev(lay))
    y1, i1 = api.ffn_forward(lay, info=True)
    y1 = y1.clone()
    ref = {k: cpu(i1[k]).copy() for k in ("counts", "offsets", "sorted_pairs", "pair_slot", "num_blocks")}
    nb = int(ref["num_blocks"][0])
    ref["blocks"] = cpu(i1["blocks"])[:nb].copy()
    host = torch.empty(api.host_blockmap_ints(lay), dtype=torch.int32, pin_memory=True)
    y2, i2 = api.ffn_forward(lay, info=True, host_blockmap=host)
    torch.cuda.synchronize()
    for k in ("counts", "offsets", "sorted_pairs", "pair_slot", "num_blocks"):
        assert np.array_equal(cpu(i2[k]), ref[k]), k
    assert np.array_equal(cpu(i2["blocks"])[:nb], ref["blocks"])
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("case", ["prefill_t512", "ragged_g32", "imbalanced_t8192", "ragged_zeropoint"])
def test_ffn_unfused_identical(case):
    """The unfused ablation multiplies the same fp16 weights (expanded to
    HBM first, in the expert's exact or general form) in the same order:
    output bit-identical to the fused layer."""
    if case == "ragged_g32":
        lay = synth.make_custom(T=333, H=512, I=256, E=16, k=2, G=32, seed=62)
    elif case == "ragged_zeropoint":
        lay = synth.make_custom(T=333, H=512, I=256, E=16, k=2, G=64, seed=63, bias="zeropoint")
    else:
        lay = synth.make_layer(case)
    lay = api.pack_layer(on_dev(lay))
    y1 = api.ffn_forward(lay).clone()
    ex = torch.empty(api.unfused_bytes(lay), dtype=torch.uint8, device=DEV)
    y2 = api.ffn_forward(lay, expanded=ex)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_ffn_t0():
    lay = synth.make_custom(T=0, H=256, I=128, E=8, k=2, G=32, seed=34)
    y = api.ffn_forward(on_dev(lay))
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


def test_ffn_deterministic():
    """Two runs give identical routing structures and a bit-identical output
    (the combine adds each token's k rows in a fixed order)."""
    lay = on_dev(synth.make_custom(T=700, H=512, I=256, E=32, k=4, G=64, seed=35))
    a, ia = api.ffn_forward(lay, info=True)
    a = a.clone()
    ia = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in ia.items()}
    b, ib = api.ffn_forward(lay, info=True)
    torch.cuda.synchronize()
    for key in ("topk_ids", "counts", "offsets", "sorted_pairs", "pair_slot", "num_blocks"):
        assert torch.equal(ia[key], ib[key]), key
    nb = int(ia["num_blocks"][0])
    assert torch.equal(ia["blocks"][:nb], ib["blocks"][:nb])
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["decode_t1", "prefill_t512"])
def test_graph_replay_matches_eager(name):
    """The layer captured in a HIP graph (one stream, no host round trip, no
    allocation, no memset) replays to the eager result, bit for bit, on
    every replay, with other work on the same buffers between replays."""
    lay = api.pack_layer(on_dev(synth.make_layer(name)))
    other = api.pack_layer(on_dev(synth.make_custom(T=lay.T, H=lay.H, I=lay.I, E=lay.E, k=lay.k,
                                                    G=lay.G, seed=36)))
    ws = torch.empty(max(api.ffn_workspace_bytes(lay), api.ffn_workspace_bytes(other)),
                     dtype=torch.uint8, device=DEV)
    y_eager = api.ffn_forward(lay, workspace=ws).clone()
    y = torch.empty_like(y_eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.ffn_forward(lay, y=y, workspace=ws)
    for r in range(4):
        y.fill_(float("nan"))
        api.ffn_forward(other, workspace=ws)  # rewrites the shared workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r}"
