"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises ``AssertionError`` when
the oracle disagrees with what the definitions and the mathematics fix:
hand-derived fixtures (``tests/golden``), brute force on tiny inputs, library
special cases (stable ``numpy.argsort``), closed forms (identity-like
experts, all-zero weights), invariants (bijective scatter, tile coverage) and
an independent dense fp64 computation of the whole layer.  The same pins are
run against deliberately broken builds of the oracle in
``test_oracle_mutants.py`` to show that each plausible mistake is caught.
"""

from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from quantized_moe_top_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32_ulp(x) -> np.ndarray:
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(np.maximum(x, np.float32(np.finfo(np.float32).tiny)))


def _logits_array(rows):
    return np.array([[float(v) for v in r] for r in rows], np.float32)


def _closed_form(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"exp": math.exp}))


# ---------------------------------------------------------------- routing --
def pin_route_golden(orc):
    """Hand-derived routing cases (ties, -inf, k=1, k=E)."""
    for case in _golden("route_hand.json")["cases"]:
        l = _logits_array(case["logits"])
        ids, w = orc.route(l, case["k"])
        assert ids.tolist() == case["ids"], (case["note"], ids.tolist())
        exp_w = np.array([[_closed_form(e) for e in r] for r in case["weights_closed_form"]])
        err = np.abs(w.astype(np.float64) - exp_w)
        assert np.all(err <= 4 * _f32_ulp(exp_w)), (case["note"], w, exp_w)


def _brute_topk(l: np.ndarray, k: int):
    """Maximal exact sum over all k-subsets; ties -> lexicographically
    smallest sorted index tuple.  -inf is replaced by a value below every
    finite logit."""
    finite = l[np.isfinite(l)]
    floor = Fraction(int(math.floor(finite.min())) - 1000 if finite.size else -1000)
    vals = [Fraction(float(v)) if np.isfinite(v) else floor for v in l]
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(l)), k):
        s = sum(vals[i] for i in sub)
        if best_sum is None or s > best_sum:
            best, best_sum = sub, s
    return best


def pin_route_bruteforce(orc):
    """Top-k set equals brute-force enumeration on tiny inputs with ties and
    -inf; within the set the order is (logit desc, index asc)."""
    rng = np.random.default_rng(11)
    for trial in range(120):
        E = int(rng.integers(2, 10))
        k = int(rng.integers(1, min(E, 4) + 1))
        T = 3
        l = rng.integers(-3, 4, size=(T, E)).astype(np.float32) * np.float32(0.5)
        ninf = rng.random((T, E)) < 0.15
        l[ninf] = -np.inf
        for t in range(T):
            if np.isfinite(l[t]).sum() < k:
                l[t, :k] = 0.0
        ids, _ = orc.route(l, k)
        for t in range(T):
            assert tuple(sorted(ids[t].tolist())) == _brute_topk(l[t], k), (l[t], k, ids[t])
            seq = [(-float(l[t, e]), int(e)) for e in ids[t]]
            assert seq == sorted(seq), (l[t], ids[t])


def pin_route_argsort(orc):
    """Library special case: ids equal the first k of a stable argsort of
    -logits (equal logits keep increasing index order)."""
    rng = np.random.default_rng(12)
    for E, k in ((8, 2), (128, 8), (16, 16), (5, 1)):
        l = rng.standard_normal((64, E)).astype(np.float32)
        l[::3, : E // 2] = np.round(l[::3, : E // 2])  # plenty of exact ties
        ids, _ = orc.route(l, k)
        ref = np.argsort(-l, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)


def pin_route_weights_softmax(orc):
    """Combine weights equal the full softmax renormalised on the selected
    set (fp64 reference), sum to 1, and are exactly 1/k for equal logits and
    exactly 1 for k = 1."""
    rng = np.random.default_rng(13)
    for E, k in ((8, 2), (128, 8), (12, 12)):
        l = (2.0 * rng.standard_normal((50, E))).astype(np.float32)
        ids, w = orc.route(l, k)
        full = np.exp(l.astype(np.float64) - l.max(1, keepdims=True))
        full /= full.sum(1, keepdims=True)
        sel = np.take_along_axis(full, ids.astype(np.int64), 1)
        ref = sel / sel.sum(1, keepdims=True)
        assert np.all(np.abs(w - ref) <= 8 * _f32_ulp(ref) + 1e-30)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23)
    ids, w = orc.route(np.zeros((4, 6), np.float32), 3)
    assert np.all(w == np.float32(1.0 / 3.0))
    ids, w = orc.route(rng.standard_normal((4, 6)).astype(np.float32), 1)
    assert np.all(w == 1.0)


# ------------------------------------------- histogram / scan / scatter ---
def pin_blocks_golden(orc):
    g = _golden("blocks_hand.json")
    bb = orc.build_blocks(np.array(g["ids"], np.int32), g["E"], g["BM"])
    for key in ("counts", "offsets", "sorted_pairs", "pair_slot", "blocks"):
        assert bb[key].tolist() == g[key], (key, bb[key].tolist(), g[key])
    assert bb["num_blocks"] == len(g["blocks"])


def check_blocks_invariants(ids: np.ndarray, E: int, BM: int, bb: dict):
    """Invariants of histogram, scan, scatter and block map (also used by the
    GPU tests on the library's own outputs)."""
    flat = ids.ravel().astype(np.int64)
    P = flat.size
    counts, offsets = bb["counts"], bb["offsets"]
    sp, ps, blocks = bb["sorted_pairs"], bb["pair_slot"], bb["blocks"]
    assert counts.sum() == P
    assert np.array_equal(counts, np.bincount(flat, minlength=E)[:E])
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(sp), np.arange(P))            # a permutation
    assert np.array_equal(ps[sp], np.arange(P))                  # pair_slot is its inverse
    assert np.array_equal(sp, np.argsort(flat, kind="stable"))   # stable counting sort
    slot_expert = flat[sp]
    assert np.all(np.diff(slot_expert) >= 0)
    nb = bb["num_blocks"]
    assert nb == int(sum(-(-int(c) // BM) for c in counts))
    covered = np.zeros(P, np.int64)
    prev = (-1, -1)
    for e, start, rows in blocks[:nb]:
        assert 1 <= rows <= BM and counts[e] > 0
        assert offsets[e] <= start and start + rows <= offsets[e + 1]
        assert (e, start) > prev
        prev = (e, start)
        covered[start:start + rows] += 1
    assert np.all(covered == 1)


def pin_blocks_invariants(orc):
    rng = np.random.default_rng(14)
    for T, k, E, BM in ((16, 2, 8, 32), (300, 8, 128, 64), (257, 4, 16, 16), (1, 8, 128, 8),
                        (64, 3, 5, 1)):
        l = rng.standard_normal((T, E)).astype(np.float32)
        l[:, 3::4] = -np.inf if E > 8 else l[:, 3::4]
        ids, _ = orc.route(l, k)
        check_blocks_invariants(ids, E, BM, orc.build_blocks(ids, E, BM))


# ---------------------------------------------------------------- dequant --
def unpack_codes_bytewise(qweight: np.ndarray) -> np.ndarray:
    """4-bit codes from packed words via the little-endian byte view: byte b
    of word w holds codes 8w+2b (low nibble) and 8w+2b+1 (high nibble)."""
    by = np.ascontiguousarray(qweight).view(np.uint8)
    out = np.empty(by.shape[:-1] + (by.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = by & 15
    out[..., 1::2] = by >> 4
    return out


def dense_weights(bank, G: int) -> np.ndarray:
    """fp64 dense [E, N, K] weights of a bank, from the byte view above."""
    q = unpack_codes_bytewise(bank.qweight.numpy()).astype(np.float64)
    s = np.repeat(bank.scales.float().numpy().astype(np.float64), G, axis=-1)
    b = np.repeat(bank.biases.float().numpy().astype(np.float64), G, axis=-1)
    return q * s + b


def pin_dequant_golden(orc):
    g = _golden("dequant_hand.json")
    words = np.array(g["words"], np.uint32).reshape(1, 1, -1)
    bank = synth.W4Bank(torch.from_numpy(words.view(np.int32)),
                        torch.tensor(g["scales"]).to(torch.bfloat16).reshape(1, 1, -1),
                        torch.tensor(g["biases"]).to(torch.bfloat16).reshape(1, 1, -1))
    assert synth.pack_codes(np.array(g["codes"], np.uint8)).tolist() == g["words"]
    assert orc.dequant_row(bank, 0, 0, g["G"]).tolist() == g["weights"]


def pin_dequant_dense(orc):
    """Random codes, scales and biases: every dequantised weight equals the
    byte-view unpacking (exact: bias = -8*scale makes q*s+b = (q-8)*s), and
    codes 8 dequantise to exactly zero."""
    lay = synth.make_custom(T=1, H=64, I=32, E=3, k=1, G=16, seed=15)
    for bank, N in ((lay.gate, 32), (lay.down, 64)):
        dense = dense_weights(bank, 16)
        q = unpack_codes_bytewise(bank.qweight.numpy())
        for e in range(3):
            for n in (0, 5, N - 1):
                row = orc.dequant_row(bank, e, n, 16)
                assert np.array_equal(row.astype(np.float64), dense[e, n])
                assert np.all(row[q[e, n] == 8] == 0.0)


# -------------------------------------------------------------------- FFN --
def _silu(z):
    return z / (1.0 + np.exp(-z))


def _custom_bank(codes: np.ndarray, scale_per_expert, G: int) -> synth.W4Bank:
    E, N, K = codes.shape
    words = synth.pack_codes(codes)
    s = torch.tensor(scale_per_expert, dtype=torch.float32).to(torch.bfloat16)
    s = s.view(E, 1, 1).expand(E, N, K // G).contiguous()
    b = (-8.0 * s.float()).to(torch.bfloat16)
    return synth.W4Bank(torch.from_numpy(words.view(np.int32)), s, b)


def pin_ffn_zero(orc):
    """All codes 8 with bias -8*scale: every weight is 0, so y is exactly 0."""
    lay = synth.make_custom(T=5, H=64, I=32, E=4, k=2, G=16, seed=16)
    z = lambda E, N, K: _custom_bank(np.full((E, N, K), 8, np.uint8), [0.01, 0.02, 0.5, 3.0], 16)
    ids, w = orc.route(lay.logits, 2)
    y = orc.ffn(lay.x, ids, w, z(4, 32, 64), z(4, 32, 64), z(4, 64, 32), 16)
    assert np.all(y == 0.0)


def pin_ffn_identity_closed_form(orc):
    """Experts with one non-zero weight per row, a different scale per expert
    and per bank, have the closed form
        y[t, 2i] = sum_j w_tj c_e silu(a_e x_t[i]) b_e x_t[H-1-i],  y[t, odd] = 0
    (gate row i picks x[i], up row i picks x[H-1-i], down row 2i picks h_i)."""
    H, I, E, k, G, T = 32, 16, 4, 2, 16, 6
    a, b, c = [1.0, 0.5, 2.0, 0.25], [1.5, 0.75, 1.0, 3.0], [0.5, 1.0, 2.0, 0.125]
    gq = np.full((E, I, H), 8, np.uint8)
    uq = np.full((E, I, H), 8, np.uint8)
    dq = np.full((E, H, I), 8, np.uint8)
    for i in range(I):
        gq[:, i, i] = 9
        uq[:, i, H - 1 - i] = 9
        dq[:, 2 * i, i] = 9
    gate, up, down = _custom_bank(gq, a, G), _custom_bank(uq, b, G), _custom_bank(dq, c, G)
    lay = synth.make_custom(T=T, H=H, I=I, E=E, k=k, G=G, seed=17)
    ids, w = orc.route(lay.logits, k)
    y = orc.ffn(lay.x, ids, w, gate, up, down, G).astype(np.float64)
    x = lay.x.float().numpy().astype(np.float64)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            ref[t, 0::2] += w[t, j] * c[e] * _silu(a[e] * x[t, :I]) * b[e] * x[t, ::-1][:I]
    assert np.all(np.abs(y - ref) <= _f32_ulp(ref) + 1e-30), np.abs(y - ref).max()


def _dense_ffn(x, Wg, Wu, Wd):
    """Textbook SwiGLU FFN in fp64: Wd (silu(Wg x) * (Wu x))."""
    g = x @ Wg.T
    u = x @ Wu.T
    return (g / (1.0 + torch.exp(-g)) * u) @ Wd.T


def pin_ffn_dense_single_expert(orc):
    """E = k = 1 reduces the layer to one dense SwiGLU FFN (torch fp64)."""
    lay = synth.make_custom(T=7, H=128, I=64, E=1, k=1, G=32, seed=18)
    ids, w = orc.route(lay.logits, 1)
    assert np.all(ids == 0) and np.all(w == 1.0)
    y = orc.ffn(lay.x, ids, w, lay.gate, lay.up, lay.down, 32).astype(np.float64)
    x = lay.x.double()
    ref = _dense_ffn(x, *(torch.from_numpy(dense_weights(b, 32)[0])
                          for b in (lay.gate, lay.up, lay.down))).numpy()
    assert np.all(np.abs(y - ref) <= _f32_ulp(ref) + 1e-30), np.abs(y - ref).max()


def dense_masked_layer(lay, ids, w) -> np.ndarray:
    """Y = sum_e diag(M[:, e]) FFN_e(X), M[t, e] = w[t, j] where ids[t, j] = e,
    computed expert-major over every expert with torch fp64 batched matmuls."""
    X = lay.x.double()
    Wg, Wu, Wd = (torch.from_numpy(dense_weights(b, lay.G)) for b in (lay.gate, lay.up, lay.down))
    Xb = X.unsqueeze(0).expand(lay.E, -1, -1)
    g = torch.bmm(Xb, Wg.transpose(1, 2).contiguous())
    u = torch.bmm(Xb, Wu.transpose(1, 2).contiguous())
    out = torch.bmm(g / (1.0 + torch.exp(-g)) * u, Wd.transpose(1, 2).contiguous())  # [E, T, H]
    M = torch.zeros((lay.T, lay.E), dtype=torch.float64)
    M.scatter_(1, torch.from_numpy(ids.astype(np.int64)), torch.from_numpy(w.astype(np.float64)))
    return torch.einsum("te,eth->th", M, out).numpy()


def pin_ffn_dense_masked(orc):
    """The whole tiny workload against the expert-major dense computation."""
    lay = synth.make_layer("tiny_t16")
    ids, w = orc.route(lay.logits, lay.k)
    y = orc.ffn(lay.x, ids, w, lay.gate, lay.up, lay.down, lay.G).astype(np.float64)
    ref = dense_masked_layer(lay, ids, w)
    assert np.all(np.abs(y - ref) <= _f32_ulp(ref) + 1e-12 * np.abs(ref).max()), np.abs(y - ref).max()


def pin_ffn_token_subset(orc):
    """Rows computed for a token subset equal the same rows of the full call."""
    lay = synth.make_layer("tiny_t16")
    ids, w = orc.route(lay.logits, lay.k)
    full = orc.ffn(lay.x, ids, w, lay.gate, lay.up, lay.down, lay.G)
    sub = [13, 2, 2, 7]
    part = orc.ffn(lay.x, ids, w, lay.gate, lay.up, lay.down, lay.G, tokens=sub)
    assert np.array_equal(part, full[sub])


def pin_expert_hidden_down(orc):
    """The per-pair SwiGLU hidden vector and down projection agree with the
    dense fp64 forms, and their weighted sum over a token's pairs is its
    layer output."""
    lay = synth.make_layer("tiny_t16")
    ids, w = orc.route(lay.logits, lay.k)
    toks = np.repeat(np.arange(lay.T, dtype=np.int32), lay.k)
    h = orc.expert_hidden(lay.x, toks, ids.ravel(), lay.gate, lay.up, lay.G)
    X = lay.x.double().numpy()
    Wg, Wu, Wd = (dense_weights(b, lay.G) for b in (lay.gate, lay.up, lay.down))
    for p in (0, 5, 31):
        e = ids.ravel()[p]
        g = Wg[e] @ X[toks[p]]
        u = Wu[e] @ X[toks[p]]
        assert np.allclose(h[p], _silu(g) * u, rtol=1e-12, atol=1e-12)
    o = orc.expert_down(h, ids.ravel(), lay.down, lay.G)
    for p in (1, 6, 30):
        assert np.allclose(o[p], Wd[ids.ravel()[p]] @ h[p], rtol=1e-12, atol=1e-12)
    y = (o.reshape(lay.T, lay.k, -1) * w[:, :, None].astype(np.float64)).sum(1)
    full = orc.ffn(lay.x, ids, w, lay.gate, lay.up, lay.down, lay.G).astype(np.float64)
    assert np.all(np.abs(full - y) <= _f32_ulp(y) + 1e-12)


# ----------------------------------------------------------------- router --
def pin_router_logits(orc):
    """Router logits equal an fp64 library matmul rounded to fp32 (to within
    one fp32 ulp: both sums are exact to ~1e-13 relative before rounding)."""
    lay = synth.make_custom(T=33, H=256, I=32, E=24, k=2, G=32, seed=19, router="weight")
    l = orc.router_logits(lay.x, lay.router_weight)
    ref = (lay.x.double() @ lay.router_weight.double().T).numpy()
    assert np.all(np.abs(l.astype(np.float64) - ref) <= _f32_ulp(ref)), np.abs(l - ref).max()


# ---------------------------------------------- either side of the layer --
def _bf16_bits_rne(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits, nearest with ties to even, in one step (numpy's
    rint rounds half to even); written here independently of the oracle."""
    v = np.asarray(v, np.float64)
    out = np.zeros(v.shape, np.uint16)
    nz = v != 0
    _, e = np.frexp(v[nz])
    ulp = np.ldexp(1.0, e - 8)
    r = (np.rint(v[nz] / ulp) * ulp).astype(np.float32)
    out[nz] = (r.view(np.uint32) >> 16).astype(np.uint16)
    out[~nz] = np.where(np.signbit(v[~nz]), 0x8000, 0).astype(np.uint16)
    return out


def pin_rmsnorm_library(orc):
    """RMSNorm equals the library routine (torch rms_norm in fp64) rounded
    to bf16: bit-exact on seeded rows (both are exact to ~1e-16 before the
    one rounding), including rows of very different scale."""
    g = torch.Generator().manual_seed(71)
    x = torch.randn(40, 384, generator=g, dtype=torch.float64)
    x[::5] *= 30.0
    x[1::7] *= 1e-3
    xb = x.to(torch.bfloat16)
    gamma = (torch.rand(384, generator=g, dtype=torch.float64) * 2 - 0.5).to(torch.bfloat16)
    eps = 1e-6
    ref = torch.nn.functional.rms_norm(xb.double(), (384,), weight=gamma.double(), eps=eps).numpy()
    got = orc.rmsnorm(xb, gamma, eps)
    assert np.array_equal(got, _bf16_bits_rne(ref))


def pin_rmsnorm_closed_forms(orc):
    """Constant rows c with eps = 0 normalise to sign(c) * gamma exactly;
    scaling a row by a power of two changes nothing (eps = 0)."""
    H = 64
    x = torch.tensor([[1.5] * H, [-0.375] * H, [96.0] * H], dtype=torch.bfloat16)
    gamma = torch.tensor([2.0 ** (h % 5 - 2) for h in range(H)], dtype=torch.bfloat16)
    got = orc.rmsnorm(x, gamma, 0.0)
    ref = np.stack([gamma.float().numpy(), -gamma.float().numpy(), gamma.float().numpy()])
    assert np.array_equal(got, _bf16_bits_rne(ref))
    g = torch.Generator().manual_seed(72)
    y = torch.randn(6, H, generator=g).to(torch.bfloat16)
    assert np.array_equal(orc.rmsnorm(y, gamma, 0.0), orc.rmsnorm(y * 8, gamma, 0.0))


def pin_residual_out(orc):
    """bf16(residual + y) rounds the exact sum once, ties to even: 1 + 2^-9
    is halfway between 1 and 1 + 2^-7 and goes to 1, 1 + 3 * 2^-9 goes up;
    the rest against an independent fp64 sum and rounding, also on seeded
    values."""
    res = torch.tensor([1.0, 1.0, -2.0, 0.5, 3.0], dtype=torch.bfloat16)
    y = np.array([2.0 ** -9, 3 * 2.0 ** -9, 2.0 ** -8 - 2.0 ** -30, -0.5, 1e-3], np.float32)
    got = orc.residual_out(res, y)
    assert list(got[:2]) == [0x3F80, 0x3F81]
    assert np.array_equal(got, _bf16_bits_rne(res.double().numpy() + y.astype(np.float64)))
    g = torch.Generator().manual_seed(73)
    r = torch.randn(50, 32, generator=g).to(torch.bfloat16)
    yy = (torch.randn(50, 32, generator=g) * 3).numpy()
    assert np.array_equal(orc.residual_out(r, yy),
                          _bf16_bits_rne(r.double().numpy() + yy.astype(np.float64)))


# ------------------------------------------------------- decode attention --
def _gather_kv(case, b):
    """Logical [Hkv, L, D] keys and values of sequence b (fp64)."""
    L = int(case.lens[b])
    blk = case.table[b].long()
    pos = torch.arange(L)
    k = case.kcache.double()[blk[pos // case.block], :, pos % case.block, :]  # [L, Hkv, D]
    v = case.vcache.double()[blk[pos // case.block], :, :, pos % case.block]  # [L, Hkv, D]
    return k.permute(1, 0, 2), v.permute(1, 0, 2)


def pin_attention_library(orc):
    """Decode attention equals the library routine (torch
    scaled_dot_product_attention in fp64, the KV heads repeated for their
    query-head groups) to within fp32 rounding, through a scattered block
    table, with a sequence of length 0 giving zeros."""
    case = synth.make_attention([150, 64, 0, 1, 200], Hq=8, Hkv=2, D=32, block=16, seed=94)
    got = orc.decode_attention(case.q, case.kcache, case.vcache, case.table, case.lens)
    g = case.q.shape[1] // case.kcache.shape[1]
    for b in range(case.q.shape[0]):
        if int(case.lens[b]) == 0:
            assert np.all(got[b] == 0)
            continue
        k, v = _gather_kv(case, b)
        k, v = k.repeat_interleave(g, 0), v.repeat_interleave(g, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            case.q[b].double()[:, None, :], k, v)[:, 0, :].numpy()
        assert np.all(np.abs(got[b].astype(np.float64) - ref) <= 2 * _f32_ulp(ref) + 1e-12), b


def pin_attention_closed_forms(orc):
    """Equal keys give a uniform softmax, so every query head returns the
    mean of its KV head's values; moving physical blocks (and the table with
    them) changes nothing."""
    case = synth.make_attention([96, 40], Hq=4, Hkv=2, D=16, block=16, seed=95)
    kc = case.kcache.clone()
    kc[:] = kc[0, :, 0:1, :]  # one key row everywhere, per KV head 0's first row
    got = orc.decode_attention(case.q, kc, case.vcache, case.table, case.lens)
    for b in range(2):
        _, v = _gather_kv(case, b)
        mean = v.mean(dim=1).numpy()  # [Hkv, D]
        ref = np.repeat(mean, 2, axis=0)
        assert np.all(np.abs(got[b] - ref) <= 4 * _f32_ulp(ref) + 1e-12)
    base = orc.decode_attention(case.q, case.kcache, case.vcache, case.table, case.lens)
    NB = case.kcache.shape[0]
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(96))
    kc2, vc2 = torch.empty_like(case.kcache), torch.empty_like(case.vcache)
    kc2[perm] = case.kcache
    vc2[perm] = case.vcache
    moved = orc.decode_attention(case.q, kc2, vc2, perm[case.table.long()].to(torch.int32), case.lens)
    assert np.array_equal(base, moved)


PINS = [
    pin_route_golden, pin_route_bruteforce, pin_route_argsort, pin_route_weights_softmax,
    pin_blocks_golden, pin_blocks_invariants,
    pin_dequant_golden, pin_dequant_dense,
    pin_ffn_zero, pin_ffn_identity_closed_form, pin_ffn_dense_single_expert,
    pin_ffn_dense_masked, pin_ffn_token_subset, pin_expert_hidden_down,
    pin_router_logits,
    pin_rmsnorm_library, pin_rmsnorm_closed_forms, pin_residual_out,
    pin_attention_library, pin_attention_closed_forms,
]
