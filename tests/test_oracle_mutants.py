"""Plants one plausible mistake at a time in a copy of the oracle's C source
(on the CPU only), builds it, and checks that at least one pin rejects it.
This is evidence that the pins constrain every step of the oracle, not a test
of the library."""
import os

import pytest

import oracle
from oracle_pins import PINS

# (what the mistake is, original text, mistaken text)
MUTATIONS = [
    ("top-k tie keeps the higher index",
     "if (best < 0 || l[e] > l[best]) best = e;", "if (best < 0 || l[e] >= l[best]) best = e;"),
    ("softmax exponent sign flipped",
     "a[j] = expf(l[ids[t * k + j]] - m);", "a[j] = expf(m - l[ids[t * k + j]]);"),
    ("combine weights not normalised",
     "weights[t * k + j] = a[j] / s;", "weights[t * k + j] = a[j];"),
    ("offsets not accumulated",
     "offsets[e + 1] = offsets[e] + counts[e];", "offsets[e + 1] = counts[e];"),
    ("scatter visits pairs in reverse order",
     "for (int64_t p = 0; p < P; p++) {\n    int32_t s = cursor[ids[p]]++;",
     "for (int64_t p = P - 1; p >= 0; p--) {\n    int32_t s = cursor[ids[p]]++;"),
    ("last tile of an expert not clipped",
     "int64_t rows = counts[e] - r < BM ? counts[e] - r : BM;", "int64_t rows = BM;"),
    ("nibble order reversed within a word",
     "uint32_t q = (qrow[kk / 8] >> (4 * (kk % 8))) & 15u;",
     "uint32_t q = (qrow[kk / 8] >> (4 * (7 - kk % 8))) & 15u;"),
    ("scale group index dropped",
     "bf16_bits_to_float(srow[kk / G])", "bf16_bits_to_float(srow[0])"),
    ("bias dropped from the dequantisation",
     "return fmaf((float)q, bf16_bits_to_float(srow[kk / G]), bf16_bits_to_float(brow[kk / G]));",
     "return (float)q * bf16_bits_to_float(srow[kk / G]);"),
    ("silu sign flipped",
     "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("gate and up swapped in SwiGLU",
     "hout[i] = silu(g) * u;", "hout[i] = silu(u) * g;"),
    ("routing weight dropped from the combine",
     "acc[n] += w * o[n];", "acc[n] += o[n];"),
    ("every choice uses the first expert",
     "const int64_t e = ids[t * k + j];", "const int64_t e = ids[t * k];"),
    ("router weight read transposed",
     "(double)bf16_bits_to_float(wr[e * H + h])", "(double)bf16_bits_to_float(wr[h * E + e])"),
    ("down projection reads the gate bank",
     "expert_down_row(h, e, H, I, G, dq, ds, db, o);", "expert_down_row(h, e, H, I, G, gq, gs, gb, o);"),
    ("activation row of the list position instead of the token",
     "expert_hidden_row(x + t * H, e, H, I, G, gq, gs, gb, uq, us, ub, h);",
     "expert_hidden_row(x + r * H, e, H, I, G, gq, gs, gb, uq, us, ub, h);"),
    ("down projection rows reversed",
     "const int64_t row = e * H + n;", "const int64_t row = e * H + (H - 1 - n);"),
    ("up projection reads the gate bank",
     "u += (double)oracle_dequant(uq + row * (H / 8), us + row * (H / G), ub + row * (H / G), h, G) * xv;",
     "u += (double)oracle_dequant(gq + row * (H / 8), gs + row * (H / G), gb + row * (H / G), h, G) * xv;"),
    ("softmax sums only the first selected logit",
     "s += a[j];", "s = a[0];"),
    ("RMSNorm gain dropped",
     " * r *\n                                           (double)bf16_bits_to_float(gamma[h]));",
     " * r);"),
    ("RMSNorm mean over H + 1 terms",
     "const double r = 1.0 / sqrt(ss / (double)H + eps);", "const double r = 1.0 / sqrt(ss / (double)(H + 1) + eps);"),
    ("RMSNorm epsilon outside the square root",
     "const double r = 1.0 / sqrt(ss / (double)H + eps);", "const double r = 1.0 / (sqrt(ss / (double)H) + eps);"),
    ("bf16 rounding truncates",
     "const double r = nearbyint(v / ulp) * ulp;", "const double r = trunc(v / ulp) * ulp;"),
    ("attention scale dropped",
     "sc[t] = acc / sqrt((double)D);", "sc[t] = acc;"),
    ("attention KV head chosen by query head modulo",
     "const int64_t h = j / group, L = lens[b];", "const int64_t h = j % Hkv, L = lens[b];"),
    ("attention block offset ignored",
     "const uint16_t* krow = kc + ((blk * Hkv + h) * BLK + t % BLK) * D;",
     "const uint16_t* krow = kc + ((blk * Hkv + h) * BLK) * D;"),
    ("attention softmax not normalised",
     "out[(b * Hq + j) * D + d] = L > 0 ? (float)(o / den) : 0.0f;",
     "out[(b * Hq + j) * D + d] = L > 0 ? (float)o : 0.0f;"),
    ("residual dropped",
     "out[i] = double_to_bf16_bits((double)bf16_bits_to_float(residual[i]) + (double)y[i]);",
     "out[i] = double_to_bf16_bits((double)y[i]);"),
]


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, what, old, new):
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    path = tmp_path / "moe_oracle_mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.compile_oracle(str(path), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError) as exc:  # noqa: PERF203
            failed.append(pin.__name__)
            break
    assert failed, f"no pin rejects the planted mistake: {what}"
