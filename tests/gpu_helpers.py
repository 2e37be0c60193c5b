"""Shared helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# The floating-point bar for the layer output (and, applied the same way, for
# the intermediate h): relative L2 error <= 5e-3 and max abs error <= 2e-2 *
# rms of the oracle's tensor.
REL_L2_MAX = 5e-3
MAX_ABS_OVER_RMS = 2e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def f32_ulp(x) -> np.ndarray:
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(np.maximum(x, np.float32(np.finfo(np.float32).tiny))).astype(np.float64)


def assert_fp_close(got, ref, what: str, rms_ref: float | None = None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    rms = rms_ref if rms_ref is not None else float(np.sqrt(np.mean(ref ** 2)))
    mx = float(np.abs(err).max()) if err.size else 0.0
    say(f"  {what}: relL2 {rel:.3e}  maxabs {mx:.3e}  (bound {MAX_ABS_OVER_RMS * rms:.3e}, rms {rms:.3e})")
    assert rel <= REL_L2_MAX, f"{what}: relative L2 {rel:.3e} > {REL_L2_MAX}"
    assert mx <= MAX_ABS_OVER_RMS * rms + 1e-30, f"{what}: max abs {mx:.3e} > {MAX_ABS_OVER_RMS} * rms {rms:.3e}"
    return rel, mx


def assert_weights_close(got, ref):
    """Combine weights of the same ids, both computed in fp32 as
    w_j = a_j / (a_0 + ... + a_{k-1}), a_j = expf(l_j - l_0), summed in rank
    order.  The two sides differ only through expf (device at most 1 ulp,
    host at most 0.5 ulp: 1.5 ulp of a_j between them) and the roundings
    that follow: a_j carries 1.5 ulp, the sum 1.5 ulp plus one rounding per
    add (k - 1), the division one rounding per side.  With ulp(x) <= 2^-23 |x|
    that bounds the difference by (3 + k) 2^-23 |w| (plus the smallest
    normal, for weights in the subnormal range)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    k = ref.shape[-1] if ref.ndim else 1
    bound = (3 + k) * 2.0 ** -23 * np.abs(ref) + float(np.finfo(np.float32).tiny)
    worst = float((np.abs(got - ref) / f32_ulp(ref)).max()) if ref.size else 0.0
    assert np.all(np.abs(got - ref) <= bound), f"max diff {np.abs(got - ref).max():.3e} ({worst:.1f} ulp)"


def cpu(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


# Within every run of 8 columns the library stores h in the order
# (0,4,1,5,2,6,3,7) ("operand order", include/moe_w4.h): column j of a run
# sits at position 2*(j % 4) + j // 4.
_H_POS = np.array([2 * (j % 4) + j // 4 for j in range(8)])


def h_natural(h_stored: np.ndarray) -> np.ndarray:
    """Columns of h in natural order, from the library's operand order."""
    n = h_stored.shape[-1]
    idx = (np.arange(n) // 8) * 8 + _H_POS[np.arange(n) % 8]
    return h_stored[..., idx]


def h_values(h16: np.ndarray, hexp: np.ndarray) -> np.ndarray:
    """h in natural column order, fp64, from the library's fp16 values
    (operand order) and their exponents per 16-column block:
    h = h16 * 2^exp (include/moe_w4.h)."""
    v = h_natural(np.asarray(h16).astype(np.float64))
    e = np.repeat(np.asarray(hexp).astype(np.int64), 16, axis=-1)
    return np.ldexp(v, e)


def router_error_bound(x: torch.Tensor, wr: torch.Tensor) -> np.ndarray:
    """Forward error bound of an fp32 sum of H exact products in any order,
    gamma_H * sum_h |x_h Wr_eh| with gamma_H = H u / (1 - H u), u = 2^-24,
    plus one ulp for the oracle's own final rounding to fp32."""
    H = x.shape[1]
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    s = (x.double().abs() @ wr.double().abs().T).numpy()
    return gamma * s
