"""CPU oracle for the W4 MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library path never calls it.

This module is marshalling only: it compiles ``moe_oracle.c`` with gcc
(``-O2 -fopenmp``) into ``libmoe_oracle.so`` beside it and exposes its C
functions through ctypes, taking and returning NumPy arrays (torch CPU
tensors are accepted as inputs).  All arithmetic is in ``moe_oracle.c``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "moe_oracle.c")
LIBRARY = os.path.join(_HERE, "libmoe_oracle.so")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def compile_oracle(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc; returns the library path."""
    tmp = output + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra",
           "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, output)
    return output


def _np(a, dtype) -> np.ndarray:
    """Host contiguous array of `dtype` (bf16 torch tensors become uint16 bits)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16)
            a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(a)
    if a.dtype != dtype:
        if a.dtype.itemsize == np.dtype(dtype).itemsize and a.dtype.kind in "iu" and np.dtype(dtype).kind in "iu":
            a = a.view(dtype)
        else:
            a = a.astype(dtype)
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_p)


class Oracle:
    """ctypes view of one build of ``moe_oracle.c``."""

    def __init__(self, path: Optional[str] = None):
        if path is None:
            path = LIBRARY
            if (not os.path.exists(path)) or os.path.getmtime(path) < os.path.getmtime(SOURCE):
                compile_oracle()
        self.path = path
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_router_logits.argtypes = [_p, _p, _i64, _i64, _i64, _p]
        L.oracle_route.argtypes = [_p, _i64, _i64, _i64, _p, _p]
        L.oracle_build_blocks.argtypes = [_p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p]
        L.oracle_dequant.argtypes = [_p, _p, _p, _i64, _i64]
        L.oracle_dequant.restype = ctypes.c_float
        L.oracle_expert_hidden.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64] + [_p] * 6 + [_p]
        L.oracle_expert_down.argtypes = [_p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _p]
        L.oracle_ffn.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64] + [_p] * 9 + [_p]
        L.oracle_rmsnorm.argtypes = [_p, _p, ctypes.c_double, _i64, _i64, _p]
        L.oracle_residual_out.argtypes = [_p, _p, _i64, _p]
        L.oracle_decode_attention.argtypes = [_p, _p, _p, _p, _p] + [_i64] * 6 + [_p]

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    # -- router ---------------------------------------------------------
    def router_logits(self, x, wr) -> np.ndarray:
        x = _np(x, np.uint16)
        wr = _np(wr, np.uint16)
        T, H = x.shape
        E = wr.shape[0]
        assert wr.shape == (E, H)
        out = np.empty((T, E), np.float32)
        self.lib.oracle_router_logits(_ptr(x), _ptr(wr), T, H, E, _ptr(out))
        return out

    def route(self, logits, k: int):
        l = _np(logits, np.float32)
        T, E = l.shape
        if not 1 <= k <= E:
            raise ValueError("need 1 <= k <= E")
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float32)
        self.lib.oracle_route(_ptr(l), T, E, k, _ptr(ids), _ptr(w))
        return ids, w

    # -- histogram / scan / scatter / block map --------------------------
    def build_blocks(self, ids, E: int, block_m: int) -> dict:
        ids = _np(ids, np.int32)
        T, k = ids.shape
        P = T * k
        counts = np.empty(E, np.int32)
        offsets = np.empty(E + 1, np.int32)
        sorted_pairs = np.empty(P, np.int32)
        pair_slot = np.empty(P, np.int32)
        max_blocks = P // block_m + min(E, P) if P else 0
        blocks = np.zeros((max(max_blocks, 1), 3), np.int32)
        nb = np.zeros(1, np.int32)
        self.lib.oracle_build_blocks(_ptr(ids), T, k, E, block_m, _ptr(counts), _ptr(offsets),
                                     _ptr(sorted_pairs), _ptr(pair_slot), _ptr(blocks), _ptr(nb))
        n = int(nb[0])
        return dict(counts=counts, offsets=offsets, sorted_pairs=sorted_pairs,
                    pair_slot=pair_slot, blocks=blocks[:n].copy(), num_blocks=n)

    # -- weights and expert FFN -----------------------------------------
    @staticmethod
    def _bank(bank):
        return (_np(bank.qweight, np.uint32), _np(bank.scales, np.uint16), _np(bank.biases, np.uint16))

    def dequant_row(self, bank, e: int, n: int, G: int) -> np.ndarray:
        q, s, b = self._bank(bank)
        K = q.shape[2] * 8
        qrow, srow, brow = (np.ascontiguousarray(a[e, n]) for a in (q, s, b))
        return np.array([self.lib.oracle_dequant(_ptr(qrow), _ptr(srow), _ptr(brow), kk, G)
                         for kk in range(K)], np.float32)

    def expert_hidden(self, x, tokens, experts, gate, up, G: int) -> np.ndarray:
        x = _np(x, np.uint16)
        tokens = _np(tokens, np.int32).ravel()
        experts = _np(experts, np.int32).ravel()
        H = x.shape[1]
        gq, gs, gb = self._bank(gate)
        uq, us, ub = self._bank(up)
        I = gq.shape[1]
        out = np.empty((tokens.size, I), np.float64)
        self.lib.oracle_expert_hidden(_ptr(x), _ptr(tokens), _ptr(experts), tokens.size, H, I, G,
                                      _ptr(gq), _ptr(gs), _ptr(gb), _ptr(uq), _ptr(us), _ptr(ub),
                                      _ptr(out))
        return out

    def expert_down(self, h, experts, down, G: int) -> np.ndarray:
        h = _np(h, np.float64)
        experts = _np(experts, np.int32).ravel()
        dq, ds, db = self._bank(down)
        H = dq.shape[1]
        I = h.shape[1]
        out = np.empty((experts.size, H), np.float64)
        self.lib.oracle_expert_down(_ptr(h), _ptr(experts), experts.size, H, I, G,
                                    _ptr(dq), _ptr(ds), _ptr(db), _ptr(out))
        return out

    def ffn(self, x, ids, weights, gate, up, down, G: int, tokens=None) -> np.ndarray:
        """Layer output rows for `tokens` (default: all), fp32 [len(tokens), H]."""
        x = _np(x, np.uint16)
        ids = _np(ids, np.int32)
        w = _np(weights, np.float32)
        T, H = x.shape
        k = ids.shape[1]
        if tokens is None:
            tokens = np.arange(T, dtype=np.int32)
        tokens = _np(tokens, np.int32).ravel()
        gq, gs, gb = self._bank(gate)
        uq, us, ub = self._bank(up)
        dq, ds, db = self._bank(down)
        I = gq.shape[1]
        y = np.empty((tokens.size, H), np.float32)
        self.lib.oracle_ffn(_ptr(x), _ptr(ids), _ptr(w), _ptr(tokens), tokens.size, H, I, k, G,
                            _ptr(gq), _ptr(gs), _ptr(gb), _ptr(uq), _ptr(us), _ptr(ub),
                            _ptr(dq), _ptr(ds), _ptr(db), _ptr(y))
        return y

    # -- either side of the layer ------------------------------------------
    def rmsnorm(self, x, gamma, eps: float) -> np.ndarray:
        """bf16 bits [T, H] of the RMSNorm of x (bf16 [T, H]) with gain gamma (bf16 [H])."""
        x = _np(x, np.uint16)
        g = _np(gamma, np.uint16).ravel()
        T, H = x.shape
        assert g.size == H
        out = np.empty((T, H), np.uint16)
        self.lib.oracle_rmsnorm(_ptr(x), _ptr(g), float(eps), T, H, _ptr(out))
        return out

    def residual_out(self, residual, y) -> np.ndarray:
        """bf16 bits of residual (bf16) + y (fp32), same shape."""
        r = _np(residual, np.uint16)
        yy = _np(y, np.float32)
        assert r.shape == yy.shape
        out = np.empty(r.shape, np.uint16)
        self.lib.oracle_residual_out(_ptr(r), _ptr(yy), r.size, _ptr(out))
        return out

    # -- decode attention (second workload) ------------------------------
    def decode_attention(self, q, kcache, vcache, table, lens) -> np.ndarray:
        """fp32 [B, Hq, D]: q bf16 [B, Hq, D]; keys bf16 [NB, Hkv, BLK, D];
        values bf16 [NB, Hkv, D, BLK]; table int32 [B, MB]; lens int32 [B]."""
        q = _np(q, np.uint16)
        kc = _np(kcache, np.uint16)
        vc = _np(vcache, np.uint16)
        tb = _np(table, np.int32)
        ln = _np(lens, np.int32).ravel()
        B, Hq, D = q.shape
        NB, Hkv, BLK, D2 = kc.shape
        assert D2 == D and vc.shape == (NB, Hkv, D, BLK) and tb.shape[0] == B and ln.size == B and Hq % Hkv == 0
        assert np.all(ln <= tb.shape[1] * BLK) and np.all((tb >= 0) & (tb < NB))
        out = np.empty((B, Hq, D), np.float32)
        self.lib.oracle_decode_attention(_ptr(q), _ptr(kc), _ptr(vc), _ptr(tb), _ptr(ln), B, Hq, Hkv, D,
                                         BLK, tb.shape[1], _ptr(out))
        return out

    def layer(self, layer, block_m: int, tokens=None) -> dict:
        """Every step of the layer on a ``synth.MoELayer``: logits (from the
        router weight when the layer has one), routing, block map, output."""
        logits = (self.router_logits(layer.x, layer.router_weight)
                  if layer.router_weight is not None else _np(layer.logits, np.float32))
        ids, w = self.route(logits, layer.k)
        bb = self.build_blocks(ids, layer.E, block_m)
        y = self.ffn(layer.x, ids, w, layer.gate, layer.up, layer.down, layer.G, tokens)
        return dict(logits=logits, ids=ids, weights=w, y=y, **bb)


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
