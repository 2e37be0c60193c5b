"""torch-tensor wrappers over the C entry points of libmoe_w4.so.

Argument marshalling only: tensors are checked for device, dtype and
contiguity, outputs and workspaces are allocated with torch, and the call is
enqueued on torch's current stream.  Every step of the layer runs in the HIP
kernels of the library.
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import (MOE_GEMM_DOWN, MOE_GEMM_GATE_UP_SWIGLU, Bank, Dims, GemmArgs, Layer, Packed,
                   RouteInfo)

__all__ = ["pack_bank", "pack_layer", "PackedBank", "PackedLayer",
           "route", "build_blocks", "w4_grouped_gemm", "ffn_forward", "ffn_workspace_bytes",
           "single_sync", "single_sync_ints",
           "ffn_block_m", "max_blocks", "stage_events", "h_exp_bytes", "MOE_GEMM_GATE_UP_SWIGLU",
           "MOE_GEMM_DOWN"]


def _L():
    return _lib.load()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _bank(b, name: str) -> Bank:
    return Bank(_dev(b.qweight, f"{name}.qweight", torch.int32),
                _dev(b.scales, f"{name}.scales", torch.bfloat16),
                _dev(b.biases, f"{name}.biases", torch.bfloat16))


@dataclasses.dataclass
class PackedBank:
    """A W4 bank in the kernels' tile-major layout (moe_w4_pack)."""
    words: torch.Tensor  # int32 [E * N * K / 8]
    sb: torch.Tensor     # int32 [E * N * K / G]
    E: int
    N: int
    K: int
    G: int

    def struct(self) -> Packed:
        return Packed(_dev(self.words, "words", torch.int32), _dev(self.sb, "sb", torch.int32))


def pack_bank(bank, G: int) -> PackedBank:
    """Packs a row-major device bank (``synth.W4Bank``) with moe_w4_pack."""
    E, N, K8 = bank.qweight.shape
    K = K8 * 8
    nw = int(_L().moe_w4_packed_words_bytes(E, N, K))
    ns = int(_L().moe_w4_packed_sb_bytes(E, N, K, G))
    if nw == 0 or ns == 0:
        raise ValueError(f"unsupported bank shape for packing: E={E} N={N} K={K} G={G}")
    dev = bank.qweight.device
    words = torch.empty(nw // 4, dtype=torch.int32, device=dev)
    sb = torch.empty(ns // 4, dtype=torch.int32, device=dev)
    src = _bank(bank, "bank")
    _lib.check(_L().moe_w4_pack(ctypes.byref(src), E, N, K, G, words.data_ptr(), sb.data_ptr(),
                                _stream()), "moe_w4_pack")
    return PackedBank(words, sb, E, N, K, G)


@dataclasses.dataclass
class PackedLayer:
    """A device ``synth.MoELayer`` whose banks are packed for the kernels."""
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    G: int
    x: torch.Tensor
    logits: Optional[torch.Tensor]
    router_weight: Optional[torch.Tensor]
    gate: PackedBank
    up: PackedBank
    down: PackedBank


def pack_layer(layer) -> PackedLayer:
    """Packs the three banks of a device ``synth.MoELayer``."""
    return PackedLayer(layer.name, layer.T, layer.H, layer.I, layer.E, layer.k, layer.G, layer.x,
                       layer.logits, layer.router_weight, pack_bank(layer.gate, layer.G),
                       pack_bank(layer.up, layer.G), pack_bank(layer.down, layer.G))


def _packed(bank, G: int) -> PackedBank:
    return bank if isinstance(bank, PackedBank) else pack_bank(bank, G)


def max_blocks(T: int, top_k: int, E: int, block_m: int) -> int:
    return int(_L().moe_max_blocks(T, top_k, E, block_m))


def route(top_k: int, logits: Optional[torch.Tensor] = None, x: Optional[torch.Tensor] = None,
          router_weight: Optional[torch.Tensor] = None):
    """S0 (when ``router_weight`` is given) and S1.  Returns
    ``(topk_ids int32 [T, k], topk_weights fp32 [T, k], logits fp32 [T, E])``."""
    if router_weight is not None:
        T, H = x.shape
        E = router_weight.shape[0]
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    else:
        T, E = logits.shape
        H = 0
    dev = logits.device
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    st = _L().moe_route(_dev(x, "x", torch.bfloat16), _dev(router_weight, "router_weight", torch.bfloat16),
                        _dev(logits, "logits", torch.float32), T, H, E, top_k,
                        ids.data_ptr(), w.data_ptr(), _stream())
    _lib.check(st, "moe_route")
    return ids, w, logits


def build_blocks(topk_ids: torch.Tensor, E: int, block_m: int) -> dict:
    """S2-S5.  Returns counts, offsets, sorted_pairs, pair_slot, blocks
    ``[max_blocks, 3]`` (rows past num_blocks unspecified) and num_blocks
    (a 1-element device tensor)."""
    T, k = topk_ids.shape
    P = T * k
    dev = topk_ids.device
    mb = max(1, max_blocks(T, k, E, block_m))
    out = dict(
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        sorted_pairs=torch.empty(P, dtype=torch.int32, device=dev),
        pair_slot=torch.empty(P, dtype=torch.int32, device=dev),
        blocks=torch.empty((mb, 3), dtype=torch.int32, device=dev),
        num_blocks=torch.zeros(1, dtype=torch.int32, device=dev),
    )
    wsb = int(_L().moe_build_blocks_workspace_bytes(T, k, E))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = _L().moe_build_blocks(_dev(topk_ids, "topk_ids", torch.int32), T, k, E, block_m,
                               out["counts"].data_ptr(), out["offsets"].data_ptr(),
                               out["sorted_pairs"].data_ptr(), out["pair_slot"].data_ptr(),
                               out["blocks"].data_ptr(), out["num_blocks"].data_ptr(),
                               ws.data_ptr(), wsb, _stream())
    _lib.check(st, "moe_build_blocks")
    return out


def h_exp_bytes(T: int, top_k: int, E: int, I: int, block_m: int) -> int:
    return int(_L().moe_w4_h_exp_bytes(T, top_k, E, I, block_m))


def w4_grouped_gemm(mode: int, a: torch.Tensor, bank0, bank1, sorted_pairs: torch.Tensor,
                    blocks: torch.Tensor, num_blocks: torch.Tensor, *, T: int, top_k: int, E: int,
                    group_size: int, block_m: int, topk_weights: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, h_exp: Optional[torch.Tensor] = None):
    """S6 (mode MOE_GEMM_GATE_UP_SWIGLU: a = x bf16 [T, H]; returns
    ``(h16, h_exp)``: h16 fp16 [P, I] in operand order and h_exp, a uint8
    device tensor of ``h_exp_bytes`` holding the int8 exponents [P, I / 16]
    and the per-tile flags, h = h16 * 2^exp) or S7 (MOE_GEMM_DOWN: a = h16,
    with ``h_exp`` from the S6 call; returns y_sorted fp32 [P, H]).  Slots
    outside every tile are left as they were in ``out``."""
    gate_up = mode == MOE_GEMM_GATE_UP_SWIGLU
    bank0 = _packed(bank0, group_size)
    bank1 = _packed(bank1, group_size) if bank1 is not None else None
    N, K = bank0.N, bank0.K
    P = T * top_k
    hb = h_exp_bytes(T, top_k, E, N if gate_up else K, block_m)
    if h_exp is None:
        if not gate_up:
            raise ValueError("the down mode needs h_exp from the gate/up call")
        h_exp = torch.empty(max(hb, 16), dtype=torch.uint8, device=a.device)
    if out is None:
        out = torch.empty((P, N), dtype=torch.float16 if gate_up else torch.float32, device=a.device)
    args = GemmArgs(mode=mode, T=T, top_k=top_k, E=E, N=N, K=K, group_size=group_size,
                    block_m=block_m,
                    a=_dev(a, "a", torch.bfloat16 if gate_up else torch.float16),
                    bank0=bank0.struct(),
                    bank1=bank1.struct() if bank1 is not None else Packed(0, 0),
                    sorted_pairs=_dev(sorted_pairs, "sorted_pairs", torch.int32),
                    topk_weights=_dev(topk_weights, "topk_weights", torch.float32),
                    blocks=_dev(blocks, "blocks", torch.int32),
                    num_blocks=_dev(num_blocks, "num_blocks", torch.int32),
                    out=_dev(out, "out", torch.float16 if gate_up else torch.float32))
    wsb = int(_L().moe_w4_grouped_gemm_workspace_bytes(ctypes.byref(args)))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=a.device)
    args.workspace = ws.data_ptr()
    args.workspace_bytes = wsb
    args.h_exp = _dev(h_exp, "h_exp", torch.uint8)
    args.h_exp_bytes = h_exp.numel()
    _lib.check(_L().moe_w4_grouped_gemm(ctypes.byref(args), _stream()), "moe_w4_grouped_gemm")
    return (out, h_exp) if gate_up else out


def _dims(layer, T: int) -> Dims:
    return Dims(T, layer.H, layer.I, layer.E, layer.k, layer.G)


def ffn_block_m(layer, T: Optional[int] = None) -> int:
    d = _dims(layer, layer.T if T is None else T)
    return int(_L().moe_ffn_block_m(ctypes.byref(d)))


def ffn_workspace_bytes(layer, T: Optional[int] = None) -> int:
    d = _dims(layer, layer.T if T is None else T)
    return int(_L().moe_ffn_workspace_bytes(ctypes.byref(d), int(layer.router_weight is not None)))


def make_layer_struct(layer: PackedLayer, T: int) -> Layer:
    return Layer(_dims(layer, T),
                 _dev(layer.router_weight, "router_weight", torch.bfloat16),
                 layer.gate.struct(), layer.up.struct(), layer.down.struct())


def stage_events(n: int = _lib.MOE_NUM_STAGES + 1):
    """``n`` timing events usable as ``ffn_forward(stage_events=...)``.  torch
    creates an event's handle on its first record, so each is recorded once
    here."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    return evs


def unpack_y16e(mant: torch.Tensor, exp: torch.Tensor) -> torch.Tensor:
    """fp32 values of the layer's weighted expert outputs in block floating
    point (``info["y_sorted"]`` int16 [P, H] and ``info["y_sorted_exp"]`` int8
    [P, H / 16]): value = mantissa * 2^exponent of its 16-value block."""
    e = exp.to(torch.int32).repeat_interleave(16, dim=-1)
    return torch.ldexp(mant.to(torch.float32), e)


def unfused_bytes(layer, T: Optional[int] = None) -> int:
    """Bytes of the device buffer ``ffn_forward(expanded=...)`` needs (0 when
    T <= 8)."""
    return int(_L().moe_ffn_unfused_bytes(ctypes.byref(_dims(layer, layer.T if T is None else T))))


def host_blockmap_ints(layer, T: Optional[int] = None) -> int:
    """int32 elements of the pinned host buffer ``ffn_forward(host_blockmap=...)``
    needs (0 when T <= 8: the GEMV path has no host variant)."""
    return int(_L().moe_ffn_host_blockmap_ints(ctypes.byref(_dims(layer, layer.T if T is None else T))))


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``moe_rmsnorm``: bf16 [T, H] rows of x normalised by their rms and
    scaled by gamma (bf16 [H])."""
    T, H = x.shape
    if out is None:
        out = torch.empty_like(x)
    _lib.check(_L().moe_rmsnorm(_dev(x, "x", torch.bfloat16), _dev(gamma, "gamma", torch.bfloat16),
                                float(eps), T, H, _dev(out, "out", torch.bfloat16), _stream()),
               "moe_rmsnorm")
    return out


def decode_attention(case, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     max_len: Optional[int] = None) -> torch.Tensor:
    """``moe_decode_attention`` on a device ``synth.AttnCase``: fp32 [B, Hq, D]."""
    B, Hq, D = case.q.shape
    NB, Hkv, BLK, _ = case.kcache.shape
    if tuple(case.vcache.shape) != (NB, Hkv, D, BLK):
        raise ValueError(f"vcache shape {tuple(case.vcache.shape)}, expected {(NB, Hkv, D, BLK)}")
    MB = case.table.shape[1]
    if max_len is None:
        max_len = int(case.lens.max().item()) if B else 0
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=case.q.device)
    wsb = int(_L().moe_decode_attention_workspace_bytes(B, Hq, Hkv, max_len))
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=case.q.device)
    _lib.check(_L().moe_decode_attention(
        _dev(case.q, "q", torch.bfloat16), _dev(case.kcache, "kcache", torch.bfloat16),
        _dev(case.vcache, "vcache", torch.bfloat16), _dev(case.table, "table", torch.int32),
        _dev(case.lens, "lens", torch.int32), B, Hq, Hkv, D, BLK, MB, NB, max_len,
        _dev(out, "out", torch.float32), _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream()), "moe_decode_attention")
    return out


def ffn_io_workspace_bytes(layer, T: Optional[int] = None) -> int:
    T = layer.T if T is None else T
    return int(_L().moe_ffn_io_workspace_bytes(ctypes.byref(_dims(layer, T)),
                                                int(layer.router_weight is not None)))


def ffn_forward(layer, x: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                info: bool = False, stage_events=None, host_blockmap: Optional[torch.Tensor] = None,
                expanded: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
                norm_eps: float = 1e-6, residual: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, sync: Optional[torch.Tensor] = None):
    """The whole layer (S0/S1-S8) for a ``PackedLayer`` (a device
    ``synth.MoELayer`` is packed first).  ``x`` and ``logits`` default to the
    layer's own.  Returns y
    fp32 [T, H], plus a dict of routing-structure views into the workspace
    when ``info`` is true.  ``stage_events`` (from ``stage_events()``) runs
    ``moe_ffn_forward_timed``, recording one event per stage boundary.
    ``host_blockmap`` (a pinned int32 CPU tensor of ``host_blockmap_ints``
    elements) runs the host-round-trip ablation
    ``moe_ffn_forward_host_blockmap`` instead (it synchronises the stream).
    ``expanded`` (a device uint8 tensor of ``unfused_bytes``) runs the
    unfused-dequantisation ablation ``moe_ffn_forward_unfused`` instead.
    ``norm_weight`` (bf16 [H]) and/or ``residual`` with ``out`` (bf16 [T, H])
    run ``moe_ffn_forward_io``: RMSNorm in front, out = bf16(residual + y)
    behind.  ``sync`` (``single_sync()``: device int32 counters, zero between
    calls) runs the single-launch decode layer ``moe_ffn_forward_single``."""
    if not isinstance(layer, PackedLayer):
        layer = pack_layer(layer)
    x = layer.x if x is None else x
    T, H = x.shape
    if layer.router_weight is None and logits is None:
        logits = layer.logits
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    use_io = norm_weight is not None or out is not None
    wsb = ffn_io_workspace_bytes(layer, T) if use_io else ffn_workspace_bytes(layer, T)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=x.device)
    if workspace.numel() < wsb:
        raise ValueError("workspace too small")
    lay = make_layer_struct(layer, T)
    ri = RouteInfo()
    args = (ctypes.byref(lay), _dev(x, "x", torch.bfloat16),
            _dev(logits, "logits", torch.float32) if layer.router_weight is None else 0,
            _dev(y, "y", torch.float32), ctypes.byref(ri),
            _dev(workspace, "workspace", torch.uint8), workspace.numel())
    if use_io:
        io = _lib.FfnIO(_dev(norm_weight, "norm_weight", torch.bfloat16) if norm_weight is not None else 0,
                        float(norm_eps),
                        _dev(residual, "residual", torch.bfloat16) if residual is not None else 0,
                        _dev(out, "out", torch.bfloat16) if out is not None else 0)
        _lib.check(_L().moe_ffn_forward_io(args[0], args[1], args[2], args[3], ctypes.byref(io),
                                           *args[4:], _stream()), "moe_ffn_forward_io")
    elif sync is not None:
        if sync.dtype != torch.int32 or sync.numel() < single_sync_ints():
            raise ValueError("sync must be a device int32 tensor of single_sync_ints() elements")
        _lib.check(_L().moe_ffn_forward_single(*args, _dev(sync, "sync", torch.int32), _stream()),
                   "moe_ffn_forward_single")
    elif expanded is not None:
        _lib.check(_L().moe_ffn_forward_unfused(*args, _dev(expanded, "expanded", torch.uint8),
                                                expanded.numel(), _stream()),
                   "moe_ffn_forward_unfused")
    elif host_blockmap is not None:
        if not (host_blockmap.is_pinned() and host_blockmap.dtype == torch.int32):
            raise ValueError("host_blockmap must be a pinned int32 CPU tensor")
        _lib.check(_L().moe_ffn_forward_host_blockmap(*args, host_blockmap.data_ptr(),
                                                      host_blockmap.numel(), _stream()),
                   "moe_ffn_forward_host_blockmap")
    elif stage_events is None:
        _lib.check(_L().moe_ffn_forward(*args, _stream()), "moe_ffn_forward")
    else:
        if len(stage_events) != _lib.MOE_NUM_STAGES + 1:
            raise ValueError(f"need {_lib.MOE_NUM_STAGES + 1} stage events")
        handles = (ctypes.c_void_p * len(stage_events))(*[e.cuda_event for e in stage_events])
        _lib.check(_L().moe_ffn_forward_timed(*args, handles, _stream()), "moe_ffn_forward_timed")
    if not info:
        return y
    return y, _info_views(ri, workspace, layer, T, logits)


def _info_views(ri: RouteInfo, ws: torch.Tensor, layer, T: int, logits) -> dict:
    base = ws.data_ptr()
    P = T * layer.k
    mb = max(1, max_blocks(T, layer.k, layer.E, ri.block_m))

    def view(ptr, numel, dtype, shape):
        if ptr == 0 or numel == 0:
            return torch.empty(shape, dtype=dtype, device=ws.device)
        off = ptr - base
        nbytes = numel * torch.empty((), dtype=dtype).element_size()
        return ws[off:off + nbytes].view(dtype).reshape(shape)

    out = dict(
        block_m=ri.block_m, path=ri.path,
        topk_ids=view(ri.topk_ids, P, torch.int32, (T, layer.k)),
        topk_weights=view(ri.topk_weights, P, torch.float32, (T, layer.k)),
        counts=view(ri.counts, layer.E, torch.int32, (layer.E,)),
        offsets=view(ri.offsets, layer.E + 1, torch.int32, (layer.E + 1,)),
        sorted_pairs=view(ri.sorted_pairs, P, torch.int32, (P,)),
        pair_slot=view(ri.pair_slot, P, torch.int32, (P,)),
        blocks=view(ri.blocks, mb * 3, torch.int32, (mb, 3)),
        num_blocks=view(ri.num_blocks, 1, torch.int32, (1,)),
        h=view(ri.h, P * layer.I, torch.float16, (P, layer.I)),
        # h = h * 2^h_exp per 16-column block
        h_exp=view(ri.h_exp, P * (layer.I // 16), torch.int8, (P, layer.I // 16)),
        # fp32, or int16 mantissas with y_sorted_exp (unpack_y16e gives fp32)
        y_sorted=(view(ri.y_sorted, P * layer.H, torch.float32, (P, layer.H))
                  if ri.y_sorted_bytes == 4 else
                  view(ri.y_sorted, P * layer.H, torch.int16, (P, layer.H))),
        y_sorted_exp=(view(ri.y_sorted_exp, P * (layer.H // 16), torch.int8, (P, layer.H // 16))
                      if ri.y_sorted_exp else None),
    )
    out["logits"] = (view(ri.logits, T * layer.E, torch.float32, (T, layer.E))
                     if layer.router_weight is not None else logits)
    return out


def single_sync_ints() -> int:
    return int(_L().moe_ffn_single_sync_ints())


_SYNC = {}


def single_sync(device=None) -> torch.Tensor:
    """The counters of the single-launch decode layer for ``device``: one
    zeroed int32 tensor per device, kept for the process (every call leaves
    it zero again).  Calls that share it must be ordered, as on one stream."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    if dev not in _SYNC:
        _SYNC[dev] = torch.zeros(single_sync_ints(), dtype=torch.int32, device=dev)
    return _SYNC[dev]


def ffn_forward_noalloc(layer, x: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                        y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``moe_ffn_forward_noalloc``: the layer with the library's fixed
    scratch area as its workspace (no workspace argument; the layer's
    workspace must fit ``moe_ffn_noalloc_max_bytes``).  Returns y fp32
    [T, H]."""
    if not isinstance(layer, PackedLayer):
        layer = pack_layer(layer)
    x = layer.x if x is None else x
    T, H = x.shape
    if layer.router_weight is None and logits is None:
        logits = layer.logits
    if y is None:
        y = torch.empty((T, H), dtype=torch.float32, device=x.device)
    lay = make_layer_struct(layer, T)
    _lib.check(_L().moe_ffn_forward_noalloc(
        ctypes.byref(lay), _dev(x, "x", torch.bfloat16),
        _dev(logits, "logits", torch.float32) if layer.router_weight is None else 0,
        _dev(y, "y", torch.float32), None, _stream()), "moe_ffn_forward_noalloc")
    return y
