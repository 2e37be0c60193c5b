"""ctypes view of libmoe_w4.so (declarations mirror include/moe_w4.h).

The library is loaded after ``import torch`` so that it binds to the HIP
runtime torch already loaded (both carry the SONAME libamdhip64.so.7) and can
run on torch's streams.  There is no fallback: a missing library raises.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (load torch's HIP runtime first)

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_w4.so")

c_i32, c_i64, c_sz, c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

MOE_GEMM_GATE_UP_SWIGLU = 0
MOE_GEMM_DOWN = 1

# Exported symbols, in header order.
SYMBOLS = (
    "moe_status_string", "moe_last_error", "moe_version",
    "moe_w4_packed_words_bytes", "moe_w4_packed_sb_bytes", "moe_w4_pack",
    "moe_route", "moe_max_blocks", "moe_build_blocks_workspace_bytes", "moe_build_blocks",
    "moe_w4_grouped_gemm_workspace_bytes", "moe_w4_h_exp_bytes", "moe_w4_grouped_gemm",
    "moe_ffn_block_m", "moe_ffn_workspace_bytes", "moe_ffn_forward", "moe_ffn_forward_timed",
    "moe_ffn_host_blockmap_ints", "moe_ffn_forward_host_blockmap",
    "moe_ffn_unfused_bytes", "moe_ffn_forward_unfused",
    "moe_rmsnorm", "moe_ffn_io_workspace_bytes", "moe_ffn_forward_io",
    "moe_decode_attention_workspace_bytes", "moe_decode_attention",
    "moe_ffn_single_sync_ints", "moe_ffn_forward_single",
    "moe_ffn_noalloc_max_bytes", "moe_ffn_forward_noalloc",
)

# Stage boundaries of moe_ffn_forward_timed (enum moe_stage).
STAGES = ("route", "build_blocks", "gate_up", "down", "combine")
MOE_NUM_STAGES = len(STAGES)


class Dims(ctypes.Structure):
    _fields_ = [("T", c_i32), ("H", c_i32), ("I", c_i32), ("E", c_i32), ("top_k", c_i32),
                ("group_size", c_i32)]


class Bank(ctypes.Structure):
    """Row-major W4 bank (moe_w4_bank)."""
    _fields_ = [("qweight", c_p), ("scales", c_p), ("biases", c_p)]


class Packed(ctypes.Structure):
    """Packed W4 bank (moe_w4_packed)."""
    _fields_ = [("words", c_p), ("sb", c_p)]


class Layer(ctypes.Structure):
    _fields_ = [("dims", Dims), ("router_weight", c_p), ("gate", Packed), ("up", Packed),
                ("down", Packed)]


class FfnIO(ctypes.Structure):
    """The steps around the layer (moe_ffn_io)."""
    _fields_ = [("norm_weight", c_p), ("norm_eps", ctypes.c_float), ("residual", c_p), ("out", c_p)]


class GemmArgs(ctypes.Structure):
    _fields_ = [("mode", c_i32), ("T", c_i32), ("top_k", c_i32), ("E", c_i32), ("N", c_i32),
                ("K", c_i32), ("group_size", c_i32), ("block_m", c_i32), ("a", c_p),
                ("bank0", Packed), ("bank1", Packed), ("sorted_pairs", c_p), ("topk_weights", c_p),
                ("blocks", c_p), ("num_blocks", c_p), ("out", c_p), ("workspace", c_p),
                ("workspace_bytes", c_sz), ("h_exp", c_p), ("h_exp_bytes", c_sz)]


class RouteInfo(ctypes.Structure):
    _fields_ = [("block_m", c_i32), ("path", c_i32), ("logits", c_p), ("topk_ids", c_p),
                ("topk_weights", c_p), ("counts", c_p), ("offsets", c_p), ("sorted_pairs", c_p),
                ("pair_slot", c_p), ("blocks", c_p), ("num_blocks", c_p), ("h", c_p),
                ("y_sorted", c_p), ("y_sorted_bytes", c_i32), ("h_exp", c_p), ("y_sorted_exp", c_p)]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


_lib = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m quantized_moe_top_amd.build`")
    L = ctypes.CDLL(path)
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_version.restype = ctypes.c_char_p
    L.moe_w4_packed_words_bytes.restype = c_sz
    L.moe_w4_packed_words_bytes.argtypes = [c_i32, c_i32, c_i32]
    L.moe_w4_packed_sb_bytes.restype = c_sz
    L.moe_w4_packed_sb_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32]
    L.moe_w4_pack.argtypes = [ctypes.POINTER(Bank), c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p]
    L.moe_route.argtypes = [c_p, c_p, c_p, c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p]
    L.moe_max_blocks.restype = c_i64
    L.moe_max_blocks.argtypes = [c_i32, c_i32, c_i32, c_i32]
    L.moe_build_blocks_workspace_bytes.restype = c_sz
    L.moe_build_blocks_workspace_bytes.argtypes = [c_i32, c_i32, c_i32]
    L.moe_build_blocks.argtypes = [c_p, c_i32, c_i32, c_i32, c_i32] + [c_p] * 7 + [c_sz, c_p]
    L.moe_w4_grouped_gemm_workspace_bytes.restype = c_sz
    L.moe_w4_grouped_gemm_workspace_bytes.argtypes = [ctypes.POINTER(GemmArgs)]
    L.moe_w4_grouped_gemm.argtypes = [ctypes.POINTER(GemmArgs), c_p]
    L.moe_w4_h_exp_bytes.restype = c_sz
    L.moe_w4_h_exp_bytes.argtypes = [c_i32] * 5
    L.moe_ffn_block_m.restype = c_i32
    L.moe_ffn_block_m.argtypes = [ctypes.POINTER(Dims)]
    L.moe_ffn_workspace_bytes.restype = c_sz
    L.moe_ffn_workspace_bytes.argtypes = [ctypes.POINTER(Dims), c_i32]
    L.moe_ffn_forward.argtypes = [ctypes.POINTER(Layer), c_p, c_p, c_p, ctypes.POINTER(RouteInfo),
                                  c_p, c_sz, c_p]
    L.moe_ffn_forward_timed.argtypes = [ctypes.POINTER(Layer), c_p, c_p, c_p,
                                        ctypes.POINTER(RouteInfo), c_p, c_sz, c_p, c_p]
    L.moe_ffn_host_blockmap_ints.restype = c_sz
    L.moe_ffn_host_blockmap_ints.argtypes = [ctypes.POINTER(Dims)]
    L.moe_ffn_forward_host_blockmap.argtypes = [ctypes.POINTER(Layer), c_p, c_p, c_p,
                                                ctypes.POINTER(RouteInfo), c_p, c_sz, c_p, c_sz,
                                                c_p]
    L.moe_ffn_unfused_bytes.restype = c_sz
    L.moe_ffn_unfused_bytes.argtypes = [ctypes.POINTER(Dims)]
    L.moe_ffn_forward_unfused.argtypes = [ctypes.POINTER(Layer), c_p, c_p, c_p,
                                          ctypes.POINTER(RouteInfo), c_p, c_sz, c_p, c_sz, c_p]
    L.moe_rmsnorm.argtypes = [c_p, c_p, ctypes.c_float, c_i32, c_i32, c_p, c_p]
    L.moe_ffn_io_workspace_bytes.restype = c_sz
    L.moe_ffn_io_workspace_bytes.argtypes = [ctypes.POINTER(Dims), c_i32]
    L.moe_ffn_forward_io.argtypes = [ctypes.POINTER(Layer), c_p, c_p, c_p, ctypes.POINTER(FfnIO),
                                     ctypes.POINTER(RouteInfo), c_p, c_sz, c_p]
    L.moe_decode_attention_workspace_bytes.restype = c_sz
    L.moe_decode_attention_workspace_bytes.argtypes = [c_i32] * 4
    L.moe_decode_attention.argtypes = [c_p] * 5 + [c_i32] * 8 + [c_p, c_p, c_sz, c_p]
    L.moe_ffn_single_sync_ints.restype = c_sz
    L.moe_ffn_single_sync_ints.argtypes = []
    L.moe_ffn_forward_single.argtypes = [ctypes.POINTER(Layer), c_p, c_p, c_p, ctypes.POINTER(RouteInfo),
                                         c_p, c_sz, c_p, c_p]
    L.moe_ffn_noalloc_max_bytes.restype = c_sz
    L.moe_ffn_noalloc_max_bytes.argtypes = []
    L.moe_ffn_forward_noalloc.argtypes = [ctypes.POINTER(Layer), c_p, c_p, c_p, ctypes.POINTER(RouteInfo),
                                          c_p]
    for name in ("moe_w4_pack", "moe_route", "moe_build_blocks", "moe_w4_grouped_gemm",
                 "moe_ffn_forward", "moe_ffn_forward_timed", "moe_ffn_forward_host_blockmap",
                 "moe_ffn_forward_unfused", "moe_rmsnorm", "moe_ffn_forward_io",
                 "moe_decode_attention", "moe_ffn_forward_single", "moe_ffn_forward_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int, where: str) -> None:
    if status != 0:
        L = load()
        detail = L.moe_last_error().decode() or L.moe_status_string(status).decode()
        raise MoEError(status, where, detail)
