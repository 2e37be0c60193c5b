"""The C ABI on the host, no GPU needed: the library loads, exports every
function include/moe_w4.h declares, and rejects bad arguments with the
documented status before anything is enqueued (no compute call is made:
every call below either fails validation or has T = 0)."""
import ctypes
import os
import re

import pytest

from quantized_moe_top_amd import _lib
from quantized_moe_top_amd._lib import Bank, Dims, GemmArgs, Layer, Packed, RouteInfo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, -1, -2, -3, -4, -5
A = 0x10000  # a 16-byte aligned stand-in address; validation never dereferences it


@pytest.fixture(scope="module")
def L():
    return _lib.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.SYMBOLS) == names


def test_status_strings(L):
    for s in (OK, NULL, SHAPE, UNSUP, ALIGN, WS, -6):
        assert L.moe_status_string(s)
    assert b"gfx950" in L.moe_version()


def test_max_blocks_and_workspace_queries(L):
    assert L.moe_max_blocks(512, 8, 128, 64) == 4096 // 64 + 128
    assert L.moe_max_blocks(1, 8, 128, 8) == 1 + 8
    assert L.moe_max_blocks(0, 8, 128, 8) == 0
    assert L.moe_build_blocks_workspace_bytes(8192, 8, 128) >= 64 * 128 * 4
    d = Dims(512, 2048, 512, 128, 8, 64)
    assert L.moe_ffn_block_m(ctypes.byref(d)) == 64
    d.T = 8
    assert L.moe_ffn_block_m(ctypes.byref(d)) == 8
    d.T = 32768
    assert L.moe_ffn_block_m(ctypes.byref(d)) == 128
    d.T = 16
    d.H, d.I, d.E, d.top_k, d.group_size = 256, 128, 8, 2, 32
    assert L.moe_ffn_block_m(ctypes.byref(d)) == 32
    # at least x staged in fp16 and h [P, I] in fp16
    assert L.moe_ffn_workspace_bytes(ctypes.byref(d), 0) >= 16 * 256 * 2 + 16 * 2 * 128 * 2
    d.H = 100
    assert L.moe_ffn_workspace_bytes(ctypes.byref(d), 0) == 0


def route(L, x=0, wr=0, logits=A, T=4, H=256, E=8, k=2, ids=A, w=A):
    return L.moe_route(x, wr, logits, T, H, E, k, ids, w, None)


def test_route_validation(L):
    assert route(L, E=0) == SHAPE
    assert route(L, T=-1) == SHAPE
    assert route(L, k=0) == SHAPE
    assert route(L, E=300) == UNSUP
    assert route(L, k=9) == UNSUP
    assert route(L, E=64, k=17) == UNSUP
    assert route(L, logits=0) == NULL
    assert route(L, ids=0) == NULL
    assert route(L, wr=A) == NULL                 # router weight without x
    assert route(L, wr=A, x=A + 4) == ALIGN
    assert route(L, wr=A, x=A, H=100) == UNSUP
    assert route(L, T=0) == OK                    # nothing enqueued
    assert L.moe_last_error() == b""
    route(L, E=0)
    assert b"E >= 1" in L.moe_last_error()


def test_build_blocks_validation(L):
    def bb(ids=A, T=4, k=2, E=8, bm=32, ws=A, wsb=1 << 20):
        return L.moe_build_blocks(ids, T, k, E, bm, A, A, A, A, A, A, ws, wsb, None)
    assert bb(bm=0) == SHAPE
    assert bb(ids=0) == NULL
    assert bb(wsb=0) == WS
    assert bb(ws=0) == NULL
    assert bb(k=9) == UNSUP
    assert bb(T=0) == OK


def gemm_args(**kw):
    bank = Packed(A, A)
    a = GemmArgs(mode=0, T=64, top_k=2, E=8, N=128, K=256, group_size=32, block_m=32, a=A,
                 bank0=bank, bank1=bank, sorted_pairs=A, topk_weights=A, blocks=A, num_blocks=A,
                 out=A, workspace=A, workspace_bytes=1 << 30, h_exp=A, h_exp_bytes=1 << 30)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_gemm_validation(L):
    g = lambda **kw: L.moe_w4_grouped_gemm(ctypes.byref(gemm_args(**kw)), None)
    assert g(mode=2) == SHAPE
    assert g(group_size=48) == UNSUP
    assert g(K=96, group_size=32) == UNSUP          # K % 64
    assert g(N=96) == UNSUP                         # gate/up N % 128
    assert g(mode=1, N=128) == UNSUP                # down N % 256
    assert g(block_m=16) == UNSUP                   # MFMA path tiles
    assert g(block_m=0) == SHAPE
    assert g(a=0) == NULL
    assert g(mode=1, N=256, topk_weights=0) == NULL
    assert g(bank1=Packed(0, A)) == NULL
    assert g(bank0=Packed(A + 8, A)) == ALIGN
    assert g(out=A + 2) == ALIGN
    assert g(workspace_bytes=10) == WS
    assert g(h_exp=0) == NULL
    assert g(h_exp=A + 4) == ALIGN
    assert g(h_exp_bytes=10) == WS
    assert g(mode=1, N=256, h_exp_bytes=10) == WS
    assert g(T=0) == OK
    # h's exponents: P * I / 16 bytes padded to 16, then one int32 flag per tile
    assert L.moe_w4_h_exp_bytes(64, 2, 8, 128, 32) == 1024 + 4 * (128 // 32 + 8)
    assert L.moe_w4_h_exp_bytes(3, 2, 8, 128, 8) == 48 + 4 * (6 // 8 + 6)
    assert L.moe_w4_h_exp_bytes(0, 2, 8, 128, 32) == 0
    assert L.moe_w4_grouped_gemm_workspace_bytes(ctypes.byref(gemm_args())) >= 64 * 256 * 2
    assert L.moe_w4_grouped_gemm_workspace_bytes(ctypes.byref(gemm_args(mode=1))) == 0


def test_ffn_validation(L):
    bank = Packed(A, A)

    def ffn(T=16, H=256, I=128, E=8, k=2, G=32, wr=0, logits=A, x=A, y=A, ws=A, wsb=1 << 30, gate=bank):
        lay = Layer(Dims(T, H, I, E, k, G), wr, gate, bank, bank)
        return L.moe_ffn_forward(ctypes.byref(lay), x, logits, y, None, ws, wsb, None)
    assert ffn(H=200) == UNSUP
    assert ffn(I=96) == UNSUP
    assert ffn(G=16) == UNSUP
    assert ffn(wr=A) == SHAPE                       # both router weight and logits
    assert ffn(logits=0) == SHAPE                   # neither
    assert ffn(x=0) == NULL
    assert ffn(y=A + 4) == ALIGN
    assert ffn(gate=Packed(A, 0)) == NULL
    assert ffn(ws=A + 16) == ALIGN
    assert ffn(wsb=100) == WS
    info = RouteInfo()
    lay = Layer(Dims(0, 256, 128, 8, 2, 32), 0, bank, bank, bank)
    assert L.moe_ffn_forward(ctypes.byref(lay), A, A, A, ctypes.byref(info), A, 1 << 20, None) == OK
    assert info.block_m == 8 and info.path == 1


def test_ffn_timed_validation(L):
    bank = Packed(A, A)
    lay = Layer(Dims(16, 256, 128, 8, 2, 32), 0, bank, bank, bank)
    # no event array: rejected before anything is enqueued
    assert L.moe_ffn_forward_timed(ctypes.byref(lay), A, A, A, None, A, 1 << 30, None, None) == NULL
    # argument errors are reported exactly as by moe_ffn_forward
    evs = (ctypes.c_void_p * (_lib.MOE_NUM_STAGES + 1))()
    lay.dims.H = 200
    assert L.moe_ffn_forward_timed(ctypes.byref(lay), A, A, A, None, A, 1 << 30, evs, None) == UNSUP


def test_pack_queries_and_validation(L):
    assert L.moe_w4_packed_words_bytes(128, 512, 2048) == 128 * 512 * 2048 // 2
    # the words, then the tail: 2^-c and the dequantisation form per expert, padded to 16 bytes
    assert L.moe_w4_packed_sb_bytes(128, 512, 2048, 64) == 128 * 512 * 32 * 4 + 128 * 8
    assert L.moe_w4_packed_sb_bytes(3, 128, 256, 32) == 3 * 128 * 8 * 4 + 32
    assert L.moe_w4_packed_words_bytes(8, 100, 256) == 0          # N % 128
    assert L.moe_w4_packed_words_bytes(8, 96, 256) == 0
    assert L.moe_w4_packed_sb_bytes(8, 128, 192, 64) == 0         # K % 128
    assert L.moe_w4_packed_sb_bytes(8, 128, 256, 48) == 0         # G
    src = Bank(A, A, A)
    pk = lambda **kw: L.moe_w4_pack(ctypes.byref(kw.pop("src", src)), kw.get("E", 8), kw.get("N", 128),
                                    kw.get("K", 256), kw.get("G", 32), kw.get("w", A), kw.get("sb", A), None)
    assert pk(w=0) == NULL
    assert pk(src=Bank(A, 0, A)) == NULL
    assert pk(N=100) == UNSUP
    assert pk(N=96) == UNSUP
    assert pk(K=192) == UNSUP
    assert pk(G=16) == UNSUP
    assert pk(E=0) == SHAPE
    assert pk(w=A + 4) == ALIGN


def test_rmsnorm_and_io_validation(L):
    norm = lambda x=A, g=A, T=4, H=256, out=A: L.moe_rmsnorm(x, g, 1e-6, T, H, out, None)
    assert norm(H=0) == SHAPE
    assert norm(T=-1) == SHAPE
    assert norm(H=100) == UNSUP                    # H % 8
    assert norm(g=0) == NULL
    assert norm(out=A + 2) == ALIGN
    assert norm(T=0) == OK                         # nothing enqueued
    bank = Packed(A, A)
    lay = Layer(Dims(16, 256, 128, 8, 2, 32), 0, bank, bank, bank)
    d = Dims(16, 256, 128, 8, 2, 32)
    extra = L.moe_ffn_io_workspace_bytes(ctypes.byref(d), 0) - L.moe_ffn_workspace_bytes(ctypes.byref(d), 0)
    assert extra >= 16 * 256 * 2                   # the normalised activations

    def io_call(io, wsb=1 << 30):
        return L.moe_ffn_forward_io(ctypes.byref(lay), A, A, A, ctypes.byref(io), None, A, wsb, None)
    assert io_call(_lib.FfnIO(0, 1e-6, 0, A)) == NULL        # out without residual
    assert io_call(_lib.FfnIO(A + 2, 1e-6, 0, 0)) == ALIGN   # norm weight misaligned
    assert io_call(_lib.FfnIO(0, 1e-6, A, A + 4)) == ALIGN   # out misaligned
    need_plain = L.moe_ffn_workspace_bytes(ctypes.byref(d), 0)
    assert io_call(_lib.FfnIO(A, 1e-6, 0, 0), wsb=need_plain) == WS  # no room for the normalised x
    lay.dims.H = 200
    assert io_call(_lib.FfnIO(0, 1e-6, 0, 0)) == UNSUP       # same checks as moe_ffn_forward


def test_decode_attention_validation(L):
    def att(B=2, Hq=32, Hkv=4, D=128, blk=64, mb=4, nb=8, ml=256, ws=A, wsb=1 << 30, q=A):
        return L.moe_decode_attention(q, A, A, A, A, B, Hq, Hkv, D, blk, mb, nb, ml, A, ws, wsb, None)
    assert att(D=64) == UNSUP
    assert att(Hq=12, Hkv=4) == UNSUP               # group of 3
    assert att(Hq=30, Hkv=4) == UNSUP               # not a multiple
    assert att(Hq=64, Hkv=4) == UNSUP               # group of 16
    assert att(blk=0) == SHAPE
    assert att(blk=12) == UNSUP                     # value runs of 8 positions
    assert att(nb=0) == SHAPE
    assert att(q=0) == NULL
    assert att(q=A + 2) == ALIGN
    assert att(wsb=8) == WS
    assert att(B=0) == OK                           # nothing enqueued
    assert L.moe_decode_attention_workspace_bytes(1, 32, 4, 32768) >= 32 * 130 * 4


def test_noalloc_validation(L):
    """The fixed scratch area's size, and refusals before any device work:
    no layer, a layer whose workspace exceeds the area, T = 0."""
    assert L.moe_ffn_noalloc_max_bytes() == 40 << 20
    assert L.moe_ffn_forward_noalloc(None, A, A, A, None, None) == NULL
    bank = Packed(A, A)
    big = Layer(Dims(4096, 2048, 512, 16, 8, 64), 0, bank, bank, bank)
    assert L.moe_ffn_forward_noalloc(ctypes.byref(big), A, A, A, None, None) == UNSUP
    empty = Layer(Dims(0, 2048, 512, 16, 8, 64), 0, bank, bank, bank)
    assert L.moe_ffn_forward_noalloc(ctypes.byref(empty), 0, 0, 0, None, None) == OK
