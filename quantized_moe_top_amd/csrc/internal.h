// internal.h -- device helpers and kernel launchers shared by the .hip files
// of libmoe_w4.so.  Not part of the public ABI (include/moe_w4.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_w4.h"

namespace moe {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
// 16 bytes as a native vector (kept in registers more reliably than uint4,
// which is a struct)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;           // MI355X: 8 accelerator complex dies
constexpr int kGemvMaxTokens = 8;    // T at or below this runs the GEMV path

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Activations, and the hidden vector h, are held in "operand order": within
// every run of 8 consecutive elements the order is (0,4,1,5,2,6,3,7), the
// order in which the 4-bit unpack below yields the codes of one packed word,
// so that a fragment of 8 activations lines up with one word of codes.

// (a & mask) | magic in one VALU instruction; mask in an SGPR, magic in a
// VGPR (a VOP3 instruction may read only one scalar operand here).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
  return r;
}

// Dequantises one packed 32-bit word of eight 4-bit codes into eight fp16
// weights, in the interleaved order (q0,q4,q1,q5,q2,q6,q3,q7), for an
// "exact" expert (see the (scale, bias) words below): the result is
// q * s' + b' rounded once, s' and b' the expert's scale and bias times its
// power of two 2^c.
// The packed word is the row-major word rotated left by 5 bits, so code j
// sits at bits (4j + 5) mod 32; a right rotation by 4k brings codes k and
// k + 4 to bits 5..8 of the low and the high 16-bit half.  OR-ing them into
// the mantissa of 32.0h (whose mantissa step is 1/32) gives 32 + q exactly,
// and one fused multiply-add with the packed pair (s', b' - 32 s') gives
// (32 + q) s' + b' - 32 s' = q s' + b' with a single rounding (b' - 32 s' is
// an fp16 value exactly for such an expert; with bias = -8 scale it is
// -40 s', and every weight (q - 8) s' is exact too).  11 VALU instructions
// per word: 3 rotations, 4 v_and_or_b32, 4 v_pk_fma_f16.
__device__ __forceinline__ uint4 dequant_word(uint32_t w, half2_t s2, half2_t b2) {
  const uint32_t mask = 0x01E001E0u, k32 = 0x50005000u;  // bits 5..8 of each half; 32.0h
  const half2_t v0 = __builtin_bit_cast(half2_t, and_or(w, mask, k32));  // q0, q4
  const half2_t v1 = __builtin_bit_cast(half2_t, and_or(__builtin_amdgcn_alignbit(w, w, 4), mask, k32));
  const half2_t v2 = __builtin_bit_cast(half2_t, and_or(__builtin_amdgcn_alignbit(w, w, 8), mask, k32));
  const half2_t v3 = __builtin_bit_cast(half2_t, and_or(__builtin_amdgcn_alignbit(w, w, 12), mask, k32));
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v0, s2, b2)),
                    __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v1, s2, b2)),
                    __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v2, s2, b2)),
                    __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v3, s2, b2)));
}

// The same for a "general" expert (b' - 32 s' not an fp16 value for some
// group): t = (32 + q) s' - 32 s' = q s' with one rounding (-32 s' is exact),
// then t + b' with a second.  n2 = (-32 s', -32 s').  15 VALU instructions
// per word (4 more v_pk_add_f16).
__device__ __forceinline__ uint4 dequant_word_gen(uint32_t w, half2_t s2, half2_t n2, half2_t b2) {
  const uint32_t mask = 0x01E001E0u, k32 = 0x50005000u;
  const half2_t v0 = __builtin_bit_cast(half2_t, and_or(w, mask, k32));
  const half2_t v1 = __builtin_bit_cast(half2_t, and_or(__builtin_amdgcn_alignbit(w, w, 4), mask, k32));
  const half2_t v2 = __builtin_bit_cast(half2_t, and_or(__builtin_amdgcn_alignbit(w, w, 8), mask, k32));
  const half2_t v3 = __builtin_bit_cast(half2_t, and_or(__builtin_amdgcn_alignbit(w, w, 12), mask, k32));
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v0, s2, n2) + b2),
                    __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v1, s2, n2) + b2),
                    __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v2, s2, n2) + b2),
                    __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v3, s2, n2) + b2));
}

// A packed (scale, bias) word -- fp16 s' in the low half, fp16 b' - 32 s'
// (exact experts) or b' (general experts) in the high half -- as the two
// broadcast pairs the exact dequantisation takes.
__device__ __forceinline__ void sb_pairs(uint32_t sb, half2_t& s2, half2_t& b2) {
  const half2_t v = __builtin_bit_cast(half2_t, sb);
  s2 = half2_t{v[0], v[0]};
  b2 = half2_t{v[1], v[1]};
}

// Both forms behind one type, for the kernels that pick per expert at run
// time: gen selects the general form; c2 = (b' - 32 s') pairs (exact) or
// (-32 s') pairs (general).
struct SbPair {
  half2_t s2, c2, b2;
  bool gen;
};
__device__ __forceinline__ SbPair sb_unpack(uint32_t sb, bool gen) {
  SbPair r;
  sb_pairs(sb, r.s2, r.b2);
  r.gen = gen;
  r.c2 = gen ? r.s2 * half2_t{(half_t)-32.0f, (half_t)-32.0f} : r.b2;
  return r;
}
__device__ __forceinline__ uint4 dequant_word_any(uint32_t w, const SbPair& p) {
  return p.gen ? dequant_word_gen(w, p.s2, p.c2, p.b2) : dequant_word(w, p.s2, p.c2);
}

// The tail of a packed (scale, bias) buffer: per expert the factor 2^-c
// that undoes the expert's scaling, and whether it takes the general
// dequantisation.
struct BankTail {
  const float* unscale;
  const uint32_t* general;
};
__host__ __device__ __forceinline__ BankTail bank_tail(const moe_w4_packed& b, int E, int N, int K, int G) {
  const uint32_t* t = b.sb + (size_t)E * N * (K / G);
  return BankTail{reinterpret_cast<const float*>(t), t + E};
}

// Position of column j (0..7) of an 8-column run in the interleaved order.
__device__ __forceinline__ int interleaved_pos(int j) { return 2 * (j & 3) + (j >> 2); }

// Eight bf16 values (one 16-byte chunk) -> eight fp16 values in the
// interleaved order above.  bf16 values inside the fp16 range convert
// exactly.
__device__ __forceinline__ uint4 bf16x8_to_half_interleaved(uint4 v) {
  auto lo = [](uint32_t d) { return (half_t)__uint_as_float(d << 16); };
  auto hi = [](uint32_t d) { return (half_t)__uint_as_float(d & 0xFFFF0000u); };
  const half2_t o0 = {lo(v.x), lo(v.z)}, o1 = {hi(v.x), hi(v.z)};
  const half2_t o2 = {lo(v.y), lo(v.w)}, o3 = {hi(v.y), hi(v.w)};
  return make_uint4(__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1),
                    __builtin_bit_cast(uint32_t, o2), __builtin_bit_cast(uint32_t, o3));
}

// Makes this wave's LDS writes visible to its own later LDS reads (a wave
// barrier between two workgroup-scope fences).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP lane moves: four
// row shifts build the sums inside each 16-lane row, then two row broadcasts
// carry lane 15's total into row 1 (and lane 47's into row 3), and lane
// 31's into rows 2 and 3.  Lanes a move does not reach add 0.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// global_load_lds_dwordx4 / _dword: each lane's 16 (4) bytes at g land in
// LDS at l + 16 (4) * lane; l must be the same for the whole wave.
__device__ __forceinline__ void lds_load16(const void* g, char* l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* g, char* l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 4, 0, 0);
}

// s_waitcnt vmcnt(n) alone (expcnt and lgkmcnt not waited on).  Loads
// complete in issue order, so after it every load but the last n issued by
// this wave is done (stores only add to the count, making it conservative).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt vmcnt(n), then a workgroup barrier.  The asm is a compiler
// memory barrier, so no LDS access moves across it; no fence is used because
// a fence would also wait for the loads still in flight for later slabs.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("s_barrier" ::: "memory");
}

// s_waitcnt vmcnt(BASE + n X), then a workgroup barrier, for a runtime n in
// [0, K] (n is uniform, so the choice is a scalar branch).
template <int BASE, int X, int K>
__device__ __forceinline__ void wait_vm_barrier_n(int n) {
  if constexpr (K == 0) {
    wait_vm_barrier<BASE>();
  } else {
    if (n >= K) wait_vm_barrier<BASE + K * X>();
    else wait_vm_barrier_n<BASE, X, K - 1>(n);
  }
}

// 16-byte LDS read hidden from the compiler's memory model.  Reading a ring
// that LDS-DMA copies are still filling, the compiler cannot tell the stages
// apart and would wait for every copy in flight first; the ring's own
// count-based wait already orders the read.  The value may be used only
// after lds_wait on it.
__device__ __forceinline__ u32x4 lds_read16(const void* p) {
  u32x4 v;
  const uint32_t off = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(off));
  return v;
}
// 4-byte LDS read, hidden the same way.
__device__ __forceinline__ uint32_t lds_read4(const void* p) {
  uint32_t v;
  const uint32_t off = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(off));
  return v;
}
// Waits until at most N of this wave's LDS reads are outstanding (they
// complete in issue order); the value passed becomes usable.  lds_tie marks
// further values as usable from that point on.
template <int N>
__device__ __forceinline__ void lds_wait_n(u32x4& a) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
__device__ __forceinline__ void lds_tie(u32x4& a) { asm volatile("" : "+v"(a)); }
__device__ __forceinline__ void lds_tie(uint32_t& a) { asm volatile("" : "+v"(a)); }
// Waits for every LDS read of this wave; the values passed become usable.
__device__ __forceinline__ void lds_wait(u32x4& a) { asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a)); }
__device__ __forceinline__ void lds_wait(u32x4& a, u32x4& b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b));
}

// Block floating point for the weighted expert outputs between the down
// projection and the combine inside the layer ("y16e"): per row, each block
// of 16 consecutive values shares one exponent E (int8) and each value is an
// int16 mantissa q, value = q * 2^E.  E puts the block's largest |v| times
// (1 + 2^-15) in [2^14, 2^15) * 2^E, so that value keeps 15 bits (relative
// error at most 2^-16), no mantissa rounds beyond 32767, and every other
// value of the block has an absolute error of at most 2^(E-1); 2 + 1/16
// bytes a value.  An all-zero block has E = -128.
__device__ __forceinline__ int y16_exp(float m) {
  // selects, not branches: m (1 + 2^-15) in [2^(ex-1), 2^ex)
  const int ex = __builtin_amdgcn_frexp_expf(m * (1.0f + 0x1p-15f));
  const int e = max(-128, min(127, ex - 15));
  return m >= 0x1p127f ? 127 : m > 0.0f ? e : -128;
}
// Four values a_i * w of one block -> four int16 mantissas (8 bytes), to
// nearest: with ws = w 2^-E, one FMA a ws + 1.5 2^23 rounds the product
// once to an integer held in the low mantissa bits (|a ws| < 2^15), whose
// low 16 bits are the two's-complement mantissa; two of them are packed by
// one byte permute.  ws = 0 for an all-zero block.
__device__ __forceinline__ uint2 y16_pack4(float a, float b, float c, float d, float ws) {
  auto q = [ws](float v) { return __float_as_uint(fmaf(v, ws, 0x1.8p23f)); };
  return make_uint2(__builtin_amdgcn_perm(q(b), q(a), 0x05040100u), __builtin_amdgcn_perm(q(d), q(c), 0x05040100u));
}
// Eight int16 mantissas (16 bytes) of one block times 2^E, exact.
__device__ __forceinline__ void y16_unpack8(uint4 m, int E, float* out) {
  const float f = ldexpf(1.0f, E);
  const uint32_t w[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    out[2 * i] = (float)(int)(int16_t)(w[i] & 0xFFFFu) * f;
    out[2 * i + 1] = (float)(int)(int16_t)(w[i] >> 16) * f;
  }
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Four bf16 residual values (8 bytes) plus four fp32 values, rounded to bf16.
__device__ __forceinline__ uint2 residual_add_bf16x4(uint2 r, float4 y) {
  const float r0 = __uint_as_float(r.x << 16), r1 = __uint_as_float(r.x & 0xFFFF0000u);
  const float r2 = __uint_as_float(r.y << 16), r3 = __uint_as_float(r.y & 0xFFFF0000u);
  return make_uint2(f32_to_bf16_rne(r0 + y.x) | (f32_to_bf16_rne(r1 + y.y) << 16),
                    f32_to_bf16_rne(r2 + y.z) | (f32_to_bf16_rne(r3 + y.w) << 16));
}

// The hidden vector h leaves the gate/up kernels as fp16 values with a
// power-of-two exponent per row and 16-column block: h = h16 * 2^e.  e is 0
// unless the block's largest |h| (m) is at least 2^15 or below 2^-10 (and
// not 0); then m * 2^-e lies in [2^14, 2^15), so no block overflows fp16 or
// sinks into its subnormals, whatever the magnitudes of x and the weights.
// Rows with a nonzero exponent mark their tile of the block map, so the
// down kernels can keep the plain path for every other tile.
__device__ __forceinline__ int h_block_exp(float m) {
  if (m < 32768.0f && (m >= 0x1p-10f || m == 0.0f)) return 0;
  if (m != m) return 0;          // NaN propagates unscaled
  if (m > 3.0e38f) return 127;   // inf stays inf
  int ex;
  frexpf(m, &ex);                // m in [2^(ex-1), 2^ex)
  return max(-128, min(127, ex - 15));
}
// The largest v over each 16-lane DPP row (four row rotations; every lane
// of the row gets it, so all 16 lanes must be active).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true)));
  return v;
}
// The largest of the four signed bytes of w.
__device__ __forceinline__ int max_i8x4(uint32_t w) {
  return max(max((int)(int8_t)(w & 0xFF), (int)(int8_t)((w >> 8) & 0xFF)),
             max((int)(int8_t)((w >> 16) & 0xFF), (int)(int8_t)(w >> 24)));
}
// Eight fp16 values (16 bytes) times 2^d, d <= 0 (d below -24 gives 0).
__device__ __forceinline__ uint4 scale_half8(uint4 v, int d) {
  const half_t f = (half_t)ldexpf(1.0f, max(d, -25));
  const half2_t f2 = {f, f};
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v.x) * f2),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v.y) * f2),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v.z) * f2),
                    __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v.w) * f2));
}

// silu(g) * u = g / (1 + e^-g) * u, with the hardware exponential and
// reciprocal (about 1 ulp each; the result is then rounded to fp16).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------- launchers --
// Each returns hipSuccess or the launch error.  Arguments are validated by
// the callers in api.hip.
// Routing chunks: consecutive tokens handled by one routing workgroup and
// histogrammed together (at most 256 chunks).
int route_chunk_tokens(int64_t T);
int route_chunks(int64_t T);

// Ranges of H the router GEMM splits into when given room for partial sums
// (part: router_ksplit * T * E floats; 1 = no split, part unused).
int router_ksplit(int64_t T, int64_t H, int64_t E);
// S0 (when wr) + S1 over all T tokens; with xh and chunk_hist (both or
// neither) also the per-chunk expert histogram and the fp16 staging of x.
// part (or nullptr): scratch for the router's partial sums.
// gamma (bf16 [H], with xh): RMSNorm in front, folded in: the router sums
// bf16(x * gamma) * wr and the routing kernel scales each row's logits by
// its 1 / sqrt(mean x^2 + eps) (written back to logits), and xh holds the
// normalised rows bf16(x * r * gamma); needs route_norm_fits.
bool route_norm_fits(int64_t T, int64_t H, int64_t E, bool has_router, bool split);
hipError_t launch_route(const uint16_t* x, const uint16_t* wr, float* logits, int T, int H, int E,
                        int k, int32_t* ids, float* w, half_t* xh, int32_t* chunk_hist,
                        float* part, hipStream_t s, const uint16_t* gamma = nullptr, float eps = 0.0f);
// S0 alone: the router logits (ksplit == 1) or ksplit partial sums over
// ranges of H (ksplit == router_ksplit(T, H, E)) into out, [ksplit][T][E].
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, float* out, int T, int H,
                                int E, int ksplit, hipStream_t s);
// Per-chunk expert histogram of caller-given ids [T][k].
hipError_t launch_chunk_hist(const int32_t* ids, int T, int k, int E, int32_t* chunk_hist,
                             hipStream_t s);
// S2 (totals) - S5 from the per-chunk histograms; with chunk_start
// ([chunks][E] first slots, computed by the caller) only the S4 scatter.
// With tflags, also clears the gate/up kernel's per-tile flags [nflags].
hipError_t launch_scan_scatter(const int32_t* ids, int T, int k, int E, const int32_t* chunk_hist,
                               int block_m, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_pairs, int32_t* pair_slot, int32_t* blocks,
                               int32_t* num_blocks, hipStream_t s,
                               const int32_t* chunk_start = nullptr, int32_t* tflags = nullptr,
                               int64_t nflags = 0);

// x bf16 [T][H] -> fp16 [T][H] with every 8-chunk interleaved (see above).
// Also clears tflags [nflags] (the per-tile flags the gate/up kernel sets).
hipError_t launch_stage_x(const uint16_t* x, half_t* xh, int64_t n_elems, int32_t* tflags,
                          int64_t nflags, hipStream_t s);

// One-time repack of a row-major bank into the tile-major layout the GEMM
// and GEMV kernels read (include/moe_w4.h, moe_w4_pack).
hipError_t launch_pack(const moe_w4_bank& src, int E, int N, int K, int G, uint32_t* words,
                       uint32_t* sb, hipStream_t s);

// The unfused ablation: expands a packed bank (moe_w4_pack layout) to fp16
// weights in the GEMM's operand order, 4 KiB per 32-column block and slab
// (N * K * 2 bytes per expert): piece i of a block holds the dequantised word
// i of each (column, reduction half), 16 bytes each.
hipError_t launch_expand(const moe_w4_packed& bank, int E, int N, int K, int G, uint32_t* out,
                         hipStream_t s);

struct GemmArgs {
  int mode;  // MOE_GEMM_*
  int T, top_k, E, N, K, G, block_m;
  const half_t* a;  // gate/up: staged x (fp16, interleaved) [T][K]; down: h fp16 [P][K]
  moe_w4_packed b0, b1;
  const int32_t* sorted_pairs;
  const float* topk_weights;
  const int32_t* blocks;
  const int32_t* num_blocks;
  void* out;
  bool y16e = false;       // down: out is y16e mantissas [P][N] (exponents at yexp) instead of fp32
  int64_t grid_tiles = -1;   // >= 0: exact tile count known on the host (grid sized to it)
  bool dense = false;        // banks hold expanded fp16 weights (moe_w4_expand layout), words only
  BankTail t0{}, t1{};       // the tails of the packed (scale, bias) buffers of b0 and b1
  // h's exponents int8 [P][I / 16] and per-tile flags int32 [max_blocks]
  // (nonzero: a row of the tile has a nonzero exponent): written by gate/up,
  // read by down
  int8_t* hexp = nullptr;
  int32_t* tflags = nullptr;
  int8_t* yexp = nullptr;    // down with y16e: the exponents [P][N / 16]
};
hipError_t launch_w4_mfma(const GemmArgs& a, hipStream_t s);
hipError_t launch_w4_gemv(const GemmArgs& a, hipStream_t s);

// Decode sizes (T <= kGemvMaxTokens): S1-S5 and S6 in one launch.  Every
// workgroup routes all T tokens from the logits (ksplit partial sums
// [ksplit][T][E] added in range order) into LDS and builds the block map
// there (block_m = kGemvMaxTokens); workgroup 0 also writes the routing
// outputs (and, when ksplit > 1, the summed logits to logits_out); each
// workgroup then runs its (tile, 32-column block) of the gate/up GEMV on x
// (bf16, converted while staged) and writes h.
struct DecodeRouting {
  const float* logits;
  float* logits_out;
  int ksplit;
  int32_t *ids;
  float* w;
  int32_t *counts, *offsets, *sorted_pairs, *pair_slot, *blocks, *num_blocks;
};
// gamma (bf16 [K], or nullptr): RMSNorm of x in front, folded into the
// staging of the x rows; needs decode_norm_fits(a) (every row resident).
bool decode_norm_fits(const GemmArgs& a);
hipError_t launch_decode_gate_up(const DecodeRouting& r, const GemmArgs& a, hipStream_t s,
                                 const uint16_t* gamma = nullptr, float eps = 0.0f);
// Decode sizes: S7 and S8 in one launch, per token (a.a: h; a.out: y_sorted
// fp32 [T * k][N], written too; ids, pair_slot: [T * k]; y: [T][N]).  Needs
// decode_down_fused(K): a reduction of at most 16 slabs of 64.
bool decode_down_fused(int K);
hipError_t launch_decode_down(const GemmArgs& a, const int32_t* ids, const int32_t* pair_slot,
                              float* y, hipStream_t s, const uint16_t* residual = nullptr,
                              uint16_t* out = nullptr);
// Decode sizes, the whole layer in one launch (launch_decode_gate_up's and
// launch_decode_down's work, identical results): g the gate/up product, d
// the down product.  sync: device int32 [kDecodeSyncInts], zero before the
// first call and left zero by every call (launches that share it must not
// overlap); sync[257] is set if a wait gave up.  Needs
// decode_layer_supported(g, d): both halves on workgroups of one size.
constexpr int kDecodeSyncInts = 258;
bool decode_layer_supported(const GemmArgs& g, const GemmArgs& d);
hipError_t launch_decode_layer(const DecodeRouting& r, const GemmArgs& g, const GemmArgs& d, float* y,
                               int32_t* sync, hipStream_t s, const uint16_t* residual = nullptr,
                               uint16_t* out = nullptr);

// S8: y[t] = sum_j y_sorted[pair_slot[t * k + j]], j ascending; y_sorted
// fp32 (yexp == nullptr), or block floating point: int16 mantissas [P][H]
// with exponents yexp [P][H / 16] (y16e above).
// With out (bf16 [T][H]): also out = bf16(residual + y) (residual bf16 [T][H]).
hipError_t launch_combine(const void* y_sorted, const int8_t* yexp, const int32_t* pair_slot, float* y,
                          int T, int H, int k, hipStream_t s, const uint16_t* residual = nullptr,
                          uint16_t* out = nullptr);

// Decode attention (a second workload): ranges of positions per workgroup.
struct AttnPlan {
  int nsplit, chunk;
};
AttnPlan attn_plan(int B, int Hkv, int max_len);
// q bf16 [B][Hq][128]; kc bf16 [num_blocks][Hkv][block][128]; vc bf16
// [num_blocks][Hkv][128][block]; block a multiple of 8; table int32
// [B][max_blocks]; lens int32 [B] (<= max_len); out fp32 [B][Hq][128]; ws:
// B * Hq * nsplit * 130 floats.  Hq / Hkv in {1, 2, 4, 8}.
hipError_t launch_decode_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                                   const int32_t* table, const int32_t* lens, int B, int Hq,
                                   int Hkv, int block, int max_blocks, int num_blocks,
                                   int max_len, float* out, float* ws, hipStream_t s);

// RMSNorm in front of the layer: out[t][h] = bf16(x[t][h] * gamma[h] /
// sqrt(mean_h x[t][h]^2 + eps)) (bf16 in and out, fp32 arithmetic, H % 8 == 0).
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int T, int H,
                          uint16_t* out, hipStream_t s);


}  // namespace moe
