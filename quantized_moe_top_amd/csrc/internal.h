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

constexpr int kWave = 64;
constexpr int kNumXcd = 8;           // MI355X: 8 accelerator complex dies
constexpr int kGemvMaxTokens = 8;    // T at or below this runs the GEMV path
constexpr int kChunkPairs = 1024;    // pairs per histogram/scatter chunk

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Reorders the eight 16-bit values of a 16-byte chunk from (0..7) to
// (0,4,1,5,2,6,3,7): the order in which the 4-bit unpack below yields the
// codes of one packed word.  Activations are stored or staged in this order
// so that a fragment of 8 activations lines up with one word of codes.
__device__ __forceinline__ uint4 interleave_halves(uint4 d) {
  uint4 o;
  o.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);  // (v0, v4)
  o.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);  // (v1, v5)
  o.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);  // (v2, v6)
  o.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);  // (v3, v7)
  return o;
}

// Dequantises one 32-bit word of eight 4-bit codes into eight fp16 weights
// q * scale + bias, in the interleaved order (q0,q4,q1,q5,q2,q6,q3,q7).
// OR-ing a code into the mantissa of 1024.0h gives 1024 + q exactly; the
// subtraction recovers q exactly and the fused multiply-add rounds once (it
// is exact when bias = -8 * scale, because (q - 8) * scale then needs at most
// 11 significant bits).
__device__ __forceinline__ uint4 dequant_word(uint32_t w, half2_t s2, half2_t b2) {
  const uint32_t m = 0x000F000Fu, magic = 0x64006400u;
  const half2_t k1024 = {(half_t)1024.0f, (half_t)1024.0f};
  uint32_t r[4];
  r[0] = (w & m) | magic;
  r[1] = ((w >> 4) & m) | magic;
  r[2] = ((w >> 8) & m) | magic;
  r[3] = ((w >> 12) & m) | magic;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    half2_t q = __builtin_bit_cast(half2_t, r[i]) - k1024;
    half2_t v = __builtin_elementwise_fma(q, s2, b2);
    r[i] = __builtin_bit_cast(uint32_t, v);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ half2_t bf16_pair_to_half2(uint16_t s) {
  half_t h = (half_t)bf16_bits_to_float(s);
  return half2_t{h, h};
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------- launchers --
// Each returns hipSuccess or the launch error.  Arguments are validated by
// the callers in api.hip.
hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* wr, float* logits, int T, int H,
                              int E, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       hipStream_t s);
hipError_t launch_build_blocks(const int32_t* ids, int P, int E, int block_m, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_slot,
                               int32_t* blocks, int32_t* num_blocks, int32_t* scratch,
                               hipStream_t s);
int build_blocks_chunks(int64_t P);

// x bf16 [T][H] -> fp16 [T][H] with every 8-chunk interleaved (see above).
hipError_t launch_stage_x(const uint16_t* x, half_t* xh, int64_t n_elems, hipStream_t s);

struct GemmArgs {
  int mode;  // MOE_GEMM_*
  int T, top_k, E, N, K, G, block_m;
  const half_t* a;  // gate/up: staged x (fp16, interleaved) [T][K]; down: h fp16 [P][K]
  moe_w4_bank b0, b1;
  const int32_t* sorted_pairs;
  const float* topk_weights;
  const int32_t* blocks;
  const int32_t* num_blocks;
  void* out;
};
hipError_t launch_w4_mfma(const GemmArgs& a, hipStream_t s);
hipError_t launch_w4_gemv(const GemmArgs& a, hipStream_t s);

hipError_t launch_combine(const float* y_sorted, const int32_t* pair_slot, float* y, int T,
                          int H, int k, hipStream_t s);

}  // namespace moe
