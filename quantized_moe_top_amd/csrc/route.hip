// route.hip -- S0 router linear layer and S1 top-k routing with combine
// weights.  Page "Perplexity's Lily engine beats MLX by 35% on M5 Max",
// architecture paragraph: expert routing runs on the GPU in the same
// submission as the rest of the layer.
#include "internal.h"

namespace moe {
namespace {

// logits[t][e] = sum_h x[t][h] * wr[e][h]; bf16 x bf16 products are exact in
// fp32 and accumulate in fp32 inside the MFMA in a fixed order, so the result
// is deterministic.  One wave computes a 32-token x 32-expert tile over the
// whole H with v_mfma_f32_32x32x16_bf16, reading both operands straight from
// global memory (each row is read as 16-byte pieces; x rows are reused from
// L2 by the expert blocks of the other waves).
// grid (ceil(T/32), ceil(E/128)), block 256: wave w -> experts
// [32 * (4 * blockIdx.y + w), +32).
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          float* __restrict__ logits, int T, int H,
                                                          int E) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 32;
  const int e0 = (blockIdx.y * 4 + wave) * 32;
  if (e0 >= E) return;
  const int r = lane & 31, half = lane >> 5;
  // rows past T or E read a valid row; their results are never stored
  const int t = min(t0 + r, T - 1), e = min(e0 + r, E - 1);
  const uint4* xa = reinterpret_cast<const uint4*>(x + (size_t)t * H) + half;
  const uint4* wb = reinterpret_cast<const uint4*>(wr + (size_t)e * H) + half;
  floatx16_t acc = {};
  const int steps = H / 16;
  for (int s = 0; s < steps; s++) {
    const uint4 av = xa[2 * s];
    const uint4 bv = wb[2 * s];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                  __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
  }
  const int col = e0 + (lane & 31);
  if (col >= E) return;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int row = t0 + 8 * (i >> 2) + 4 * half + (i & 3);
    if (row < T) logits[(size_t)row * E + col] = acc[i];
  }
}

// Order-preserving map of an fp32 bit pattern onto unsigned integers
// (-inf lowest, +inf highest).  -0.0 is first folded onto +0.0: the two
// compare equal, so they must tie (and the tie goes to the lower expert).
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, off);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// One wave per token.  Lane l holds the logits of experts l, l+64, l+128,
// l+192 as 64-bit keys (ordered logit bits << 32 | (0xFFFF - e)), so the
// largest key is the largest logit and, among equal logits, the lowest
// expert.  k rounds of a wave-wide max pick the experts in order; the
// winner's key is cleared.  Combine weights: fp32 softmax over the k chosen
// logits, max-subtracted, summed in choice order.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = lane + 64 * i;
    key[i] = e < E ? (((uint64_t)ordered_bits(l[e]) << 32) | (uint32_t)(0xFFFF - e)) : 0ull;
  }
  int sel[16];
#pragma unroll
  for (int j = 0; j < 16; j++) {
    if (j < k) {
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < 4; i++) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const int e = 0xFFFF - (int)(best & 0xFFFFu);
      sel[j] = e;
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (lane + 64 * i == e) key[i] = 0ull;
    }
  }
  if (lane != 0) return;
  const float m = l[sel[0]];
  float a[16];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    if (j < k) {
      a[j] = expf(l[sel[j]] - m);
      sum += a[j];
    }
  }
#pragma unroll
  for (int j = 0; j < 16; j++) {
    if (j < k) {
      ids[(size_t)t * k + j] = sel[j];
      w[(size_t)t * k + j] = a[j] / sum;
    }
  }
}

}  // namespace

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* wr, float* logits, int T, int H,
                              int E, hipStream_t s) {
  dim3 grid((T + 31) / 32, (E + 127) / 128);
  router_gemm_kernel<<<grid, 256, 0, s>>>(x, wr, logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       hipStream_t s) {
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
