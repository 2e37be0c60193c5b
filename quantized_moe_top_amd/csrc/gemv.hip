// gemv.hip -- S9: the grouped W4 GEMM at decode sizes (T <= 8).  With at most
// 8 rows per expert the product is bound by reading the packed weights, so
// each touched expert's rows are streamed once with coalesced 16-byte loads,
// dequantised in registers (same exact fp16 dequantisation as the MFMA path)
// and dotted with the few activation rows routed to that expert using
// v_dot2_f32_f16 (fp16 products, fp32 accumulation), then reduced across
// the wave.  Experts that no token chose are never read.
#include "internal.h"

namespace moe {
namespace {

struct GemvParams {
  const half_t* a;
  moe_w4_bank b0, b1;
  const int32_t* sorted_pairs;
  const float* topk_weights;
  const int32_t* blocks;
  const int32_t* num_blocks;
  void* out;
  int N, K, G, top_k, E, P, max_blocks;
};

__device__ __forceinline__ float dot32(const uint4* w, const uint4* x, float acc) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w[i].x), __builtin_bit_cast(half2_t, x[i].x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w[i].y), __builtin_bit_cast(half2_t, x[i].y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w[i].z), __builtin_bit_cast(half2_t, x[i].z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w[i].w), __builtin_bit_cast(half2_t, x[i].w), acc, false);
  }
  return acc;
}

__device__ __forceinline__ void dequant32(const uint4 q, uint16_t s, uint16_t b, uint4* w) {
  const half2_t s2 = bf16_pair_to_half2(s), b2 = bf16_pair_to_half2(b);
  w[0] = dequant_word(q.x, s2, b2);
  w[1] = dequant_word(q.y, s2, b2);
  w[2] = dequant_word(q.z, s2, b2);
  w[3] = dequant_word(q.w, s2, b2);
}

// Reads the tile and checks it; returns false for tiles past num_blocks or
// malformed entries.
__device__ __forceinline__ bool read_tile(const GemvParams& p, int tile, int& e, int& row0,
                                          int& rows) {
  const int nblk = min(*p.num_blocks, p.max_blocks);
  if (tile >= nblk) return false;
  e = p.blocks[3 * tile];
  row0 = p.blocks[3 * tile + 1];
  rows = p.blocks[3 * tile + 2];
  return e >= 0 && e < p.E && rows > 0 && rows <= kGemvMaxTokens && row0 >= 0 &&
         row0 <= p.P - rows;
}

// S6 at decode sizes: one wave per (tile, column n) computes g_n and u_n for
// every row of the tile, lane l covering reduction indices [32l, 32l+32) of
// each 2048-wide chunk.  a = staged x (fp16, interleaved) [T][K].
__global__ __launch_bounds__(256) void gemv_gate_up_kernel(const GemvParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nq = p.N / 4;
  const int tile = blockIdx.x / nq;
  const int n = (blockIdx.x % nq) * 4 + wave;
  int e, row0, rows;
  if (!read_tile(p, tile, e, row0, rows)) return;
  const int K = p.K;
  int tok[kGemvMaxTokens];
#pragma unroll
  for (int m = 0; m < kGemvMaxTokens; m++) {
    const int pair = m < rows ? p.sorted_pairs[row0 + m] : -1;
    tok[m] = (pair >= 0 && pair < p.P) ? pair / p.top_k : -1;
  }
  float ag[kGemvMaxTokens] = {}, au[kGemvMaxTokens] = {};
  const size_t rowi = (size_t)e * p.N + n;
  for (int kb = 32 * lane; kb < K; kb += 2048) {
    const int g = kb / p.G;
    uint4 wg[4], wu[4];
    dequant32(*reinterpret_cast<const uint4*>(p.b0.qweight + rowi * (K / 8) + kb / 8),
              p.b0.scales[rowi * (K / p.G) + g], p.b0.biases[rowi * (K / p.G) + g], wg);
    dequant32(*reinterpret_cast<const uint4*>(p.b1.qweight + rowi * (K / 8) + kb / 8),
              p.b1.scales[rowi * (K / p.G) + g], p.b1.biases[rowi * (K / p.G) + g], wu);
#pragma unroll
    for (int m = 0; m < kGemvMaxTokens; m++) {
      if (tok[m] < 0) continue;
      const uint4* xp = reinterpret_cast<const uint4*>(p.a + (size_t)tok[m] * K + kb);
      uint4 xv[4] = {xp[0], xp[1], xp[2], xp[3]};
      ag[m] = dot32(wg, xv, ag[m]);
      au[m] = dot32(wu, xv, au[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < kGemvMaxTokens; m++) {
    if (m >= rows) break;
    float g = ag[m], u = au[m];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      g += __shfl_xor(g, off);
      u += __shfl_xor(u, off);
    }
    if (lane == 0 && tok[m] >= 0)  // h in operand order (see the MFMA kernel)
      reinterpret_cast<half_t*>(p.out)[(size_t)(row0 + m) * p.N + (n & ~7) + interleaved_pos(n & 7)] =
          (half_t)silu_mul(g, u);
  }
}

// S7 at decode sizes: a group of L lanes (L = largest power of two <=
// min(64, K/32)) owns one output row n of the down bank; a wave covers 64/L
// rows, a workgroup 4 waves.  a = h fp16 [P][K], already in the dequantised
// code order.
__global__ __launch_bounds__(256) void gemv_down_kernel(const GemvParams p, int L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = 64 / L;
  const int ng = p.N / (4 * R);
  const int tile = blockIdx.x / ng;
  const int n = (blockIdx.x % ng) * 4 * R + wave * R + lane / L;
  const int j = lane % L;
  int e, row0, rows;
  if (!read_tile(p, tile, e, row0, rows)) return;
  const int K = p.K;
  float wgt[kGemvMaxTokens];
#pragma unroll
  for (int m = 0; m < kGemvMaxTokens; m++) {
    const int pair = m < rows ? p.sorted_pairs[row0 + m] : -1;
    wgt[m] = (pair >= 0 && pair < p.P) ? p.topk_weights[pair] : 0.0f;
  }
  float acc[kGemvMaxTokens] = {};
  const size_t rowi = (size_t)e * p.N + n;
  for (int kb = 32 * j; kb < K; kb += 32 * L) {
    const int g = kb / p.G;
    uint4 w[4];
    dequant32(*reinterpret_cast<const uint4*>(p.b0.qweight + rowi * (K / 8) + kb / 8),
              p.b0.scales[rowi * (K / p.G) + g], p.b0.biases[rowi * (K / p.G) + g], w);
#pragma unroll
    for (int m = 0; m < kGemvMaxTokens; m++) {
      if (m >= rows) break;
      const uint4* hp = reinterpret_cast<const uint4*>(p.a + (size_t)(row0 + m) * K + kb);
      uint4 hv[4] = {hp[0], hp[1], hp[2], hp[3]};
      acc[m] = dot32(w, hv, acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < kGemvMaxTokens; m++) {
    if (m >= rows) break;
    float v = acc[m];
    for (int off = L / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (j == 0) reinterpret_cast<float*>(p.out)[(size_t)(row0 + m) * p.N + n] = wgt[m] * v;
  }
}

}  // namespace

hipError_t launch_w4_gemv(const GemmArgs& a, hipStream_t s) {
  const int64_t P = (int64_t)a.T * a.top_k;
  const int64_t max_blocks = P / a.block_m + (P < a.E ? P : a.E);
  GemvParams p{a.a, a.b0, a.b1, a.sorted_pairs, a.topk_weights, a.blocks, a.num_blocks, a.out,
               a.N, a.K, a.G, a.top_k, a.E, (int)P, (int)max_blocks};
  if (a.mode == MOE_GEMM_GATE_UP_SWIGLU) {
    gemv_gate_up_kernel<<<max_blocks * (a.N / 4), 256, 0, s>>>(p);
  } else {
    int L = 1;
    while (L * 2 <= 64 && L * 2 <= a.K / 32) L *= 2;
    const int R = 64 / L;
    gemv_down_kernel<<<max_blocks * (a.N / (4 * R)), 256, 0, s>>>(p, L);
  }
  return hipGetLastError();
}

}  // namespace moe
