// gemv.hip -- S9: the grouped W4 GEMM at decode sizes (T <= 8).  With at most
// 8 rows per expert the product is bound by reading the packed weights, so
// each touched expert's weights are streamed once and experts that no token
// chose are never read.
//
// One workgroup (8 waves) per (tile, 32-column block).  In the packed layout
// (see moe_w4_pack) each 64-wide reduction slab of a 32-column block is one
// contiguous 1 KiB piece, read by one wave instruction: lane l holds 32
// codes of column l / 2, reduction half l % 2.  The 8 waves take the slabs
// in turn (wave w: slabs w, w + 8, ...); each lane dequantises its codes in
// registers (same exact fp16 dequantisation as the MFMA path) and dots them
// with the activation rows routed to the tile using v_dot2_f32_f16 (fp16
// products, fp32 accumulation).  The two halves of a column are added with
// one lane exchange, the 8 waves' partial sums through LDS in wave order, so
// the result does not depend on timing.
#include "internal.h"

namespace moe {
namespace {

constexpr int kGemvWaves = 8;
constexpr int kGemvThreads = 64 * kGemvWaves;

struct GemvParams {
  const half_t* a;
  moe_w4_packed b0, b1;
  const int32_t* sorted_pairs;
  const float* topk_weights;
  const int32_t* blocks;
  const int32_t* num_blocks;
  void* out;
  int N, K, log2_G, top_k, E, P, max_blocks;
};

// 32 fp16 products summed into acc.  Each vector element is copied into a
// scalar before the bit cast: a bit cast applied to a vector-element lvalue
// was compiled to read element 0 for every index.
__device__ __forceinline__ float dot32(const u32x4* w, const u32x4* x, float acc) {
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const uint32_t wc = w[i][c], xc = x[i][c];
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, wc), __builtin_bit_cast(half2_t, xc),
                                   acc, false);
    }
  return acc;
}

// 32 codes (16 bytes) of one column and reduction half -> 32 fp16 weights
// in operand order, with the packed (scale, bias) word sb.
__device__ __forceinline__ void dequant32(const u32x4 q, uint32_t sb, u32x4* w) {
  const half2_t s2 = bf16_pair_to_half2(sb & 0xFFFFu), b2 = bf16_pair_to_half2(sb >> 16);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint4 d = dequant_word(q[i], s2, b2);
    w[i] = u32x4{d.x, d.y, d.z, d.w};
  }
}

template <int MODE>
__global__ __launch_bounds__(kGemvThreads) void w4_gemv_kernel(const GemvParams p) {
  constexpr bool GATE_UP = MODE == MOE_GEMM_GATE_UP_SWIGLU;
  constexpr int NB = GATE_UP ? 2 : 1;  // banks read: gate and up, or down
  __shared__ float red[kGemvWaves][NB][kGemvMaxTokens][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 1, half = lane & 1;
  const int nbl = p.N / 32;
  const int tile = blockIdx.x / nbl, blk = blockIdx.x % nbl;

  const int nblk = min(*p.num_blocks, p.max_blocks);
  if (tile >= nblk) return;
  const int e = p.blocks[3 * tile], row0 = p.blocks[3 * tile + 1], rows = p.blocks[3 * tile + 2];
  // a malformed block map is skipped, never dereferenced out of bounds
  if (e < 0 || e >= p.E || rows <= 0 || rows > kGemvMaxTokens || row0 < 0 || row0 > p.P - rows)
    return;
  const int K = p.K, S = K / 64, gpr = K >> p.log2_G;

  // activation row of each tile row: token x (S6) or slot h (S7), both
  // already in operand order
  int arow[kGemvMaxTokens];
#pragma unroll
  for (int m = 0; m < kGemvMaxTokens; m++) {
    int r = row0 + min(m, rows - 1);
    if (GATE_UP) {
      const int pair = p.sorted_pairs[r];
      r = (pair >= 0 && pair < p.P) ? pair / p.top_k : 0;
    }
    arow[m] = r;
  }

  const size_t bidx = (size_t)e * nbl + blk;
  float acc[NB][kGemvMaxTokens];
#pragma unroll
  for (int b = 0; b < NB; b++)
#pragma unroll
    for (int m = 0; m < kGemvMaxTokens; m++) acc[b][m] = 0.0f;

  for (int s = wave; s < S; s += kGemvWaves) {
    const int g = (64 * s + 32 * half) >> p.log2_G;
    u32x4 w[NB][4];
#pragma unroll
    for (int b = 0; b < NB; b++) {
      const moe_w4_packed& bank = b == 0 ? p.b0 : p.b1;
      const u32x4 q = *reinterpret_cast<const u32x4*>(
          bank.words + (((bidx >> 2) * S + s) * 4 + (bidx & 3)) * 256 + 4 * lane);
      const uint32_t sb = bank.sb[((bidx >> 2) * gpr + g) * 128 + (bidx & 3) * 32 + c];
      dequant32(q, sb, w[b]);
    }
#pragma unroll
    for (int m = 0; m < kGemvMaxTokens; m++) {
      if (m >= rows) break;
      const u32x4* xp =
          reinterpret_cast<const u32x4*>(p.a + (size_t)arow[m] * K + 64 * s + 32 * half);
      u32x4 xv[4] = {xp[0], xp[1], xp[2], xp[3]};
#pragma unroll
      for (int b = 0; b < NB; b++) acc[b][m] = dot32(w[b], xv, acc[b][m]);
    }
  }
  // the column's two reduction halves, then the waves in order
#pragma unroll
  for (int b = 0; b < NB; b++)
#pragma unroll
    for (int m = 0; m < kGemvMaxTokens; m++) {
      const float v = acc[b][m] + __shfl_xor(acc[b][m], 1);
      if (half == 0) red[wave][b][m][c] = v;
    }
  __syncthreads();
  if (tid >= rows * 32) return;
  const int m = tid >> 5, cc = tid & 31;
  float v[NB];
#pragma unroll
  for (int b = 0; b < NB; b++) {
    v[b] = red[0][b][m][cc];
#pragma unroll
    for (int w2 = 1; w2 < kGemvWaves; w2++) v[b] += red[w2][b][m][cc];
  }
  const int n = blk * 32 + cc;
  if (GATE_UP) {
    // h in operand order (see the MFMA kernel)
    reinterpret_cast<half_t*>(p.out)[(size_t)(row0 + m) * p.N + (n & ~7) + interleaved_pos(n & 7)] =
        (half_t)silu_mul(v[0], v[NB - 1]);
  } else {
    const int pair = p.sorted_pairs[row0 + m];
    const float wgt = (pair >= 0 && pair < p.P) ? p.topk_weights[pair] : 0.0f;
    reinterpret_cast<float*>(p.out)[(size_t)(row0 + m) * p.N + n] = wgt * v[0];
  }
}

}  // namespace

hipError_t launch_w4_gemv(const GemmArgs& a, hipStream_t s) {
  const int64_t P = (int64_t)a.T * a.top_k;
  const int64_t max_blocks = P / a.block_m + (P < a.E ? P : a.E);
  const int log2_G = a.G == 32 ? 5 : a.G == 64 ? 6 : 7;  // G in {32, 64, 128}
  GemvParams p{a.a, a.b0, a.b1, a.sorted_pairs, a.topk_weights, a.blocks, a.num_blocks, a.out,
               a.N, a.K, log2_G, a.top_k, a.E, (int)P, (int)max_blocks};
  const int64_t grid = max_blocks * (a.N / 32);
  if (a.mode == MOE_GEMM_GATE_UP_SWIGLU)
    w4_gemv_kernel<MOE_GEMM_GATE_UP_SWIGLU><<<grid, kGemvThreads, 0, s>>>(p);
  else
    w4_gemv_kernel<MOE_GEMM_DOWN><<<grid, kGemvThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
