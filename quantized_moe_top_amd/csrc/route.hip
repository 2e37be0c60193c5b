// route.hip -- S0 router linear layer and S1 top-k routing with combine
// weights, fused with the first half of S2 (per-chunk expert histogram) and
// with the fp16 operand staging of the activations.  Page "Perplexity's
// Lily engine beats MLX by 35% on M5 Max", architecture paragraph: expert
// routing runs on the GPU in the same submission as the rest of the layer.
//
// S0 (only when a router weight is given) is its own kernel: one
// workgroup per 32-token x 32-expert tile of the logits, on
// v_mfma_f32_32x32x16_bf16, with the H sums split over the workgroup's 8
// waves and added in a fixed order, so that a few hundred tokens already
// fill the chip and the logits are deterministic.
//
// The routing kernel: one workgroup (8 waves) owns a chunk of consecutive
// tokens and walks it in sub-tiles of up to 32 tokens:
//   1. the sub-tile's logits into LDS;
//   2. top-k per token, one wave per token, by a radix select over the
//      order-preserving integer image of the logits: 32 rounds of a
//      wave-wide ballot count find the k-th largest key; keys above it and
//      the lowest-index keys equal to it are the selection; ranks among the
//      k selected give (logit descending, index ascending) order;
//   3. (whole-layer mode) the chunk's expert histogram (LDS atomics: counts
//      do not depend on order), and x bf16 -> fp16 in the interleaved order
//      the grouped GEMM reads.
#include "scan_scatter.h"

namespace moe {
namespace {

constexpr int kSub = 32;        // tokens per sub-tile
constexpr int kRouteThreads = 512;
constexpr int kRouterBatch = 16;  // MFMA steps whose loads are issued together

// ------------------------------------------------------------------ S0 ---
// logits[t][e] = sum_h x[t][h] * wr[e][h] for one 32-token x 32-expert tile
// per workgroup.  The 8 waves split the H sums into 8 contiguous ranges,
// each wave issuing the loads of its whole range at once (H <= 4096: one
// round trip); their 32x32 partial tiles are added in wave order through
// LDS, so the result does not depend on timing.  One-dimensional grid of
// ceil(T/32) * ceil(E/32) workgroups, expert tile fastest: the expert tiles
// of one token tile are dispatched together, so x is read from HBM once and
// shared through L2.
constexpr int kRouterWaves = 8;
__global__ __launch_bounds__(64 * kRouterWaves) void router_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, float* __restrict__ logits,
    int T, int H, int E) {
  __shared__ float red[kRouterWaves][32 * 33];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, half = lane >> 5;
  const int ne = (E + 31) / 32;
  const int t0 = (blockIdx.x / ne) * 32, e0 = (blockIdx.x % ne) * 32;
  const int t = min(t0 + r, T - 1);  // rows past T or E read a valid row, never stored
  const int e = min(e0 + r, E - 1);
  const int steps = H / 16 / kRouterWaves;  // H % 128 == 0
  const uint4* xa = reinterpret_cast<const uint4*>(x + (size_t)t * H) + half + 2 * wave * steps;
  const uint4* wb = reinterpret_cast<const uint4*>(wr + (size_t)e * H) + half + 2 * wave * steps;
  floatx16_t acc = {};
  int s = 0;
  for (; s + kRouterBatch <= steps; s += kRouterBatch) {
    uint4 av[kRouterBatch], bv[kRouterBatch];
#pragma unroll
    for (int u = 0; u < kRouterBatch; u++) {
      av[u] = xa[2 * (s + u)];
      bv[u] = wb[2 * (s + u)];
    }
    // keep every load of the batch ahead of the first MFMA (one round trip),
    // instead of the compiler's rolling schedule with a few loads in flight
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kRouterBatch; u++)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[u]),
                                                    __builtin_bit_cast(bf16x8_t, bv[u]), acc, 0, 0,
                                                    0);
  }
  for (; s < steps; s++)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, xa[2 * s]),
                                                  __builtin_bit_cast(bf16x8_t, wb[2 * s]), acc, 0, 0,
                                                  0);
#pragma unroll
  for (int i = 0; i < 16; i++) red[wave][(8 * (i >> 2) + 4 * half + (i & 3)) * 33 + r] = acc[i];
  __syncthreads();
  // thread -> (row, col) of the tile, two elements each
  for (int idx = threadIdx.x; idx < 32 * 32; idx += 64 * kRouterWaves) {
    const int row = idx >> 5, col = idx & 31;
    float v = red[0][row * 33 + col];
#pragma unroll
    for (int w = 1; w < kRouterWaves; w++) v += red[w][row * 33 + col];
    if (t0 + row < T && e0 + col < E) logits[(size_t)(t0 + row) * E + e0 + col] = v;
  }
}

// -------------------------------------------------------------- S1, S2 ---
struct RouteParams {
  const uint16_t* x;    // bf16 [T][H] (staging)
  const float* logits;  // fp32 [T][E]
  int32_t* ids;         // [T][k]
  float* w;             // [T][k]
  half_t* xh;           // fp16 [T][H] staged activations (whole-layer mode)
  int32_t* chunk_hist;  // [nchunks][E] (whole-layer mode)
  int T, H, E, k, chunk_tokens;
};

// Order-preserving map of an fp32 bit pattern onto unsigned integers
// (-inf lowest, +inf highest).  -0.0 is folded onto +0.0 first: the two
// compare equal, so they must tie (and the tie goes to the lower expert).
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Top-k of one token whose E logits are l[0..E); the calling wave writes
// ids[0..k) and w[0..k) and, when hist != nullptr, counts the chosen experts.
template <int NK>
__device__ void topk_token(const float* l, int E, int k, int32_t* ids, float* w, int* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NK];
#pragma unroll
  for (int i = 0; i < NK; i++) {
    const int e = lane + 64 * i;
    key[i] = e < E ? ordered_bits(l[e]) : 0u;  // every real key is > 0
  }
  // theta = the k-th largest key: the largest value with >= k keys >= it
  uint32_t theta = 0;
  for (int b = 31; b >= 0; b--) {
    const uint32_t cand = theta | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NK; i++) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= k) theta = cand;
  }
  // selection: every key above theta, then keys equal to theta by index
  uint64_t sel[NK];
  int need = k;
#pragma unroll
  for (int i = 0; i < NK; i++) {
    sel[i] = __ballot(key[i] > theta);
    need -= __popcll(sel[i]);
  }
#pragma unroll
  for (int i = 0; i < NK; i++) {
    uint64_t m = __ballot(key[i] == theta);
    while (need > 0 && m) {
      const uint64_t low = m & (~m + 1ull);
      sel[i] |= low;
      m ^= low;
      need--;
    }
  }
  // rank of each selected key among the selected ones; the first maximum in
  // index order is rank 0
  int rank[NK];
#pragma unroll
  for (int i = 0; i < NK; i++) rank[i] = 0;
  uint32_t best = 0;
  int best_e = 0;
#pragma unroll
  for (int i2 = 0; i2 < NK; i2++) {
    uint64_t m = sel[i2];
    while (m) {
      const int l2 = __ffsll((long long)m) - 1;
      m &= m - 1;
      const uint32_t kv = (uint32_t)__builtin_amdgcn_readlane((int)key[i2], l2);
      const int e2 = 64 * i2 + l2;
      if (kv > best) {
        best = kv;
        best_e = e2;
      }
#pragma unroll
      for (int i = 0; i < NK; i++) {
        const int e = 64 * i + lane;
        rank[i] += (kv > key[i]) || (kv == key[i] && e2 < e);
      }
    }
  }
  // combine weights: softmax over the k chosen logits, max-subtracted, the
  // denominator summed in rank order
  const float mx = l[best_e];
  float a[NK];
  bool mine[NK];
#pragma unroll
  for (int i = 0; i < NK; i++) {
    mine[i] = (sel[i] >> lane) & 1ull;
    a[i] = mine[i] ? expf(l[lane + 64 * i] - mx) : 0.0f;
  }
  float sum = 0.0f;
  for (int j = 0; j < k; j++) {
#pragma unroll
    for (int i = 0; i < NK; i++) {
      const uint64_t m = __ballot(mine[i] && rank[i] == j);
      if (m) sum += readlane_f(a[i], __ffsll((long long)m) - 1);
    }
  }
#pragma unroll
  for (int i = 0; i < NK; i++) {
    if (mine[i]) {
      const int e = lane + 64 * i;
      ids[rank[i]] = e;
      w[rank[i]] = a[i] / sum;
      if (hist) atomicAdd(&hist[e], 1);
    }
  }
}

// bf16 -> fp16 of tokens [t0, t0 + nt), each 8-element chunk reordered to
// (0,4,1,5,2,6,3,7).  Loads use clamped indices so that each batch of U is
// issued together.
__device__ void stage_rows(const RouteParams& p, int t0, int nt) {
  const int n = nt * (p.H / 8);
  const uint4* in = reinterpret_cast<const uint4*>(p.x + (size_t)t0 * p.H);
  uint4* out = reinterpret_cast<uint4*>(p.xh + (size_t)t0 * p.H);
  constexpr int U = 8;
  for (int i0 = threadIdx.x; i0 < n; i0 += kRouteThreads * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = in[min(i0 + u * kRouteThreads, n - 1)];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = i0 + u * kRouteThreads;
      if (i < n) out[i] = bf16x8_to_half_interleaved(v[u]);
    }
  }
}

// Logits of tokens [t0, t0 + nt) into lg[nt][E].
__device__ void load_logits(const RouteParams& p, int t0, int nt, float* lg) {
  const int n = nt * p.E;
  const float* src = p.logits + (size_t)t0 * p.E;
  constexpr int U = 8;
  for (int i0 = threadIdx.x; i0 < n; i0 += kRouteThreads * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = src[min(i0 + u * kRouteThreads, n - 1)];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = i0 + u * kRouteThreads;
      if (i < n) lg[i] = v[u];
    }
  }
}

template <bool FULL, int NK>
__device__ __forceinline__ void route_chunk(const RouteParams& p, int chunk) {
  __shared__ float lg[kSub * 256];
  __shared__ int hist[256];
  const int tid = threadIdx.x, wave = tid >> 6;
  constexpr int kWaves = kRouteThreads / 64;
  if (FULL && tid < 256) hist[tid] = 0;
  const int c0 = chunk * p.chunk_tokens;
  const int c1 = min(p.T, c0 + p.chunk_tokens);
  for (int t0 = c0; t0 < c1; t0 += kSub) {
    const int nt = min(kSub, c1 - t0);
    load_logits(p, t0, nt, lg);
    if (FULL) stage_rows(p, t0, nt);
    __syncthreads();
    for (int r = wave; r < nt; r += kWaves)
      topk_token<NK>(lg + r * p.E, p.E, p.k, p.ids + (size_t)(t0 + r) * p.k,
                     p.w + (size_t)(t0 + r) * p.k, FULL ? hist : nullptr);
    __syncthreads();
  }
  if (FULL && tid < p.E) p.chunk_hist[(size_t)chunk * p.E + tid] = hist[tid];
}

template <bool FULL, int NK>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const RouteParams p) {
  route_chunk<FULL, NK>(p, blockIdx.x);
}

// Outputs of S2-S5 for the fused single-chunk kernel.
struct BuildParams {
  int block_m;
  int32_t *counts, *offsets, *sorted_pairs, *pair_slot, *blocks, *num_blocks;
};

// All tokens in one chunk (decode sizes): one workgroup routes them (S1),
// then, after a barrier that makes its ids and histogram visible to the
// whole workgroup, builds counts, offsets, the scatter and the block map
// (S2-S5): one launch instead of two, same results.
template <int NK>
__global__ __launch_bounds__(kRouteThreads) void route_build_kernel(const RouteParams p,
                                                                    const BuildParams b) {
  route_chunk<true, NK>(p, 0);
  __threadfence_block();
  __syncthreads();
  scan_scatter_chunk(p.ids, p.T * p.k, p.E, p.chunk_tokens * p.k, 1, p.chunk_hist, b.block_m,
                     b.counts, b.offsets, b.sorted_pairs, b.pair_slot, b.blocks, b.num_blocks, 0);
}

template <bool FULL>
hipError_t launch_nk(const RouteParams& p, int nchunks, hipStream_t s) {
  switch ((p.E + 63) / 64) {
    case 1: route_kernel<FULL, 1><<<nchunks, kRouteThreads, 0, s>>>(p); break;
    case 2: route_kernel<FULL, 2><<<nchunks, kRouteThreads, 0, s>>>(p); break;
    case 3: route_kernel<FULL, 3><<<nchunks, kRouteThreads, 0, s>>>(p); break;
    case 4: route_kernel<FULL, 4><<<nchunks, kRouteThreads, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int route_chunk_tokens(int64_t T) {
  // at least 8 tokens, at most 256 chunks, a multiple of 8
  const int64_t per = (T + 8 * 256 - 1) / (8 * 256);
  return (int)(8 * (per > 1 ? per : 1));
}

int route_chunks(int64_t T) {
  const int ct = route_chunk_tokens(T);
  return (int)((T + ct - 1) / ct);
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, float* logits, int T, int H, int E,
                        int k, int32_t* ids, float* w, half_t* xh, int32_t* chunk_hist,
                        hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (wr) {
    const int64_t grid = (int64_t)((E + 31) / 32) * ((T + 31) / 32);
    router_gemm_kernel<<<grid, 64 * kRouterWaves, 0, s>>>(x, wr, logits, T, H, E);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  RouteParams p{x, logits, ids, w, xh, chunk_hist, T, H, E, k, route_chunk_tokens(T)};
  const int n = route_chunks(T);
  return xh ? launch_nk<true>(p, n, s) : launch_nk<false>(p, n, s);
}

bool route_build_fused(int64_t T) { return route_chunks(T) == 1; }

hipError_t launch_route_build(const uint16_t* x, const uint16_t* wr, float* logits, int T, int H,
                              int E, int k, int32_t* ids, float* w, half_t* xh,
                              int32_t* chunk_hist, int block_m, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_pairs, int32_t* pair_slot, int32_t* blocks,
                              int32_t* num_blocks, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (wr) {
    const int64_t grid = (int64_t)((E + 31) / 32) * ((T + 31) / 32);
    router_gemm_kernel<<<grid, 64 * kRouterWaves, 0, s>>>(x, wr, logits, T, H, E);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  RouteParams p{x, logits, ids, w, xh, chunk_hist, T, H, E, k, route_chunk_tokens(T)};
  BuildParams b{block_m, counts, offsets, sorted_pairs, pair_slot, blocks, num_blocks};
  switch ((E + 63) / 64) {
    case 1: route_build_kernel<1><<<1, kRouteThreads, 0, s>>>(p, b); break;
    case 2: route_build_kernel<2><<<1, kRouteThreads, 0, s>>>(p, b); break;
    case 3: route_build_kernel<3><<<1, kRouteThreads, 0, s>>>(p, b); break;
    case 4: route_build_kernel<4><<<1, kRouteThreads, 0, s>>>(p, b); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
