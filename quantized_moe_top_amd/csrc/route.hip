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
// tokens and walks it in passes of 8, 32 or 64 tokens (64, 16 or 8 lanes
// per token):
//   1. the pass's logits into LDS;
//   2. top-k per token, in (logit descending, index ascending) order: for
//      chunks of at most 8 tokens a wave per token runs a radix select
//      (topk_token); for larger chunks a group of 16 or 8 lanes per token
//      keeps per-lane sorted lists of 64-bit keys (logit image, inverted
//      index) and merges them across the group by bitonic merges
//      (topk_group), all on the VALU, so many tokens proceed at once;
//   3. (whole-layer mode) the chunk's expert histogram (LDS atomics: counts
//      do not depend on order), and x bf16 -> fp16 in the interleaved order
//      the grouped GEMM reads.
#include "scan_scatter.h"

namespace moe {
namespace {

constexpr int kLgFloats = 16384;  // LDS logits of one pass (64 KiB)
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
  int lpt_log2;         // lanes per token in the top-k (log2)
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

// Top-k of one token by a whole wave (few tokens per chunk: the serial
// chain of ballots is shorter than the merges of a lane group), the E
// logits at l[0..E): a 32-round radix select over the order-preserving
// keys (each round a ballot count of keys at or above the candidate) finds
// the k-th largest key; keys above it and the lowest-index keys equal to it
// are the selection; ranks among the selected give (logit descending, index
// ascending) order.  The wave writes ids[0..k) and w[0..k) and, when
// hist != nullptr, counts the chosen experts.
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

// Selection key of expert e with logit v: the order-preserving image of v
// in the high word and ~e in the low word, so a larger key is a larger logit
// or, between equal logits, the lower expert index (the tie rule).  Every
// key of a real expert is above 0, the key of an empty slot.
__device__ __forceinline__ uint64_t sel_key(float v, int e) {
  return ((uint64_t)ordered_bits(v) << 32) | (uint32_t)~e;
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Partner value for butterfly round m of a lane group: lanes 0..m-1 and
// m..2m-1 of every 2m-lane block are paired up.  Up to 8 the pairing runs
// on DPP lane moves inside the VALU (quad permutations for 1 and 2, the
// 8- and 16-lane mirrors for 4 and 8, which pair lane i with 2m - 1 - i);
// beyond, a ds_bpermute exchange with lane ^ m.
template <int M>
__device__ __forceinline__ uint32_t partner32(uint32_t v) {
  const int x = (int)v;
  if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);   // quad_perm 1,0,3,2
  else if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);   // quad_perm 2,3,0,1
  else if constexpr (M == 4) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);  // row_half_mirror
  else if constexpr (M == 8) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true);  // row_mirror
  else return (uint32_t)__shfl_xor(x, M);
}
template <int M>
__device__ __forceinline__ uint64_t partner64(uint64_t v) {
  return ((uint64_t)partner32<M>((uint32_t)(v >> 32)) << 32) | partner32<M>((uint32_t)v);
}


// Compare-exchange: K[i] gets the larger key, K[j] the smaller.
__device__ __forceinline__ void cex(uint64_t& a, uint64_t& b) {
  const uint64_t x = a, y = b;
  const bool gt = x > y;
  a = gt ? x : y;
  b = gt ? y : x;
}

// Sorts a bitonic sequence of L keys into descending order.
template <int L>
__device__ __forceinline__ void bitonic_merge_desc(uint64_t (&K)[L]) {
#pragma unroll
  for (int d = L / 2; d >= 1; d >>= 1)
#pragma unroll
    for (int i = 0; i < L; i++)
      if ((i & d) == 0) cex(K[i], K[i + d]);
}

// Sorts L arbitrary keys into descending order (bitonic sorting network).
template <int L>
__device__ __forceinline__ void bitonic_sort_desc(uint64_t (&K)[L]) {
#pragma unroll
  for (int size = 2; size <= L; size <<= 1)
#pragma unroll
    for (int d = size / 2; d >= 1; d >>= 1)
#pragma unroll
      for (int i = 0; i < L; i++)
        if ((i & d) == 0) {
          if ((i & size) == 0) cex(K[i], K[i + d]);
          else cex(K[i + d], K[i]);
        }
}

// K = the L largest of K and P, both sorted descending: the elementwise
// larger of K and reversed P is a bitonic sequence holding them.
template <int L>
__device__ __forceinline__ void merge_top(uint64_t (&K)[L], const uint64_t (&P)[L]) {
#pragma unroll
  for (int i = 0; i < L; i++) K[i] = K[i] > P[L - 1 - i] ? K[i] : P[L - 1 - i];
  bitonic_merge_desc<L>(K);
}

// Butterfly rounds M, 2M, ... below LPT (unrolled at compile time).
template <int L, int LPT, int M>
__device__ __forceinline__ void butterfly(uint64_t (&K)[L]) {
  if constexpr (M < LPT) {
    uint64_t P[L];
#pragma unroll
    for (int i = 0; i < L; i++) P[i] = partner64<M>(K[i]);
    merge_top<L>(K, P);
    butterfly<L, LPT, 2 * M>(K);
  }
}

// Top-k of one token by a group of LPT consecutive lanes (LPT in {8, 16,
// 64}), sub = lane within the group, l = the token's E logits.
//  1. Lane sub keeps the L largest keys (L >= k) of experts sub, sub + lpt,
//     ..., sorted in descending order: blocks of L keys are sorted by a
//     bitonic network and merged into the list.
//  2. log2(lpt) butterfly rounds: a lane and its partner hold the sorted top
//     L of disjoint expert sets and both merge them into the top L of the
//     union, so after the last round every lane holds the token's top L in
//     (logit descending, index ascending) order: rank j is entry j.
//  3. Softmax over the first k logits, max-subtracted, the denominator
//     summed in rank order; lane sub writes ranks sub, sub + lpt, ... < k
//     and, when hist != nullptr, counts the chosen experts.
// All branches are uniform over the group, so a group never diverges.
template <int L, int LPT>
__device__ __forceinline__ void topk_group(const float* l, int E, int k, int sub, int32_t* ids,
                                           float* w, int* hist) {
  constexpr int lpt = LPT;
  uint64_t K[L];
  for (int base = 0; base < E; base += L * lpt) {
    uint64_t B[L];
#pragma unroll
    for (int i = 0; i < L; i++) {
      const int e = base + sub + lpt * i;
      B[i] = e < E ? sel_key(l[e], e) : 0;
    }
    bitonic_sort_desc<L>(B);
    if (base == 0) {
#pragma unroll
      for (int i = 0; i < L; i++) K[i] = B[i];
    } else {
      merge_top<L>(K, B);
    }
  }
  butterfly<L, LPT, 1>(K);
  const float mx = key_logit(K[0]);
  float a[L];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < L; j++) {
    a[j] = j < k ? expf(key_logit(K[j]) - mx) : 0.0f;
    sum += a[j];  // rank order; the terms past k are 0
  }
#pragma unroll
  for (int j = 0; j < L; j++) {
    if (j < k && (j & (lpt - 1)) == sub) {
      const int e = key_expert(K[j]);
      ids[j] = e;
      w[j] = a[j] / sum;
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

// Logits of tokens [t0, t0 + nt) into lg[nt][stride] (rows padded so that
// the lane groups of a wave read different LDS banks).
__device__ void load_logits(const RouteParams& p, int t0, int nt, float* lg, int stride) {
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
      if (i < n) {
        const int r = i / p.E;
        lg[r * stride + (i - r * p.E)] = v[u];
      }
    }
  }
}

// One chunk of tokens, in passes of kRouteThreads / LPT tokens (one group of
// LPT lanes per token).  LPT = 64: radix select by a wave, A = ceil(E / 64)
// keys per lane; LPT = 8 or 16: sort-merge top-k, A = L, the list length.
template <bool FULL, int A, int LPT>
__device__ __forceinline__ void route_chunk(const RouteParams& p, int chunk) {
  __shared__ float lg[kLgFloats];
  __shared__ int hist[256];
  const int tid = threadIdx.x;
  constexpr int tp = kRouteThreads / LPT;
  const int stride = p.E + LPT;
  const int grp = tid / LPT, sub = tid % LPT;
  if (FULL && tid < 256) hist[tid] = 0;
  const int c0 = chunk * p.chunk_tokens;
  const int c1 = min(p.T, c0 + p.chunk_tokens);
  for (int t0 = c0; t0 < c1; t0 += tp) {
    const int nt = min(tp, c1 - t0);
    load_logits(p, t0, nt, lg, stride);
    if (FULL) stage_rows(p, t0, nt);
    __syncthreads();
    if (grp < nt)
    {
      int32_t* ids = p.ids + (size_t)(t0 + grp) * p.k;
      float* w = p.w + (size_t)(t0 + grp) * p.k;
      if constexpr (LPT == 64) topk_token<A>(lg + grp * stride, p.E, p.k, ids, w, FULL ? hist : nullptr);
      else topk_group<A, LPT>(lg + grp * stride, p.E, p.k, sub, ids, w, FULL ? hist : nullptr);
    }
    __syncthreads();
  }
  if (FULL && tid < p.E) p.chunk_hist[(size_t)chunk * p.E + tid] = hist[tid];
}

template <bool FULL, int A, int LPT>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const RouteParams p) {
  route_chunk<FULL, A, LPT>(p, blockIdx.x);
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
  route_chunk<true, NK, 64>(p, 0);  // at most 8 tokens: a wave each
  __threadfence_block();
  __syncthreads();
  scan_scatter_chunk(p.ids, p.T * p.k, p.E, p.chunk_tokens * p.k, 1, p.chunk_hist, b.block_m,
                     b.counts, b.offsets, b.sorted_pairs, b.pair_slot, b.blocks, b.num_blocks, 0);
}

// List length L of the top-k: the power of two in {2, 4, 8, 16} at or above k.
template <bool FULL, int L>
void launch_route_group(const RouteParams& p, int nchunks, hipStream_t s) {
  if (p.lpt_log2 == 3) route_kernel<FULL, L, 8><<<nchunks, kRouteThreads, 0, s>>>(p);
  else route_kernel<FULL, L, 16><<<nchunks, kRouteThreads, 0, s>>>(p);
}

template <bool FULL>
hipError_t launch_route_l(const RouteParams& p, int nchunks, hipStream_t s) {
  if (p.lpt_log2 == 6) {
    switch ((p.E + 63) / 64) {
      case 1: route_kernel<FULL, 1, 64><<<nchunks, kRouteThreads, 0, s>>>(p); break;
      case 2: route_kernel<FULL, 2, 64><<<nchunks, kRouteThreads, 0, s>>>(p); break;
      case 3: route_kernel<FULL, 3, 64><<<nchunks, kRouteThreads, 0, s>>>(p); break;
      default: route_kernel<FULL, 4, 64><<<nchunks, kRouteThreads, 0, s>>>(p); break;
    }
  } else if (p.k <= 2) launch_route_group<FULL, 2>(p, nchunks, s);
  else if (p.k <= 4) launch_route_group<FULL, 4>(p, nchunks, s);
  else if (p.k <= 8) launch_route_group<FULL, 8>(p, nchunks, s);
  else launch_route_group<FULL, 16>(p, nchunks, s);
  return hipGetLastError();
}

// Lanes per token (log2): a wave per token (radix select) for chunks of at
// most 8 tokens; 16 lanes for chunks of up to 32 tokens; otherwise 8
// (passes of 64 tokens) when their logits fit the LDS rows.
int route_lpt_log2(int chunk_tokens, int E) {
  if (chunk_tokens <= 8) return 6;
  if (chunk_tokens <= 32 || (kRouteThreads / 8) * (E + 8) > kLgFloats) return 4;
  return 3;
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
  const int ct = route_chunk_tokens(T);
  RouteParams p{x, logits, ids, w, xh, chunk_hist, T, H, E, k, ct, route_lpt_log2(ct, E)};
  const int n = route_chunks(T);
  return xh ? launch_route_l<true>(p, n, s) : launch_route_l<false>(p, n, s);
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
  const int ct = route_chunk_tokens(T);
  RouteParams p{x, logits, ids, w, xh, chunk_hist, T, H, E, k, ct, route_lpt_log2(ct, E)};
  BuildParams b{block_m, counts, offsets, sorted_pairs, pair_slot, blocks, num_blocks};
  switch ((E + 63) / 64) {
    case 1: route_build_kernel<1><<<1, kRouteThreads, 0, s>>>(p, b); break;
    case 2: route_build_kernel<2><<<1, kRouteThreads, 0, s>>>(p, b); break;
    case 3: route_build_kernel<3><<<1, kRouteThreads, 0, s>>>(p, b); break;
    default: route_build_kernel<4><<<1, kRouteThreads, 0, s>>>(p, b); break;
  }
  return hipGetLastError();
}

}  // namespace moe
