// topk.h -- per-token top-k selection by one wave, and the S2-S5 build of
// a few pairs by one wave, both from LDS: the routing of decode-sized
// batches.  Page "Perplexity's Lily engine beats MLX by 35% on M5 Max",
// architecture paragraph: routing, histogram, prefix scan, scatter and the
// tile block map all run on the GPU, in the same submission as the experts.
// Device code only; included by route.hip and gemv.hip.
#pragma once
#include "internal.h"

namespace moe {
namespace {

constexpr int kSmallPairs = kGemvMaxTokens * 16;  // decode sizes: T <= 8 tokens, k <= 16
// Tiles of the decode block map (block_m = kGemvMaxTokens): at most
// kSmallPairs / block_m full tiles plus one ragged tile per touched expert.
constexpr int kSmallMaxBlocks = kSmallPairs / kGemvMaxTokens + kSmallPairs;


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

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(x, d);
    if (lane >= d) x += v;
  }
  return x;
}

// S2-S5 for at most kSmallPairs pairs, by the 64 lanes of one wave (the
// caller runs it on one wave only), with no block-wide scan.  ids: the P
// expert ids in pair order; cnt: the E expert counts (LDS, both filled by
// the caller); next: LDS scratch of E ints.  Outputs through generic
// pointers (LDS or global), counts only when non-null:
//   - exclusive prefix sums over the E <= 256 experts (4 consecutive experts
//     per lane, then a wave prefix sum): offsets, and the first tile of each
//     expert for the block map;
//   - the stable scatter of the pairs in order, 64 at a time: lanes with the
//     same expert are matched with ballots over the expert-id bits, and a
//     lane's slot is its expert's next free slot plus the number of matching
//     lanes below it (a counting sort that keeps pair order in each expert).
__device__ __forceinline__ void small_build(const int32_t* ids, const int* cnt, int* next, int P, int E,
                                            int block_m, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                                            int32_t* pair_slot, int32_t* blocks, int32_t* num_blocks) {
  const int lane = threadIdx.x & 63;
  // expert e = 4 lane + i
  int c[4], tl[4], cs = 0, ts = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = 4 * lane + i;
    c[i] = e < E ? cnt[e] : 0;
    tl[i] = (c[i] + block_m - 1) / block_m;
    cs += c[i];
    ts += tl[i];
  }
  int off = wave_inclusive_sum(cs) - cs, tile = wave_inclusive_sum(ts) - ts;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = 4 * lane + i;
    if (e < E) {
      if (counts) counts[e] = c[i];
      offsets[e] = off;
      next[e] = off;
      for (int j = 0; j < tl[i]; j++) {
        int32_t* blk = blocks + 3 * (size_t)(tile + j);
        blk[0] = e;
        blk[1] = off + j * block_m;
        blk[2] = min(block_m, c[i] - j * block_m);
      }
    }
    off += c[i];
    tile += tl[i];
  }
  if (lane == 63) {
    offsets[E] = P;
    num_blocks[0] = tile;  // total tiles (inclusive sum of the last lane)
  }
  wave_lds_sync();
  int bits = 1;
  while ((1 << bits) < E) bits++;
  for (int base = 0; base < P; base += 64) {
    const int q = base + lane;
    const int id = q < P ? ids[q] : -1;
    const bool active = id >= 0 && id < E;
    const int ex = active ? id : 0;
    uint64_t match = __ballot(active);
    for (int bt = 0; bt < bits; bt++) {
      const bool bit = (ex >> bt) & 1;
      const uint64_t bal = __ballot(bit);
      match &= bit ? bal : ~bal;
    }
    const uint64_t below = match & ((1ull << lane) - 1ull);
    const int start = active ? next[ex] : 0;
    wave_lds_sync();
    if (active) {
      const int slot = start + __popcll(below);
      sorted_pairs[slot] = q;
      pair_slot[q] = slot;
      if (below == 0) next[ex] = start + __popcll(match);  // lowest lane of its group
    }
    wave_lds_sync();
  }
}

}  // namespace
}  // namespace moe
