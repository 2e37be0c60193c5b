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

// Inverse of ordered_bits (-0.0 comes back as +0.0).
__device__ __forceinline__ float ordered_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Largest value over the 64 lanes of a wave, returned to every lane, on DPP
// lane moves: two quad permutations and two row rotations give each 16-lane
// row its maximum, then two row broadcasts combine rows 0-1 into lane 31
// and all rows into lane 63, which is read out.  Lanes a broadcast does not
// reach compare against 0, the smallest value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#define MOE_DPP_MAX(ctrl, row_mask) \
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, row_mask, 0xF, false))
  MOE_DPP_MAX(0xB1, 0xF);   // quad_perm 1,0,3,2
  MOE_DPP_MAX(0x4E, 0xF);   // quad_perm 2,3,0,1
  MOE_DPP_MAX(0x124, 0xF);  // row_ror:4
  MOE_DPP_MAX(0x128, 0xF);  // row_ror:8
  MOE_DPP_MAX(0x142, 0xA);  // row_bcast:15 -> rows 1, 3
  MOE_DPP_MAX(0x143, 0xC);  // row_bcast:31 -> rows 2, 3
#undef MOE_DPP_MAX
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of one token by a whole wave, the E logits at l[0..E), k <= 64:
// k rounds, each taking the largest remaining order-preserving key (a wave
// maximum) and, among the keys equal to it, the lowest expert index, so the
// choices come out in (logit descending, index ascending) order.  Lane j < k
// keeps choice j.  The combine weights are a softmax over the k chosen
// logits, shifted by the largest, the denominator summed in rank order.
// The wave writes ids[0..k) and w[0..k) and, when hist != nullptr, counts
// the chosen experts.
template <int NK>
__device__ void topk_token(const float* l, int E, int k, int32_t* ids, float* w, int* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NK];
#pragma unroll
  for (int i = 0; i < NK; i++) {
    const int e = lane + 64 * i;
    key[i] = e < E ? ordered_bits(l[e]) : 0u;  // every real key is > 0
  }
  uint32_t kj = 0, m0 = 0;  // lane j < k: the j-th chosen key; m0: the largest
  int ej = 0;               // lane j < k: the j-th chosen expert
  for (int j = 0; j < k; j++) {
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < NK; i++) m = max(m, key[i]);
    m = wave_max_u32(m);
    int owner = -1;
#pragma unroll
    for (int i = 0; i < NK; i++) {
      const uint64_t b = __ballot(key[i] == m);
      if (owner < 0 && b) owner = 64 * i + __ffsll((long long)b) - 1;
    }
#pragma unroll
    for (int i = 0; i < NK; i++)
      if (lane + 64 * i == owner) key[i] = 0u;  // taken
    if (j == 0) m0 = m;
    if (lane == j) {
      kj = m;
      ej = owner;
    }
  }
  const float mx = ordered_value(m0);
  const float a = lane < k ? expf(ordered_value(kj) - mx) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < k; j++) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), j));
  if (lane < k) {
    ids[lane] = ej;
    w[lane] = a / sum;
    if (hist) atomicAdd(&hist[ej], 1);
  }
}


// S2-S5 for at most kSmallPairs pairs, by the 64 lanes of one wave (the
// caller runs it on one wave only), with no block-wide scan.  ids: the P
// expert ids in pair order; cnt: the E expert counts (LDS, both filled by
// the caller); next: LDS scratch of E ints.  Outputs through generic
// pointers (LDS or global), counts only when non-null; no block-map entry
// at or past max_tiles (and no slot past P) is written:
//   - exclusive prefix sums over the E <= 256 experts (4 consecutive experts
//     per lane, then a wave prefix sum): offsets, and the first tile of each
//     expert for the block map;
//   - the stable scatter of the pairs in order, 64 at a time: lanes with the
//     same expert are matched with ballots over the expert-id bits, and a
//     lane's slot is its expert's next free slot plus the number of matching
//     lanes below it (a counting sort that keeps pair order in each expert).
__device__ __forceinline__ void small_build(const int32_t* ids, const int* cnt, int* next, int P, int E,
                                            int block_m, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                                            int32_t* pair_slot, int32_t* blocks, int32_t* num_blocks,
                                            int max_tiles) {
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
      for (int j = 0; j < tl[i] && tile + j < max_tiles; j++) {
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
    num_blocks[0] = min(tile, max_tiles);  // total tiles (inclusive sum of the last lane)
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
    const int slot = start + __popcll(below);
    if (active && slot < P) {
      sorted_pairs[slot] = q;
      pair_slot[q] = slot;
      if (below == 0) next[ex] = start + __popcll(match);  // lowest lane of its group
    }
    wave_lds_sync();
  }
}

}  // namespace
}  // namespace moe
