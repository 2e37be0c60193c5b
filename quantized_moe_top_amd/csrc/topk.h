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


// S2-S5 at decode sizes by a whole workgroup, in three phases separated by
// barriers (the caller's barrier ends the third).  ids: the P <= kSmallPairs
// expert ids in pair order p = t * k + j, T <= block_m tokens, every token
// choosing distinct experts; cnt: the E <= 256 expert counts; tokmask: LDS,
// E words, zero on entry; wsc: LDS, 8 ints.  So each expert holds at most
// block_m pairs: one tile.  Outputs (LDS): offsets[0..E], the stable scatter
// (sorted_pairs, pair_slot), the block map (at most max_tiles tiles, in
// expert order) and its tile count.
//   A. per pair, the token's bit in its expert's token mask; per 64-expert
//      chunk (one wave), the inclusive prefix of the counts and a ballot of
//      the touched experts, the chunk's totals to wsc;
//   B. per expert, its offset (the chunks before it plus the prefix) and,
//      when touched, its tile (the touched experts before it);
//   C. per pair, its slot: the expert's offset plus the tokens before it
//      that chose the same expert (pair order within an expert is token
//      order), which is the stable counting sort.
__device__ __forceinline__ void decode_build_wg(const int32_t* ids, const int* cnt, uint32_t* tokmask,
                                                int* wsc, int P, int E, int k, int32_t* offsets,
                                                int32_t* sorted_pairs, int32_t* pair_slot, int32_t* blocks,
                                                int32_t* num_blocks, int max_tiles) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), nwaves = blockDim.x >> 6;
  const int nch = (E + 63) / 64;
  for (int p = tid; p < P; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicOr(&tokmask[e], 1u << (p / k));
  }
  int incl[4] = {0, 0, 0, 0};
  uint64_t touched[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int c = wave + i * nwaves;
    if (c >= nch) break;
    const int e = 64 * c + lane;
    const int n = e < E ? cnt[e] : 0;
    incl[i] = wave_inclusive_sum(n);
    touched[i] = __ballot(n > 0);
    if (lane == 63) {
      wsc[c] = incl[i];
      wsc[4 + c] = __popcll(touched[i]);
    }
  }
  __syncthreads();
  int ntiles = 0;
  for (int c = 0; c < nch; c++) ntiles += wsc[4 + c];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int c = wave + i * nwaves;
    if (c >= nch) break;
    const int e = 64 * c + lane;
    int base = 0, tbase = 0;
    for (int c2 = 0; c2 < c; c2++) {
      base += wsc[c2];
      tbase += wsc[4 + c2];
    }
    const int n = e < E ? cnt[e] : 0;
    const int off = base + incl[i] - n;
    if (e < E) offsets[e] = off;
    const int tile = tbase + __popcll(touched[i] & ((1ull << lane) - 1ull));
    if (n > 0 && tile < max_tiles) {
      blocks[3 * tile] = e;
      blocks[3 * tile + 1] = off;
      blocks[3 * tile + 2] = n;
    }
  }
  if (tid == 0) {
    offsets[E] = P;
    num_blocks[0] = min(ntiles, max_tiles);
  }
  __syncthreads();
  for (int p = tid; p < P; p += blockDim.x) {
    const int e = ids[p];
    if (e < 0 || e >= E) continue;
    const int slot = offsets[e] + __popc(tokmask[e] & ((1u << (p / k)) - 1u));
    if (slot < P) {
      sorted_pairs[slot] = p;
      pair_slot[p] = slot;
    }
  }
}

}  // namespace
}  // namespace moe
