// scan_scatter.h -- the body of S2-S5 for one chunk of pairs (exclusive scan
// of the chunk histograms, stable counting-sort scatter, block map), shared
// by the multi-chunk launch and the single-chunk decode kernel that fuses it
// with routing.  Device code only; included by build_blocks.hip and
// route.hip.
#pragma once
#include <type_traits>

#include "internal.h"

namespace moe {
namespace {

constexpr int kScanThreads = 512;
constexpr int kScanWaves = kScanThreads / 64;

// Exclusive scan over kScanThreads values held one per thread: a DPP prefix
// sum inside each wave, then each wave adds the totals of the waves before
// it (two barriers).
__device__ int block_exclusive_scan(int v, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int incl = wave_inclusive_sum(v);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; w++) base += tmp[w];
  __syncthreads();  // tmp is reused by the next scan
  return base + incl - v;
}

// One workgroup of kScanThreads threads, chunk c of nchunks: see
// build_blocks.hip for the algorithm.  With chunk_start (nchunks x E, the
// first slot of chunk c's pairs of expert e, computed elsewhere) only the
// scatter runs: no sums, no scan, no block map.
__device__ __forceinline__ void scan_scatter_chunk(
    const int32_t* __restrict__ ids, int P, int E, int chunk_pairs, int nchunks,
    const int32_t* __restrict__ chunk_hist, int block_m, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_slot, int32_t* __restrict__ blocks, int32_t* __restrict__ num_blocks,
    int c, const int32_t* __restrict__ chunk_start = nullptr) {
  __shared__ int tmp[kScanThreads];
  __shared__ int spre[kScanThreads], stot[kScanThreads];
  __shared__ int wnext[kScanWaves][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = tid;
  // The chunk's pairs, one contiguous segment per wave, read first: their
  // loads and the histogram loads below share one round trip, and the
  // counting and ranking passes both use the ids held in registers (the
  // first kIdRounds rounds of 64; longer segments read the rest in place).
  constexpr int kIdRounds = 4;
  const int p0 = c * chunk_pairs;
  const int p1 = min(P, p0 + chunk_pairs);
  const int q = (((p1 - p0) + 64 * kScanWaves - 1) / (64 * kScanWaves)) * 64;
  const int w0 = min(p1, p0 + wave * q), w1 = min(p1, w0 + q);
  int idr[kIdRounds];
#pragma unroll
  for (int r = 0; r < kIdRounds; r++) {
    const int p = w0 + 64 * r + lane;
    idr[r] = p < w1 ? ids[p] : -1;
  }
  int first = 0;  // first slot of this chunk's pairs of expert e
  if (chunk_start) {
    if (e < E) first = chunk_start[(size_t)c * E + e];
  } else {
  // ---- per expert: histogram rows of the chunks before this one, and of
  // all chunks.  Thread (g, e) sums chunks g, g + G, ...; the U loads of a
  // batch are issued together (indexes clamped, so no load sits behind a
  // branch), U the smallest of 8, 16, 32, 64 that covers every chunk in one
  // batch (batches of 64 beyond).
  {
    const int G = kScanThreads / E;
    const int e = tid % E, g = tid / E;
    int pre = 0, tot = 0;
    auto sums = [&](auto utag) {
      constexpr int U = decltype(utag)::value;
      for (int cc0 = g; cc0 < nchunks; cc0 += G * U) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; u++) v[u] = chunk_hist[(size_t)min(cc0 + u * G, nchunks - 1) * E + e];
#pragma unroll
        for (int u = 0; u < U; u++) {
          const int cc = cc0 + u * G;
          tot += cc < nchunks ? v[u] : 0;
          pre += cc < c ? v[u] : 0;
        }
      }
    };
    if (g < G) {
      if (nchunks <= 8 * G) sums(std::integral_constant<int, 8>{});
      else if (nchunks <= 16 * G) sums(std::integral_constant<int, 16>{});
      else if (nchunks <= 32 * G) sums(std::integral_constant<int, 32>{});
      else sums(std::integral_constant<int, 64>{});
    }
    spre[tid] = pre;
    stot[tid] = tot;
  }
  __syncthreads();
  int pre = 0, tot = 0;
  if (e < E) {
    const int G = kScanThreads / E;
    for (int g = 0; g < G; g++) {
      pre += spre[g * E + e];
      tot += stot[g * E + e];
    }
  }
  const int off = block_exclusive_scan(tot, tmp);

  if (c == 0) {
    const int tiles = (tot + block_m - 1) / block_m;
    const int tile0 = block_exclusive_scan(tiles, tmp);
    if (e < E) {
      counts[e] = tot;
      offsets[e] = off;
      for (int i = 0; i < tiles; i++) {
        int32_t* b = blocks + 3 * (size_t)(tile0 + i);
        b[0] = e;
        b[1] = off + i * block_m;
        b[2] = min(block_m, tot - i * block_m);
      }
    }
    if (e == E - 1) {
      offsets[E] = P;
      num_blocks[0] = tile0 + tiles;
    }
  }
  first = off + pre;
  }

  // ---- the chunk's pairs: counts per wave, then ranks
  for (int i = lane; i < E; i += 64) wnext[wave][i] = 0;
  __syncthreads();
  auto count = [&](int p, int id) {
    if (p < w1 && id >= 0 && id < E) atomicAdd(&wnext[wave][id], 1);
  };
#pragma unroll
  for (int r = 0; r < kIdRounds; r++)
    if (w0 + 64 * r < w1) count(w0 + 64 * r + lane, idr[r]);  // (uniform test)
  for (int p = w0 + 64 * kIdRounds + lane; p - lane < w1; p += 64) count(p, p < w1 ? ids[p] : -1);
  __syncthreads();
  if (e < E) {
    int run = first;
#pragma unroll
    for (int w = 0; w < kScanWaves; w++) {
      const int n = wnext[w][e];
      wnext[w][e] = run;
      run += n;
    }
  }
  __syncthreads();

  int bits = 1;
  while ((1 << bits) < E) bits++;
  int* next = wnext[wave];
  auto rank = [&](int p, int id) {
    const bool active = p < w1 && id >= 0 && id < E;
    const int ex = active ? id : 0;
    uint64_t match = __ballot(active);
    for (int b = 0; b < bits; b++) {
      const bool bit = (ex >> b) & 1;
      const uint64_t bal = __ballot(bit);
      match &= bit ? bal : ~bal;
    }
    const uint64_t below = match & ((1ull << lane) - 1ull);
    const int rk = __popcll(below);
    const int start = active ? next[ex] : 0;
    wave_lds_sync();
    if (active) {
      const int slot = start + rk;
      sorted_pairs[slot] = p;
      pair_slot[p] = slot;
      if (below == 0) next[ex] = start + __popcll(match);  // lowest lane of its group
    }
    wave_lds_sync();
  };
#pragma unroll
  for (int r = 0; r < kIdRounds; r++)
    if (w0 + 64 * r < w1) rank(w0 + 64 * r + lane, idr[r]);  // (uniform test)
  for (int p = w0 + 64 * kIdRounds + lane; p - lane < w1; p += 64) rank(p, p < w1 ? ids[p] : -1);
}


}  // namespace
}  // namespace moe
