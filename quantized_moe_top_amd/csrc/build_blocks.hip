// build_blocks.hip -- S2 expert histogram, S3 prefix scan, S4 stable scatter
// and S5 tile block map, all on the device (page "Perplexity's Lily engine
// beats MLX by 35% on M5 Max", architecture paragraph: routing, prefix scan,
// scatter and block map stay inside one GPU submission).
//
// The P pairs are cut into chunks of kChunkPairs.  Three launches on one
// stream, no host round trip:
//   1. hist:    one wave per chunk counts the chunk's pairs per expert
//               (LDS atomics; counts do not depend on order).
//   2. scan:    one workgroup: per expert, an exclusive running sum over the
//               chunks gives each chunk's first slot relative to the expert;
//               an LDS exclusive scan over experts gives offsets; then the
//               tiles of each expert are written and counted.
//   3. scatter: one wave per chunk walks its pairs in order, 64 at a time.
//               Lanes holding the same expert are found with ballots over
//               the expert id bits; a lane's rank is the number of such lanes
//               below it (mbcnt), so slots follow pair order: the counting
//               sort is stable and deterministic.
#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(64) void hist_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                  int32_t* __restrict__ chunk_hist) {
  __shared__ int32_t h[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) h[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kChunkPairs;
  const int p1 = min(P, p0 + kChunkPairs);
  for (int p = p0 + lane; p < p1; p += 64) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);  // ids outside [0, E) are ignored
  }
  __syncthreads();
  for (int e = lane; e < E; e += 64) chunk_hist[(size_t)blockIdx.x * E + e] = h[e];
}

// Exclusive scan over up to 256 values held one per thread (blockDim 256).
__device__ int block_exclusive_scan(int v, int* tmp) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  const int incl = tmp[tid];
  __syncthreads();
  return incl - v;
}

// One workgroup of 256 threads; thread e owns expert e.
// chunk_base is chunk_hist, rewritten in place to the first slot of each
// (chunk, expert) run.
__global__ __launch_bounds__(256) void scan_kernel(int32_t* __restrict__ chunk_base, int nchunks,
                                                   int P, int E, int block_m,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ blocks,
                                                   int32_t* __restrict__ num_blocks) {
  __shared__ int tmp[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; c++) {
      int32_t* cell = chunk_base + (size_t)c * E + e;
      const int n = *cell;
      *cell = run;
      run += n;
    }
  }
  const int count = e < E ? run : 0;
  const int off = block_exclusive_scan(count, tmp);
  const int tiles = (count + block_m - 1) / block_m;
  const int tile0 = block_exclusive_scan(tiles, tmp);
  if (e < E) {
    counts[e] = count;
    offsets[e] = off;
    for (int c = 0; c < nchunks; c++) chunk_base[(size_t)c * E + e] += off;
    for (int i = 0; i < tiles; i++) {
      int32_t* b = blocks + 3 * (size_t)(tile0 + i);
      b[0] = e;
      b[1] = off + i * block_m;
      b[2] = min(block_m, count - i * block_m);
    }
  }
  if (e == E - 1) {
    offsets[E] = P;
    num_blocks[0] = tile0 + tiles;
  }
}

__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                     const int32_t* __restrict__ chunk_base,
                                                     int32_t* __restrict__ sorted_pairs,
                                                     int32_t* __restrict__ pair_slot) {
  __shared__ int32_t next[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) next[e] = chunk_base[(size_t)blockIdx.x * E + e];
  __syncthreads();
  int bits = 1;
  while ((1 << bits) < E) bits++;
  const int p0 = blockIdx.x * kChunkPairs;
  const int p1 = min(P, p0 + kChunkPairs);
  for (int base = p0; base < p1; base += 64) {
    const int p = base + lane;
    const int id = p < p1 ? ids[p] : -1;
    const bool active = id >= 0 && id < E;
    const int e = active ? id : 0;
    uint64_t match = __ballot(active);
    for (int b = 0; b < bits; b++) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      match &= bit ? bal : ~bal;
    }
    const uint64_t below = match & ((1ull << lane) - 1ull);
    const int rank = __popcll(below);
    const int start = active ? next[e] : 0;
    __builtin_amdgcn_wave_barrier();
    if (active) {
      const int slot = start + rank;
      sorted_pairs[slot] = p;
      pair_slot[p] = slot;
      if (below == 0) next[e] = start + __popcll(match);  // lowest lane of its group
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  }
}

}  // namespace

int build_blocks_chunks(int64_t P) { return (int)((P + kChunkPairs - 1) / kChunkPairs); }

hipError_t launch_build_blocks(const int32_t* ids, int P, int E, int block_m, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_slot,
                               int32_t* blocks, int32_t* num_blocks, int32_t* scratch,
                               hipStream_t s) {
  const int nchunks = build_blocks_chunks(P);
  hist_kernel<<<nchunks, 64, 0, s>>>(ids, P, E, scratch);
  scan_kernel<<<1, 256, 0, s>>>(scratch, nchunks, P, E, block_m, counts, offsets, blocks,
                                num_blocks);
  scatter_kernel<<<nchunks, 64, 0, s>>>(ids, P, E, scratch, sorted_pairs, pair_slot);
  return hipGetLastError();
}

}  // namespace moe
