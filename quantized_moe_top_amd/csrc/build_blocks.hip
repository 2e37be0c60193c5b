// build_blocks.hip -- S2 expert histogram, S3 prefix scan, S4 stable scatter
// and S5 tile block map, on the device with no host round trip (page
// "Perplexity's Lily engine beats MLX by 35% on M5 Max", architecture
// paragraph: routing, prefix scan, scatter and block map stay inside one GPU
// submission).
//
// The pairs p = t * k + j are cut into chunks of chunk_tokens * k pairs, the
// same chunks the routing kernel histograms.  Given every chunk's histogram,
// one launch finishes the job, one workgroup per chunk:
//   - each workgroup sums the histogram rows (per expert: the chunks before
//     its own, and all of them) and takes an LDS exclusive scan over experts:
//     offsets, and the first slot of each (chunk, expert) run;
//   - workgroup 0 also writes counts, offsets and the block map;
//   - the chunk's pairs are split over the 8 waves in contiguous segments;
//     per-wave histograms give each wave its first slot per expert; each wave
//     then ranks its pairs 64 at a time: lanes with the same expert are found
//     with ballots over the expert-id bits, a lane's rank is the number of
//     such lanes below it, so slots follow pair order (a stable counting
//     sort, deterministic).
// moe_build_blocks, which receives the ids from the caller, runs a small
// histogram kernel first.
#include "scan_scatter.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void chunk_hist_kernel(const int32_t* __restrict__ ids, int P,
                                                         int E, int chunk_pairs,
                                                         int32_t* __restrict__ chunk_hist) {
  __shared__ int h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * chunk_pairs;
  const int p1 = min(P, p0 + chunk_pairs);
  for (int p = p0 + tid; p < p1; p += 256) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);  // ids outside [0, E) are ignored
  }
  __syncthreads();
  if (tid < E) chunk_hist[(size_t)blockIdx.x * E + tid] = h[tid];
}

__global__ __launch_bounds__(kScanThreads) void scan_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, int chunk_pairs, int nchunks,
    const int32_t* __restrict__ chunk_hist, int block_m, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_slot, int32_t* __restrict__ blocks, int32_t* __restrict__ num_blocks,
    const int32_t* __restrict__ chunk_start, int32_t* __restrict__ tflags, int nflags) {
  // the per-tile flags the gate/up kernel sets start cleared
  for (int i = blockIdx.x * kScanThreads + threadIdx.x; i < nflags; i += gridDim.x * kScanThreads)
    tflags[i] = 0;
  scan_scatter_chunk(ids, P, E, chunk_pairs, nchunks, chunk_hist, block_m, counts, offsets,
                     sorted_pairs, pair_slot, blocks, num_blocks, blockIdx.x, chunk_start);
}

}  // namespace

hipError_t launch_chunk_hist(const int32_t* ids, int T, int k, int E, int32_t* chunk_hist,
                             hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int chunk_pairs = route_chunk_tokens(T) * k;
  chunk_hist_kernel<<<route_chunks(T), 256, 0, s>>>(ids, T * k, E, chunk_pairs, chunk_hist);
  return hipGetLastError();
}

hipError_t launch_scan_scatter(const int32_t* ids, int T, int k, int E, const int32_t* chunk_hist,
                               int block_m, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_pairs, int32_t* pair_slot, int32_t* blocks,
                               int32_t* num_blocks, hipStream_t s, const int32_t* chunk_start,
                               int32_t* tflags, int64_t nflags) {
  if (T <= 0) return hipSuccess;
  const int chunk_pairs = route_chunk_tokens(T) * k;
  const int n = route_chunks(T);
  scan_scatter_kernel<<<n, kScanThreads, 0, s>>>(ids, T * k, E, chunk_pairs, n, chunk_hist, block_m, counts,
                                        offsets, sorted_pairs, pair_slot, blocks, num_blocks,
                                        chunk_start, tflags, tflags ? (int)nflags : 0);
  return hipGetLastError();
}

}  // namespace moe
