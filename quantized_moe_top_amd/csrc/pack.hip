// pack.hip -- one-time repack of a W4 bank from the caller's row-major
// layout into the tile-major layout the grouped GEMM and GEMV kernels stream
// (page "Perplexity's Lily beats MLX by 1.35x by doing one thing:
// single-model Rust/Metal engines", section "Why one model on one chip is
// faster": a single-model engine lays out its weights in whatever order its
// kernels read fastest).
//
// Packed codes: uint32 words [E][N/32][K/64][32 columns][2 halves][4 words].
// The 1 KiB block (e, column block b, slab s) holds, for column c = 32b + cc
// and half h, the four words of codes k = 64s + 32h + 8w + j (word w, nibble
// j, lowest nibble first, as in the row-major words): one 16-byte load per
// lane per slab, and one contiguous 1 KiB block per 32 columns per slab.
// Packed scales and biases: uint32 [E][N/32][K/G][32 columns], the bf16
// scale in the low half and the bf16 bias in the high half, so that the 32
// columns of a block need 128 contiguous bytes per group.
#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint32_t* __restrict__ q,
                                                         uint32_t* __restrict__ out, int64_t nwords,
                                                         int N, int K) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nwords) return;
  // i = (((e * N/32 + b) * K/64 + s) * 32 + cc) * 8 + h * 4 + w
  const int w = (int)(i & 3), h = (int)((i >> 2) & 1), cc = (int)((i >> 3) & 31);
  const int64_t rest = i >> 8;  // (e * N/32 + b) * K/64 + s
  const int slabs = K / 64;
  const int s = (int)(rest % slabs);
  const int64_t eb = rest / slabs;  // e * N/32 + b
  const int64_t row = eb * 32 + cc;  // e * N + n
  out[i] = q[row * (K / 8) + s * 8 + h * 4 + w];
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint16_t* __restrict__ sc,
                                                          const uint16_t* __restrict__ bi,
                                                          uint32_t* __restrict__ out, int64_t n,
                                                          int gpr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // i = ((e * N/32 + b) * gpr + g) * 32 + cc
  const int cc = (int)(i & 31);
  const int64_t rest = i >> 5;
  const int g = (int)(rest % gpr);
  const int64_t eb = rest / gpr;
  const int64_t src = (eb * 32 + cc) * gpr + g;
  out[i] = (uint32_t)sc[src] | ((uint32_t)bi[src] << 16);
}

}  // namespace

hipError_t launch_pack(const moe_w4_bank& src, int E, int N, int K, int G, uint32_t* words,
                       uint32_t* sb, hipStream_t s) {
  const int64_t nwords = (int64_t)E * N * K / 8;
  pack_codes_kernel<<<(nwords + 255) / 256, 256, 0, s>>>(src.qweight, words, nwords, N, K);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t nsb = (int64_t)E * N * (K / G);
  pack_scales_kernel<<<(nsb + 255) / 256, 256, 0, s>>>(src.scales, src.biases, sb, nsb, K / G);
  return hipGetLastError();
}

}  // namespace moe
