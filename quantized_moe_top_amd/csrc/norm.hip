// norm.hip -- the step in front of the layer: RMSNorm of the activations,
//   x_n[t][h] = bf16(x[t][h] * gamma[h] / sqrt(mean_h x[t][h]^2 + eps)),
// whose bf16 output then feeds the router and the experts as x does.  The
// pages describe only the MoE layer; this is the textbook normalisation an
// engine runs before it, so that the layer drops into a decoder block.
//
// One wave per row: the lanes sum the squares of their 16-byte pieces in
// fp32, a butterfly adds the 64 partial sums (every lane gets the same total:
// each step adds the same two values), then each lane scales its pieces
// (x * r, then * gamma, in fp32) and rounds them to bf16, nearest even.  The
// row is read twice (the second pass from the cache).
#include "internal.h"

namespace moe {
namespace {

constexpr int kNormRows = 4;  // rows (waves) per workgroup

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(64 * kNormRows) void rmsnorm_kernel(const uint4* __restrict__ x,
                                                                const uint4* __restrict__ gamma,
                                                                float eps, int T, int H8,
                                                                uint4* __restrict__ out) {
  const int row = blockIdx.x * kNormRows + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= T) return;
  const uint4* xr = x + (size_t)row * H8;
  float ss = 0.0f;
  for (int c = lane; c < H8; c += 64) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float a = bf_lo(w[i]), b = bf_hi(w[i]);
      ss += a * a;
      ss += b * b;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const float r = 1.0f / sqrtf(ss / (float)(8 * H8) + eps);
  uint4* orow = out + (size_t)row * H8;
  for (int c = lane; c < H8; c += 64) {
    const uint4 v = xr[c], g = gamma[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
      o[i] = f32_to_bf16_rne(bf_lo(w[i]) * r * bf_lo(gw[i])) |
             (f32_to_bf16_rne(bf_hi(w[i]) * r * bf_hi(gw[i])) << 16);
    orow[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int T, int H,
                          uint16_t* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int grid = (T + kNormRows - 1) / kNormRows;
  rmsnorm_kernel<<<grid, 64 * kNormRows, 0, s>>>(reinterpret_cast<const uint4*>(x),
                                                 reinterpret_cast<const uint4*>(gamma), eps, T,
                                                 H / 8, reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace moe
