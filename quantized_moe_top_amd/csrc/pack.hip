// pack.hip -- one-time repack of a W4 bank from the caller's row-major
// layout into the tile-major layout the grouped GEMM and GEMV kernels stream
// (page "Perplexity's Lily beats MLX by 1.35x by doing one thing:
// single-model Rust/Metal engines", section "Why one model on one chip is
// faster": a single-model engine lays out its weights in whatever order its
// kernels read fastest).
//
// Packed codes: uint32 words [E][N/128][K/64][4 blocks][32 columns]
// [2 halves][4 words].  For 128-column chunk c, slab s, 32-column block u of
// the chunk, column cc of the block and half h, the four words hold codes
// k = 64s + 32h + 8w + j of column 128c + 32u + cc (word w, nibble j, lowest
// nibble first, as in the row-major words), each word rotated left by 5 bits
// so that the dequantisation extracts two codes per instruction straight
// into the mantissa of 32.0h.  A 32-column block of one slab is 1 KiB (one
// 16-byte load per lane), and the 128 columns of a chunk are one contiguous
// 4 KiB run per slab: DRAM streams in long runs.
// Packed scales and biases: uint32 [E][N/128][K/G][128 columns], the scale
// as fp16 in the low half and bias - 32 * scale as fp16 in the high half
// (both rounded to nearest once, here): 512 contiguous bytes per chunk and
// group.
#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint32_t* __restrict__ q,
                                                         uint32_t* __restrict__ out, int64_t nwords,
                                                         int N, int K) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nwords) return;
  // i = ((((e * N/128 + c) * K/64 + s) * 4 + u) * 32 + cc) * 8 + h * 4 + w
  const int w = (int)(i & 3), h = (int)((i >> 2) & 1), cc = (int)((i >> 3) & 31);
  const int u = (int)((i >> 8) & 3);
  const int64_t rest = i >> 10;  // (e * N/128 + c) * K/64 + s
  const int slabs = K / 64;
  const int s = (int)(rest % slabs);
  const int64_t ec = rest / slabs;  // e * N/128 + c
  const int64_t row = ec * 128 + u * 32 + cc;  // e * N + n
  const uint32_t v = q[row * (K / 8) + s * 8 + h * 4 + w];
  out[i] = (v << 5) | (v >> 27);
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint16_t* __restrict__ sc,
                                                          const uint16_t* __restrict__ bi,
                                                          uint32_t* __restrict__ out, int64_t n,
                                                          int gpr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // i = ((e * N/128 + c) * gpr + g) * 128 + cc
  const int cc = (int)(i & 127);
  const int64_t rest = i >> 7;
  const int g = (int)(rest % gpr);
  const int64_t ec = rest / gpr;
  const int64_t src = (ec * 128 + cc) * gpr + g;
  const float s = __uint_as_float((uint32_t)sc[src] << 16);
  const float b = __uint_as_float((uint32_t)bi[src] << 16);
  const half_t hs = (half_t)s, hb = (half_t)(b - 32.0f * s);
  out[i] = (uint32_t)__builtin_bit_cast(uint16_t, hs) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// One thread per 16-byte unit of packed codes (the 4 words of one column and
// reduction half in one slab): the same exact dequantisation as the GEMMs,
// written as 4 x 16 bytes of fp16.
__global__ __launch_bounds__(256) void expand_kernel(const uint32_t* __restrict__ words,
                                                     const uint32_t* __restrict__ sb,
                                                     uint32_t* __restrict__ out, int64_t units,
                                                     int slabs, int gpr, int log2G) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  // u = ((ec * slabs + s) * 4 + blk) * 64 + 2 col + h, ec = e * N/128 + chunk
  const int ch = (int)(u & 63), blk = (int)((u >> 6) & 3);
  const int64_t rest = u >> 8;
  const int s = (int)(rest % slabs);
  const int64_t ec = rest / slabs;
  const int col = ch >> 1, h = ch & 1;
  const u32x4 q = reinterpret_cast<const u32x4*>(words)[u];
  const int g = (64 * s + 32 * h) >> log2G;
  half2_t s2, b2;
  sb_pairs(sb[(ec * gpr + g) * 128 + blk * 32 + col], s2, b2);
  uint4* o = reinterpret_cast<uint4*>(out) + (rest * 4 + blk) * 256 + ch;
#pragma unroll
  for (int i = 0; i < 4; i++) o[64 * i] = dequant_word(q[i], s2, b2);
}

}  // namespace

hipError_t launch_expand(const moe_w4_packed& bank, int E, int N, int K, int G, uint32_t* out,
                         hipStream_t s) {
  const int64_t units = (int64_t)E * N * K / 32;  // 16-byte units of codes
  const int log2G = G == 32 ? 5 : G == 64 ? 6 : 7;
  expand_kernel<<<(units + 255) / 256, 256, 0, s>>>(bank.words, bank.sb, out, units, K / 64, K / G,
                                                    log2G);
  return hipGetLastError();
}

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
