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
// Packed scales and biases: uint32 [E][N/128][K/G][128 columns] (512
// contiguous bytes per chunk and group), then a tail of two words per expert.
// Each expert's scales and biases are first multiplied by one power of two
// 2^c (exact) chosen so that |bias| + 32 |scale| of every group falls below
// 2^14: every fp16 quantity of the dequantisation is then a normal fp16
// number far from overflow, whatever the range of the caller's values.  The
// kernels multiply their fp32 sums by 2^-c (exact) before using them.  A
// word holds the scale s' = 2^c s as fp16 in the low half and, in the high
// half, either
//  - the offset b' - 32 s' (b' = 2^c bias), when it is exactly an fp16 value
//    for every group of the expert (the case bias = -8 scale and many
//    others): the dequantisation is one fused multiply-add, exact rounding
//    of q s' + b' ("exact" experts), or
//  - b' itself otherwise ("general" experts): the kernels form q s' with one
//    rounding and add b' with a second.
// Tail (after the E * N * K/G words): float unscale[E] = 2^-c, then uint32
// general[E] (1 for a general expert), padded to 16 bytes.
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

// One workgroup per expert: the power of two 2^c that puts the largest
// |bias| + 32 |scale| of the expert's groups in [2^13, 2^14) (c = 0 for an
// all-zero expert; |c| <= 100), and whether every group's offset
// b' - 32 s' is an fp16 value.  tail: unscale[E] then general[E].
__global__ __launch_bounds__(256) void pack_exp_kernel(const uint16_t* __restrict__ sc,
                                                       const uint16_t* __restrict__ bi,
                                                       uint32_t* __restrict__ tail, int64_t per_e,
                                                       int E) {
  __shared__ float red[256];
  __shared__ int bad[1];
  const int e = blockIdx.x, tid = threadIdx.x;
  const uint16_t* s16 = sc + (size_t)e * per_e;
  const uint16_t* b16 = bi + (size_t)e * per_e;
  float m = 0.0f;
  for (int64_t i = tid; i < per_e; i += 256)
    m = fmaxf(m, fabsf(__uint_as_float((uint32_t)b16[i] << 16)) +
                     32.0f * fabsf(__uint_as_float((uint32_t)s16[i] << 16)));
  red[tid] = m;
  if (tid == 0) bad[0] = 0;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  int c = 0;
  if (red[0] > 0.0f && red[0] <= 3.0e38f) {
    int ex;
    frexpf(red[0], &ex);  // red[0] in [2^(ex-1), 2^ex)
    c = min(100, max(-100, 14 - ex));
  }
  // is b' - 32 s' exact in fp16 for every group (computed exactly in fp64)?
  int inexact = 0;
  for (int64_t i = tid; i < per_e; i += 256) {
    const double s = ldexp((double)__uint_as_float((uint32_t)s16[i] << 16), c);
    const double b = ldexp((double)__uint_as_float((uint32_t)b16[i] << 16), c);
    const double off = b - 32.0 * s;
    if ((double)(half_t)off != off) inexact = 1;
  }
  if (inexact) atomicOr(bad, 1);
  __syncthreads();
  if (tid == 0) {
    reinterpret_cast<float*>(tail)[e] = ldexpf(1.0f, -c);
    tail[E + e] = bad[0] ? 1u : 0u;
  }
  // the tail's padding to 16 bytes
  if (e == 0 && tid < ((2 * E + 3) & ~3) - 2 * E) tail[2 * E + tid] = 0u;
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint16_t* __restrict__ sc,
                                                          const uint16_t* __restrict__ bi,
                                                          uint32_t* __restrict__ out, int64_t n,
                                                          int gpr, int64_t per_e,
                                                          const uint32_t* __restrict__ tail, int E) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // i = ((e * N/128 + c) * gpr + g) * 128 + cc
  const int cc = (int)(i & 127);
  const int64_t rest = i >> 7;
  const int g = (int)(rest % gpr);
  const int64_t ec = rest / gpr;
  const int64_t src = (ec * 128 + cc) * gpr + g;
  const int e = (int)(src / per_e);
  const float up = 1.0f / reinterpret_cast<const float*>(tail)[e];  // 2^c, exact
  const float s = __uint_as_float((uint32_t)sc[src] << 16) * up;
  const float b = __uint_as_float((uint32_t)bi[src] << 16) * up;
  const half_t hs = (half_t)s, hb = tail[E + e] ? (half_t)b : (half_t)(b - 32.0f * s);
  out[i] = (uint32_t)__builtin_bit_cast(uint16_t, hs) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// One thread per 16-byte unit of packed codes (the 4 words of one column and
// reduction half in one slab): the same dequantisation as the GEMMs (the
// expert's exact or general form), written as 4 x 16 bytes of fp16 (the
// weights times the expert's 2^c, as the GEMMs form them).
__global__ __launch_bounds__(256) void expand_kernel(const uint32_t* __restrict__ words,
                                                     const uint32_t* __restrict__ sb,
                                                     uint32_t* __restrict__ out, int64_t units,
                                                     int slabs, int gpr, int log2G, int chunks_per_e,
                                                     const uint32_t* __restrict__ general) {
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
  const SbPair sp = sb_unpack(sb[(ec * gpr + g) * 128 + blk * 32 + col], general[ec / chunks_per_e] != 0);
  uint4* o = reinterpret_cast<uint4*>(out) + (rest * 4 + blk) * 256 + ch;
#pragma unroll
  for (int i = 0; i < 4; i++) o[64 * i] = dequant_word_any(q[i], sp);
}

}  // namespace

hipError_t launch_expand(const moe_w4_packed& bank, int E, int N, int K, int G, uint32_t* out,
                         hipStream_t s) {
  const int64_t units = (int64_t)E * N * K / 32;  // 16-byte units of codes
  const int log2G = G == 32 ? 5 : G == 64 ? 6 : 7;
  const BankTail t = bank_tail(bank, E, N, K, G);
  expand_kernel<<<(units + 255) / 256, 256, 0, s>>>(bank.words, bank.sb, out, units, K / 64, K / G,
                                                    log2G, N / 128, t.general);
  return hipGetLastError();
}

hipError_t launch_pack(const moe_w4_bank& src, int E, int N, int K, int G, uint32_t* words,
                       uint32_t* sb, hipStream_t s) {
  const int64_t nwords = (int64_t)E * N * K / 8;
  pack_codes_kernel<<<(nwords + 255) / 256, 256, 0, s>>>(src.qweight, words, nwords, N, K);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t nsb = (int64_t)E * N * (K / G);
  uint32_t* tail = sb + nsb;
  pack_exp_kernel<<<E, 256, 0, s>>>(src.scales, src.biases, tail, (int64_t)N * (K / G), E);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  pack_scales_kernel<<<(nsb + 255) / 256, 256, 0, s>>>(src.scales, src.biases, sb, nsb, K / G,
                                                       (int64_t)N * (K / G), tail, E);
  return hipGetLastError();
}

}  // namespace moe
