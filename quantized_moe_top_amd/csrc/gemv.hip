// gemv.hip -- S9: the grouped W4 GEMM at decode sizes (T <= 8).  With at most
// 8 rows per expert the product is bound by reading the packed weights, so
// each touched expert's weights are streamed once, with as many bytes in
// flight as the chip holds, and experts that no token chose are never read.
//
// One workgroup per (tile, 32-column output block): S6 reads the gate and
// the up block, S7 the down block.  The reduction dimension is split over
// the waves, two or four 64-wide slabs per wave and pass (16 or 8 waves
// cover K = 2048 in one pass; with four, two workgroups share a CU, so one
// computes while the other waits on memory), and every wave issues the
// weight loads of its pass at once, straight into registers: the packed codes (one 1 KiB block per bank and
// slab; lane l takes the 32 codes of column l % 32, reduction half l / 32,
// exactly an MFMA B fragment after dequantisation), the (scale, bias) words
// and the activation rows.  The dot products run on v_mfma_f32_32x32x16_f16
// with the tile's rows (<= 8) in MFMA rows 0..7 and zeros above, so the VALU
// only dequantises (same exact fp16 dequantisation as the prefill path).
// The waves' partial sums meet in LDS and are added in wave order, so the
// result does not depend on timing.
#include <type_traits>

#include "internal.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kDecWavesMax = 16;

struct DecParams {
  const half_t* a;
  moe_w4_packed b0, b1;
  const int32_t* sorted_pairs;
  const float* topk_weights;
  const int32_t* blocks;
  const int32_t* num_blocks;
  void* out;
  BankTail t0, t1;  // per-expert 2^-c and dequantisation form of b0 / b1
  int8_t* hexp;     // h's exponents [P][I / 16] (h_block_exp): written by S6, read by S7
  int32_t* tflags;  // per tile: a row has a nonzero exponent (written by S6 when given)
  int N, K, log2_G, top_k, E, P, max_blocks;
  int red_off;     // byte offset of the partial-sum area in the dynamic LDS
  int lg_off = 0;  // fused decode gate/up: byte offset of the logits in the dynamic LDS
  bool x_res = false;  // fused decode gate/up: every x row resident in LDS ([T][K] at 0)
  // fused decode gate/up with x_res: RMSNorm of the x rows in front (bf16
  // [K], or nullptr), 1 / sqrt(mean x^2 + eps)
  const uint16_t* gamma = nullptr;
  float eps = 0.0f;
};

// One (tile, 32-column block) of the product: tile rows [row0, row0 + rows)
// of expert e (rows <= kGemvMaxTokens), output columns [32 blk, 32 blk + 32).
// SPW: 64-wide slabs per wave and pass.
// sorted_pairs: slot -> pair (global memory, or LDS in the fused kernel).
// dsm: the dynamic LDS, sized by the launch.
// GEN: the expert takes the general dequantisation (dequant_word_gen).
template <int MODE, int SPW, bool GEN>
__device__ __forceinline__ void gemv_tile(const DecParams& p, const int32_t* sorted_pairs, int e,
                                          int row0, int rows, int blk, char* dsm) {
  constexpr bool GATE_UP = MODE == MOE_GEMM_GATE_UP_SWIGLU;
  constexpr int NB = GATE_UP ? 2 : 1;  // banks read: gate and up, or down
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = blockDim.x >> 6;
  const int pass_slabs = nwaves * SPW;  // slabs per pass
  const int xw = pass_slabs * 64;       // row stride of xs
  // LDS: xs = this pass's activation rows (<= 8 rows x xw reduction
  // indices, operand order), staged once for all waves; red (at red_off) =
  // rows 0..7 of each wave's 32x32 partial (register r < 4 of lane l holds
  // row 4 (l / 32) + r, column l % 32), [wave][bank][r][lane]
  half_t* xs = reinterpret_cast<half_t*>(dsm);
  float* red = reinterpret_cast<float*>(dsm + p.red_off);
  const int col = lane & 31, khalf = lane >> 5;
  const int nbl = p.N / 32;
  const int K = p.K, S = K / 64, gpr = K >> p.log2_G;

  // packed block of this output block in each bank (chunked layout: 4 KiB
  // runs of 128 columns per slab)
  const size_t bidx = (size_t)e * nbl + blk;
  const uint32_t* wsrc[NB];
  const uint32_t* ssrc[NB];
#pragma unroll
  for (int b = 0; b < NB; b++) {
    const moe_w4_packed& bank = b == 0 ? p.b0 : p.b1;
    // 16-byte unit (column, half) of a block is number 2 * column + half
    wsrc[b] = bank.words + ((bidx >> 2) * S * 4 + (bidx & 3)) * 256 + 4 * (2 * col + khalf);
    ssrc[b] = bank.sb + (bidx >> 2) * gpr * 128 + (bidx & 3) * 32 + col;
  }

  // the expert's factors 2^-c
  const float us0 = p.t0.unscale[e], us1 = GATE_UP ? p.t1.unscale[e] : 1.0f;
  // S7: each h row's largest exponent; its blocks are brought to it while
  // staged, and the row's output is scaled by 2^it
  __shared__ int em_s[kGemvMaxTokens];
  if (!GATE_UP) {
    if (tid < rows) {
      const uint32_t* er = reinterpret_cast<const uint32_t*>(p.hexp + (size_t)(row0 + tid) * (K / 16));
      int m = -128;
      for (int b = 0; b < K / 64; b++) m = max(m, max_i8x4(er[b]));
      em_s[tid] = m;
    }
    __syncthreads();
  }
  floatx16_t acc[NB];
#pragma unroll
  for (int b = 0; b < NB; b++) acc[b] = floatx16_t{};
  for (int base = 0; base < S; base += pass_slabs) {
    // 1. this wave's codes and (scale, bias) words for the pass (slabs past
    //    the end reload the last slab and are not multiplied)
    u32x4 q[NB][SPW];
    uint32_t sb[NB][SPW];
#pragma unroll
    for (int j = 0; j < SPW; j++) {
      const int s = min(base + SPW * wave + j, S - 1);
      const int g = (64 * s + 32 * khalf) >> p.log2_G;
#pragma unroll
      for (int b = 0; b < NB; b++) {
        q[b][j] = *reinterpret_cast<const u32x4*>(wsrc[b] + (size_t)s * 1024);
        sb[b][j] = ssrc[b][(size_t)g * 128];
      }
    }
    // 2. the tile's activation rows for the pass into LDS, 16 bytes per
    //    thread and step: token x rows (S6) or slots of h (S7)
    const int nsl = min(pass_slabs, S - base);
    const int c8n = nsl * 8;  // 16-byte pieces per row
    for (int idx = tid; idx < rows * c8n; idx += blockDim.x) {
      const int m = idx / c8n, c8 = idx % c8n;
      int r = row0 + m;
      if (GATE_UP) {
        const int pair = sorted_pairs[r];
        r = (pair >= 0 && pair < p.P) ? pair / p.top_k : 0;
      }
      if constexpr (GATE_UP)
        *reinterpret_cast<uint4*>(xs + m * xw + 8 * c8) =
            *reinterpret_cast<const uint4*>(p.a + (size_t)r * K + 64 * base + 8 * c8);
      else {
        const uint4 v = *reinterpret_cast<const uint4*>(p.a + (size_t)r * K + 64 * base + 8 * c8);
        const int d = p.hexp[(size_t)r * (K / 16) + (64 * base + 8 * c8) / 16] - em_s[m];
        *reinterpret_cast<uint4*>(xs + m * xw + 8 * c8) = d ? scale_half8(v, d) : v;
      }
    }
    __syncthreads();
    // 3. dequantise and multiply; MFMA rows past the tile are zero
#pragma unroll
    for (int j = 0; j < SPW; j++) {
      const int sl = SPW * wave + j;  // slab within the pass
      if (base + sl >= S) break;      // uniform per wave
      u32x4 x[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        x[i] = col < rows ? *reinterpret_cast<const u32x4*>(xs + col * xw + 64 * sl + 32 * khalf + 8 * i)
                          : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < NB; b++) {
        const SbPair sp = sb_unpack(sb[b][j], GEN);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          uint4 d;
          if constexpr (GEN) d = dequant_word_gen(q[b][j][i], sp.s2, sp.c2, sp.b2);
          else d = dequant_word(q[b][j][i], sp.s2, sp.c2);
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(half8_t, x[i]), __builtin_bit_cast(half8_t, d), acc[b], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the next pass overwrites xs
  }
#pragma unroll
  for (int b = 0; b < NB; b++)
#pragma unroll
    for (int r = 0; r < 4; r++) red[((wave * NB + b) * 4 + r) * 64 + lane] = acc[b][r];
  __syncthreads();
  if constexpr (GATE_UP) {
    // h in fp32 per (row, column), stored as fp16 with one exponent per 16
    // columns (h_block_exp; a row's 32 columns are two 16-lane DPP rows), in
    // operand order (see the MFMA kernel)
    bool any = false;
    for (int t = tid; t < rows * 32; t += blockDim.x) {
      const int m = t >> 5, cc = t & 31;
      const int rr = m & 3, ll = cc + 32 * (m >> 2);
      float v[NB];
#pragma unroll
      for (int b = 0; b < NB; b++) {
        v[b] = red[((0 * NB + b) * 4 + rr) * 64 + ll];
        for (int w2 = 1; w2 < nwaves; w2++) v[b] += red[((w2 * NB + b) * 4 + rr) * 64 + ll];
      }
      const float hv = silu_mul(v[0] * us0, v[NB - 1] * us1);
      const int ex = h_block_exp(row16_max(fabsf(hv)));
      const int n = blk * 32 + cc;
      reinterpret_cast<half_t*>(p.out)[(size_t)(row0 + m) * p.N + (n & ~7) + interleaved_pos(n & 7)] =
          (half_t)ldexpf(hv, -ex);
      if ((cc & 15) == 0) p.hexp[(size_t)(row0 + m) * (p.N / 16) + n / 16] = (int8_t)ex;
      any |= ex != 0;
    }
    if (any && p.tflags) p.tflags[blockIdx.x / (p.N / 32)] = 1;
    return;
  }
  for (int t = tid; t < rows * 32; t += blockDim.x) {
    const int m = t >> 5, cc = t & 31;
    const int rr = m & 3, ll = cc + 32 * (m >> 2);
    float v = red[(0 * 4 + rr) * 64 + ll];
    for (int w2 = 1; w2 < nwaves; w2++) v += red[(w2 * 4 + rr) * 64 + ll];
    const int n = blk * 32 + cc;
    const int pair = sorted_pairs[row0 + m];
    const float wgt = (pair >= 0 && pair < p.P) ? ldexpf(p.topk_weights[pair] * us0, em_s[m]) : 0.0f;
    reinterpret_cast<float*>(p.out)[(size_t)(row0 + m) * p.N + n] = wgt * v;
  }
}

// The gate/up product of one (tile, 16-column block), on
// v_mfma_f32_16x16x32_f16, for the fused decode launch: tile rows [row0,
// row0 + rows) of expert e (rows <= kGemvMaxTokens), output columns
// [16 b16, 16 b16 + 16) of both banks, then h = silu(gate) * up.  Lane l
// takes column l % 16 of the block and the 8-byte half q = (l / 16) % 2 of
// the packed 16-byte unit (column, reduction half (l / 32)): its two words
// feed the two MFMAs of a slab, so MFMA m covers, for lane group (l / 16),
// reduction indices 32 (l / 32) + 16 q + 8 m + [0, 8) of the slab, and the
// activation fragment of tile row l % 16 is read to match (zeros past the
// tile).  SPW slabs per wave and pass; x is staged from bf16 as in
// gemv_tile.  The waves' partials (rows 0..7: lanes 0..31, registers 0..3)
// meet in LDS at red_off and are added in wave order.
// This wave's packed codes (two words per bank and slab) and (scale, bias)
// words for one pass (slabs base + SPW wave + [0, SPW); slabs past the end
// reload the last one and are not multiplied).
template <int SPW>
struct Frag16 {
  uint2 q[2][SPW];
  uint32_t sb[2][SPW];
};

template <int SPW>
__device__ __forceinline__ Frag16<SPW> g16_load(const DecParams& p, int e, int b16, int base) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, lg = lane >> 4, khalf = lg >> 1, qh = lg & 1;
  const int col = 16 * (b16 & 1) + c;  // column within the 32-column packed block
  const int S = p.K / 64, gpr = p.K >> p.log2_G;
  const size_t bidx = (size_t)e * (p.N / 32) + (b16 >> 1);
  Frag16<SPW> f;
#pragma unroll
  for (int b = 0; b < 2; b++) {
    const moe_w4_packed& bank = b == 0 ? p.b0 : p.b1;
    const uint32_t* wsrc = bank.words + ((bidx >> 2) * S * 4 + (bidx & 3)) * 256 + 4 * (2 * col + khalf) + 2 * qh;
    const uint32_t* ssrc = bank.sb + (bidx >> 2) * gpr * 128 + (bidx & 3) * 32 + col;
#pragma unroll
    for (int j = 0; j < SPW; j++) {
      const int s = min(base + SPW * wave + j, S - 1);
      f.q[b][j] = *reinterpret_cast<const uint2*>(wsrc + (size_t)s * 1024);
      f.sb[b][j] = ssrc[(size_t)((64 * s + 32 * khalf) >> p.log2_G) * 128];
    }
  }
  return f;
}

// The tile's x rows for one pass into LDS (bf16 -> fp16 operand order); the
// caller synchronises before they are read.
template <int SPW>
__device__ __forceinline__ void g16_stage(const DecParams& p, const int32_t* sorted_pairs, int row0,
                                          int rows, int base, char* dsm) {
  const int pass_slabs = (blockDim.x >> 6) * SPW, xw = pass_slabs * 64;
  half_t* xs = reinterpret_cast<half_t*>(dsm);
  const int nsl = min(pass_slabs, p.K / 64 - base);
  const int c8n = nsl * 8;
  for (int idx = threadIdx.x; idx < rows * c8n; idx += blockDim.x) {
    const int m = idx / c8n, c8 = idx % c8n;
    const int pair = sorted_pairs[row0 + m];
    const int r = (pair >= 0 && pair < p.P) ? pair / p.top_k : 0;
    *reinterpret_cast<uint4*>(xs + m * xw + 8 * c8) = bf16x8_to_half_interleaved(
        *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.a) + (size_t)r * p.K +
                                        64 * base + 8 * c8));
  }
}

// Dequantise this wave's fragments of one pass and multiply them with the
// staged rows (zeros past the tile) into acc.
template <int SPW, bool GEN>
__device__ __forceinline__ void g16_mma(const DecParams& p, const Frag16<SPW>& f, int rows, int base,
                                        floatx4_t (&acc)[2], const char* dsm) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pass_slabs = (blockDim.x >> 6) * SPW, xw = pass_slabs * 64;
  const half_t* xs = reinterpret_cast<const half_t*>(dsm);
  const int c = lane & 15, lg = lane >> 4, khalf = lg >> 1, qh = lg & 1;
#pragma unroll
  for (int j = 0; j < SPW; j++) {
    const int sl = SPW * wave + j;
    if (base + sl >= p.K / 64) break;  // uniform per wave
    u32x4 x[2];
#pragma unroll
    for (int m = 0; m < 2; m++)
      x[m] = c < rows ? *reinterpret_cast<const u32x4*>(xs + c * xw + 64 * sl + 32 * khalf + 16 * qh + 8 * m)
                      : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 2; b++) {
      const SbPair sp = sb_unpack(f.sb[b][j], GEN);
#pragma unroll
      for (int m = 0; m < 2; m++) {
        const uint32_t w = m == 0 ? f.q[b][j].x : f.q[b][j].y;
        const uint4 d = GEN ? dequant_word_gen(w, sp.s2, sp.c2, sp.b2) : dequant_word(w, sp.s2, sp.c2);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, x[m]),
                                                        __builtin_bit_cast(half8_t, d), acc[b], 0, 0, 0);
      }
    }
  }
}

// The waves' partials (rows 0..7: lanes 0..31, registers 0..3) meet in LDS
// at red_off and are added in wave order; h = silu(gate) * up in operand
// order.  Ends with a barrier (the LDS is reused by the next item).
// COHERENT: h and its exponents are stored with device-scope (write-through)
// stores, so a workgroup of the same launch on another XCD can read them once
// it has seen the tile's ready count (the single-launch decode layer).
// buf >= 0: the partials go to half buf of a doubled area and the epilogue
// ends without a barrier (the caller alternates the halves, so the next
// item's partials never overwrite values still being read, and the item
// after that writes this half only past the next item's barrier); buf < 0:
// one area and a closing barrier.
template <bool COHERENT = false>
__device__ __forceinline__ void g16_epilogue(const DecParams& p, const floatx4_t (&acc)[2], int row0,
                                             int rows, int b16, char* dsm, float us0, float us1,
                                             int buf = -1) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = blockDim.x >> 6;
  float* red = reinterpret_cast<float*>(dsm + p.red_off) + (buf > 0 ? nwaves * 2 * 4 * 32 : 0);
  if (lane < 32)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int i = 0; i < 4; i++) red[((wave * 2 + b) * 4 + i) * 32 + lane] = acc[b][i];
  __syncthreads();
  // h in fp32 per (row, column), stored as fp16 with the block's exponent
  // (h_block_exp; the 16 columns of a row are one 16-lane DPP row), operand
  // order
  for (int t = tid; t < rows * 16; t += blockDim.x) {
    const int m = t >> 4, cc = t & 15;
    const int rr = m & 3, ll = cc + 16 * (m >> 2);
    float v[2];
#pragma unroll
    for (int b = 0; b < 2; b++) {
      v[b] = red[(b * 4 + rr) * 32 + ll];
      for (int w2 = 1; w2 < nwaves; w2++) v[b] += red[((w2 * 2 + b) * 4 + rr) * 32 + ll];
    }
    const float hv = silu_mul(v[0] * us0, v[1] * us1);
    const int ex = h_block_exp(row16_max(fabsf(hv)));
    const int n = b16 * 16 + cc;
    half_t* hp = reinterpret_cast<half_t*>(p.out) + (size_t)(row0 + m) * p.N + (n & ~7) + interleaved_pos(n & 7);
    int8_t* ep = p.hexp + (size_t)(row0 + m) * (p.N / 16) + b16;
    const half_t hq = (half_t)ldexpf(hv, -ex);
    if constexpr (COHERENT) {
      __hip_atomic_store(reinterpret_cast<uint16_t*>(hp), __builtin_bit_cast(uint16_t, hq), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (cc == 0) __hip_atomic_store(ep, (int8_t)ex, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      *hp = hq;
      if (cc == 0) *ep = (int8_t)ex;
    }
  }
  if (buf < 0) __syncthreads();
}

// The gate/up product of one (tile, 16-column block), on
// v_mfma_f32_16x16x32_f16, for the fused decode launch: tile rows [row0,
// row0 + rows) of expert e (rows <= kGemvMaxTokens), output columns
// [16 b16, 16 b16 + 16) of both banks, then h = silu(gate) * up.  Lane l
// takes column l % 16 of the block and the 8-byte half q = (l / 16) % 2 of
// the packed 16-byte unit (column, reduction half (l / 32)): its two words
// feed the two MFMAs of a slab, so MFMA m covers, for lane group (l / 16),
// reduction indices 32 (l / 32) + 16 q + 8 m + [0, 8) of the slab, and the
// activation fragment of tile row l % 16 is read to match (zeros past the
// tile).  SPW slabs per wave and pass.
// gen, us0, us1: the expert's dequantisation form and factors 2^-c.
template <int SPW, bool COHERENT = false>
__device__ __forceinline__ void gemv_tile16(const DecParams& p, const int32_t* sorted_pairs, int e,
                                            int row0, int rows, int b16, char* dsm, bool gen,
                                            float us0, float us1) {
  const int pass_slabs = (blockDim.x >> 6) * SPW;
  floatx4_t acc[2] = {floatx4_t{}, floatx4_t{}};
  for (int base = 0; base < p.K / 64; base += pass_slabs) {
    const Frag16<SPW> f = g16_load<SPW>(p, e, b16, base);
    g16_stage<SPW>(p, sorted_pairs, row0, rows, base, dsm);
    __syncthreads();
    if (gen) g16_mma<SPW, true>(p, f, rows, base, acc, dsm);
    else g16_mma<SPW, false>(p, f, rows, base, acc, dsm);
    __syncthreads();  // the next pass overwrites xs
  }
  g16_epilogue<COHERENT>(p, acc, row0, rows, b16, dsm, us0, us1);
}

// The grouped GEMM at decode sizes on a device block map: one workgroup per
// (tile, 32-column block); tiles past the map's count exit.
template <int MODE, int SPW>
__global__ __launch_bounds__(64 * kDecWavesMax) void w4_gemv_kernel(const DecParams p) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  const int nbl = p.N / 32;
  const int tile = blockIdx.x / nbl, blk = blockIdx.x % nbl;
  // the block count and this tile's entry are read together (the grid only
  // covers tiles below max_blocks, inside the map's allocation)
  const int nbm = *p.num_blocks;
  const int e = p.blocks[3 * tile], row0 = p.blocks[3 * tile + 1], rows = p.blocks[3 * tile + 2];
  if (tile >= min(nbm, p.max_blocks)) return;
  // a malformed block map is skipped, never dereferenced out of bounds
  if (e < 0 || e >= p.E || rows <= 0 || rows > kGemvMaxTokens || row0 < 0 || row0 > p.P - rows)
    return;
  const bool gen = (p.t0.general[e] | (MODE == MOE_GEMM_GATE_UP_SWIGLU ? p.t1.general[e] : 0u)) != 0;
  if (gen) gemv_tile<MODE, SPW, true>(p, p.sorted_pairs, e, row0, rows, blk, dsm);
  else gemv_tile<MODE, SPW, false>(p, p.sorted_pairs, e, row0, rows, blk, dsm);
}

struct DecRouteParams {
  const float* logits;  // [ksplit][T][E]
  float* logits_out;    // [T][E], written when ksplit > 1
  int ksplit, T;
  int32_t* ids;
  float* w;
  int32_t *counts, *offsets, *sorted_pairs, *pair_slot, *blocks, *num_blocks;
};

// Dequantise this wave's fragments of one item and multiply them with x rows
// resident in LDS ([T][K], operand order): tile row c (lane group row c < rows)
// reads token xrow_c's row, rows past the tile read zeros.
template <int SPW, bool GEN>
__device__ __forceinline__ void g16_mma_res(const DecParams& p, const Frag16<SPW>& f, int xrow_c,
                                            floatx4_t (&acc)[2], const char* dsm) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const half_t* xs = reinterpret_cast<const half_t*>(dsm) + (size_t)max(xrow_c, 0) * p.K;
  const int lg = (lane & 63) >> 4, khalf = lg >> 1, qh = lg & 1;
#pragma unroll
  for (int j = 0; j < SPW; j++) {
    const int sl = SPW * wave + j;
    if (sl >= p.K / 64) break;  // uniform per wave
    u32x4 x[2];
#pragma unroll
    for (int m = 0; m < 2; m++) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(xs + 64 * sl + 32 * khalf + 16 * qh + 8 * m);
      x[m] = xrow_c >= 0 ? v : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int b = 0; b < 2; b++) {
      const SbPair sp = sb_unpack(f.sb[b][j], GEN);
#pragma unroll
      for (int m = 0; m < 2; m++) {
        const uint32_t w = m == 0 ? f.q[b][j].x : f.q[b][j].y;
        const uint4 d = GEN ? dequant_word_gen(w, sp.s2, sp.c2, sp.b2) : dequant_word(w, sp.s2, sp.c2);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, x[m]),
                                                        __builtin_bit_cast(half8_t, d), acc[b], 0, 0, 0);
      }
    }
  }
}

// Decode sizes, S1-S6 in one launch.  Each workgroup first routes the whole
// batch (at most kGemvMaxTokens tokens, so at most kSmallPairs pairs) into
// LDS: the summed logits, the top-k of each token by one wave
// (topk_token: logit descending, lower expert first on ties, softmax over
// the chosen logits), the expert counts, then S2-S5 by the whole workgroup
// (decode_build_wg).  Every workgroup gets the same result (same
// inputs, same operations), so the block map needs no exchange; workgroup 0 writes it,
// and the rest of the routing, to global memory for the down projection and
// the caller.  Then the workgroup runs its (tile, 16-column block) items of
// the gate/up GEMV.  When the reduction fits one pass (x_res), all T rows of
// x (bf16 -> fp16 operand order) are staged into LDS once, read in the same
// round trip as the logits, and every item reads its tile's rows from there;
// otherwise each pass stages the tile's rows through the LDS scatter.
// NK = ceil(E / 64) keys per lane in the top-k.
// The routing of a decode batch in LDS: per-expert counts and token masks,
// the top-k ids and combine weights, offsets, the stable scatter (both
// directions) and the block map.
struct DecRouteLds {
  int cnt[256], wsc[8];
  uint32_t tokmask[256];
  int32_t ids[kSmallPairs], sp[kSmallPairs], ps[kSmallPairs];
  float w[kSmallPairs];
  int32_t off[257];
  int32_t blk[3 * kSmallMaxBlocks];
  int32_t nb[1];
};

// Device-scope counters of the single-launch decode layer: per expert, the
// gate/up items whose h columns are stored; the workgroups that finished;
// a flag set when a wait gave up (never in a correct run).
constexpr int kSyncDone = 256, kSyncErr = 257;
// Bound on the polls of one wait (each a device-scope round trip of about a
// microsecond, then s_sleep 2): about a second, so every wait ends.
constexpr int kSpinLimit = 1 << 20;

// The gate/up half of the decode layer for workgroup bid of G: routing into
// rl, then items bid, bid + G, ....  READY (the single-launch layer): h is
// stored device-coherent and, once a workgroup's item is stored, the item's
// expert's count in ready is raised.
template <int NK, int SPW, bool READY, bool NORM = false>
__device__ __forceinline__ void decode_gate_up_body(const DecRouteParams& r, const DecParams& p, int bid,
                                                    int G, char* dsm, DecRouteLds& rl, int32_t* ready) {
  int* const cnt = rl.cnt;
  int* const wsc = rl.wsc;
  uint32_t* const tokmask = rl.tokmask;
  int32_t* const ids_s = rl.ids;
  int32_t* const sp_s = rl.sp;
  int32_t* const ps_s = rl.ps;
  float* const w_s = rl.w;
  int32_t* const off_s = rl.off;
  int32_t* const blk_s = rl.blk;
  int32_t* const nb_s = rl.nb;
  __shared__ float us_s[2][256];  // every expert's 2^-c for gate and up
  __shared__ int gen_s[256];      // and dequantisation form (general if either bank's is)
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = blockDim.x >> 6;
  const int T = r.T, E = p.E, k = p.top_k, P = p.P, K = p.K;
  // [T][E] logits; without x_res the activation stage reuses the space
  float* lg = reinterpret_cast<float*>(dsm + p.lg_off);
  // 0. the per-expert tables of both banks, the logits and (x_res) the x
  //    rows: every load issued before any is stored (E <= 256, blockDim.x
  //    >= 64, T * K / 8 <= 4 blockDim.x with x_res)
  // (a wave whose first index is past the end issues no load: the test is
  // uniform, so it is a scalar branch; indices inside a wave stay clamped)
  const int wt0 = wave * 64;
  // (nothing loaded is combined before the stores below, so no branch waits)
  float ua[4], ub[4];
  uint32_t ga[4], gb[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int x = min(tid + i * (int)blockDim.x, E - 1);
    if (wt0 + i * (int)blockDim.x < E) {
      ua[i] = p.t0.unscale[x];
      ub[i] = p.t1.unscale[x];
      ga[i] = p.t0.general[x];
      gb[i] = p.t1.general[x];
    }
  }
  const int c8n = K / 8, nx8 = p.x_res ? T * c8n : 0;
  constexpr bool norm = NORM;  // (with x_res and gamma, checked by the launcher)
  uint4 xv[4], gv[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int idx = min(tid + i * (int)blockDim.x, max(nx8 - 1, 0));
    if (wt0 + i * (int)blockDim.x < nx8) {
      xv[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.a) + 8 * (size_t)idx);
      if constexpr (NORM) gv[i] = reinterpret_cast<const uint4*>(p.gamma)[idx % c8n];
    }
  }
  // 1. logits: partial sums over ranges of H added in range order
  const size_t part = (size_t)T * E;
  for (int i = tid; i < T * E; i += blockDim.x) {
    float v = r.logits[i];
    for (int z = 1; z < r.ksplit; z++) v += r.logits[z * part + i];
    lg[i] = v;
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int x = tid + i * blockDim.x;
    if (x < E) {
      us_s[0][x] = ua[i];
      us_s[1][x] = ub[i];
      gen_s[x] = (ga[i] | gb[i]) != 0;
    }
    const int idx = tid + i * blockDim.x;
    if (idx < nx8)  // x row idx / c8n, 8-element chunk idx % c8n (row stride K); raw bf16 with RMSNorm
      *reinterpret_cast<uint4*>(reinterpret_cast<half_t*>(dsm) + 8 * (size_t)idx) =
          norm ? xv[i] : bf16x8_to_half_interleaved(xv[i]);
  }
  for (int i = tid; i < E; i += blockDim.x) {
    cnt[i] = 0;
    tokmask[i] = 0u;
  }
  __syncthreads();
  if constexpr (NORM) {
    // RMSNorm in front: each row's 1 / rms by a wave, from the raw rows in
    // LDS, in moe_rmsnorm's order of operations (so the normalised rows equal
    // its output bit for bit); then every thread writes its pieces as the
    // normalised fp16 operand over the raw ones
    __shared__ float rn_s[kGemvMaxTokens];
    const int lane = tid & 63;
    const uint4* xr = reinterpret_cast<const uint4*>(dsm);
    for (int t = wave; t < T; t += nwaves) {
      float ss = 0.0f;
      for (int c = lane; c < c8n; c += 64) {
        const uint4 v = xr[t * c8n + c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float a = __uint_as_float(w[e] << 16), b = __uint_as_float(w[e] & 0xFFFF0000u);
          ss += a * a;
          ss += b * b;
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
      if (lane == 0) rn_s[t] = 1.0f / sqrtf(ss / (float)K + p.eps);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int idx = tid + i * blockDim.x;
      if (idx < nx8) {
        const float rr = rn_s[idx / c8n];
        const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w}, g[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; e++)
          o[e] = f32_to_bf16_rne(__uint_as_float(w[e] << 16) * rr * __uint_as_float(g[e] << 16)) |
                 (f32_to_bf16_rne(__uint_as_float(w[e] & 0xFFFF0000u) * rr * __uint_as_float(g[e] & 0xFFFF0000u))
                  << 16);
        *reinterpret_cast<uint4*>(reinterpret_cast<half_t*>(dsm) + 8 * (size_t)idx) =
            bf16x8_to_half_interleaved(make_uint4(o[0], o[1], o[2], o[3]));
      }
    }
  }
  // 2. top-k and combine weights, a wave per token, with the expert counts
  for (int t = wave; t < T; t += nwaves) topk_token<NK>(lg + t * E, E, k, ids_s + t * k, w_s + t * k, cnt);
  __syncthreads();
  // 3. with one pass per item, this workgroup's first item's weights are
  //    requested now, ahead of the block map: at decode sizes every touched
  //    expert is exactly one tile (at most T <= block_m pairs each), tile i
  //    the i-th touched expert in ascending order, so the counts name it
  const int nb16 = p.N / 16;
  const bool one_pass = K / 64 <= nwaves * SPW;
  Frag16<SPW> fa, fb;
  if (one_pass) {
    const int lane = tid & 63;
    int t = bid / nb16, e0 = -1;
#pragma unroll
    for (int i = 0; i < NK; i++) {
      const uint64_t m = __ballot(64 * i + lane < E && cnt[64 * i + lane] > 0);
      const int c = __popcll(m);
      if (e0 < 0 && t < c) {
        uint64_t w = m;
        for (int n = 0; n < t; n++) w &= w - 1;
        e0 = 64 * i + __builtin_ctzll(w);
      }
      t -= c;
    }
    if (e0 >= 0) {
      fa = g16_load<SPW>(p, e0, bid % nb16, 0);
      asm volatile("" ::: "memory");  // keep the loads here, ahead of the build
    }
  }
  // 4. offsets, scatter and block map
  decode_build_wg(ids_s, cnt, tokmask, wsc, P, E, k, off_s, sp_s, ps_s, blk_s, nb_s,
                  min(p.max_blocks, kSmallMaxBlocks));
  __syncthreads();
  // 5. the (tile, column block) items of this workgroup: bid, then every
  //    G-th after it (G is at most what the chip holds at once, so the
  //    routing above runs once per workgroup)
  const int items = nb_s[0] * nb16;
  // 6. workgroup 0 publishes the routing
  if (bid == 0) {
    for (int i = tid; i < P; i += blockDim.x) {
      r.ids[i] = ids_s[i];
      r.w[i] = w_s[i];
      r.sorted_pairs[i] = sp_s[i];
      r.pair_slot[i] = ps_s[i];
    }
    for (int i = tid; i < E; i += blockDim.x) r.counts[i] = cnt[i];
    for (int i = tid; i <= E; i += blockDim.x) r.offsets[i] = off_s[i];
    for (int i = tid; i < 3 * nb_s[0]; i += blockDim.x) r.blocks[i] = blk_s[i];
    if (tid == 0) r.num_blocks[0] = nb_s[0];
    if (r.ksplit > 1)
      for (int i = tid; i < T * E; i += blockDim.x) r.logits_out[i] = lg[i];
  }
  if (!p.x_res) __syncthreads();  // lg is overwritten by the activation stage below
  // READY: raise expert e's count once every wave's stores of its item
  // have completed (vmcnt counts stores; the count is raised by one thread
  // after the barrier)
  auto signal = [&](int e) {
    if constexpr (READY) {
      wait_vm<0>();
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(ready + e, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  if (!one_pass) {  // more than one pass per item
    for (int it = bid; it < items; it += G) {
      const int tile = it / nb16;
      const int e = blk_s[3 * tile];
      gemv_tile16<SPW, READY>(p, sp_s, e, blk_s[3 * tile + 1], blk_s[3 * tile + 2], it % nb16, dsm,
                              gen_s[e] != 0, us_s[0][e], us_s[1][e]);
      signal(e);
    }
    return;
  }
  // one pass per item: the next item's weight loads are issued before this
  // item's multiplies (two fragment sets, alternating).  READY: an item's
  // count is raised at the next item's wait for its fragments (which also
  // covers the stores before it), or after the last item.
  int it = bid;
  const int c = tid & 15;
  int pending = -1;  // READY: the expert of the item stored last, not yet counted
  while (it < items) {
#pragma unroll
    for (int half = 0; half < 2; half++) {
      const int tile = it / nb16, b16 = it % nb16;
      const int e = blk_s[3 * tile], row0 = blk_s[3 * tile + 1], rows = blk_s[3 * tile + 2];
      const int nx = it + G;
      int xrow_c = -1;  // this lane's tile row: its token, or -1 past the tile
      if (p.x_res) {
        const int pair = c < rows ? sp_s[row0 + c] : -1;
        xrow_c = (pair >= 0 && pair < P) ? pair / k : -1;
      } else {
        g16_stage<SPW>(p, sp_s, row0, rows, 0, dsm);
      }
      // this item's fragments (issued an item ago) and any staged x rows
      // have landed; the multiplies below then wait for nothing issued
      // after this point
      wait_vm<0>();
      if (READY && pending >= 0) {
        signal(pending);
        pending = -1;
      }
      if (nx < items) {
        if (half == 0) fb = g16_load<SPW>(p, blk_s[3 * (nx / nb16)], nx % nb16, 0);
        else fa = g16_load<SPW>(p, blk_s[3 * (nx / nb16)], nx % nb16, 0);
      }
      if (!p.x_res) __syncthreads();
      floatx4_t acc[2] = {floatx4_t{}, floatx4_t{}};
      if (p.x_res) {
        if (gen_s[e]) g16_mma_res<SPW, true>(p, half == 0 ? fa : fb, xrow_c, acc, dsm);
        else g16_mma_res<SPW, false>(p, half == 0 ? fa : fb, xrow_c, acc, dsm);
      } else {
        if (gen_s[e]) g16_mma<SPW, true>(p, half == 0 ? fa : fb, rows, 0, acc, dsm);
        else g16_mma<SPW, false>(p, half == 0 ? fa : fb, rows, 0, acc, dsm);
        __syncthreads();
      }
      g16_epilogue<READY>(p, acc, row0, rows, b16, dsm, us_s[0][e], us_s[1][e], p.x_res ? half : -1);
      pending = e;
      it = nx;
      if (it >= items) break;
    }
  }
  if (READY && pending >= 0) signal(pending);
}

template <int NK, int SPW, bool NORM>
__global__ __launch_bounds__(64 * kDecWavesMax) void decode_gate_up_kernel(const DecRouteParams r,
                                                                          const DecParams p) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  __shared__ DecRouteLds rl;
  decode_gate_up_body<NK, SPW, false, NORM>(r, p, blockIdx.x, gridDim.x, dsm, rl, nullptr);
}

// Decode sizes, S7 and S8 in one launch, organised per token: workgroup
// (t, 16-column block) computes d_j = h[t, j] . dq(Wd_e)^T over the block
// for each of the token's k choices (e = its expert, h row at its slot),
// then y[t] = sum_j w[t, j] * d_j in choice order, and also writes each
// weighted row w[t, j] * d_j to y_sorted at the slot.  No other workgroup
// contributes to its outputs, so there is no cross-workgroup exchange; an
// expert chosen by several tokens of the batch is read once per token (the
// later reads mostly hit the L2 or the last-level cache).
// One wave per 64-wide slab of the reduction (K <= 64 * kDecWavesMax, one
// pass); the choices go in chunks of kDownChunk, all weight loads of a chunk
// issued at once.  Each d_j runs on v_mfma_f32_16x16x32_f16 (two per slab)
// with h in MFMA row 0 (zeros elsewhere).  Lane l takes column l % 16 of
// the block and the 8-byte half q = (l / 16) % 2 of the packed 16-byte unit
// (column, reduction half (l / 32)): its two words feed the two MFMAs, so
// MFMA m of a slab covers, for lane group (l / 16), reduction indices
// 32 (l / 32) + 16 q + 8 m + [0, 8), and the h fragment is read to match.
// The waves' row-0 partials meet in LDS and are added in wave order.  The
// weighting and the sum are plain fp32 multiplies and adds (no
// contraction), so y equals the fp32 sum in choice order of the y_sorted
// rows exactly.
constexpr int kDownChunk = 8;

// The down half for (token t, 16-column block b16).  ids, pair_slot,
// topk_w: the routing (global or LDS).  WAIT (the single-launch layer): the
// weights of a chunk of choices are requested first, then the workgroup
// waits until each chosen expert's count in ready reaches need (every
// gate/up item of its tile stored), then reads h and its exponents with
// device-scope loads.
template <bool WAIT, int SPW = 1>
__device__ __forceinline__ void decode_down_body(const DecParams& p, int t, int b16,
                                                 const int32_t* __restrict__ ids,
                                                 const int32_t* __restrict__ pair_slot,
                                                 const float* __restrict__ topk_w, float* __restrict__ y,
                                                 const uint16_t* __restrict__ residual,
                                                 uint16_t* __restrict__ out, char* dsm, int32_t* ready,
                                                 int need, int32_t* err, int done_target) {
  __shared__ int e_s[16], slot_s[16];
  __shared__ float w_s[16], v_s[16 * 16];
  __shared__ float us_s[256];  // every expert's 2^-c and dequantisation form
  __shared__ int genx_s[256];
  __shared__ __attribute__((aligned(16))) half_t zrow[16];  // zeros: the MFMA's rows other than 0
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbl = p.N / 32;
  const int K = p.K, S = K / 64, gpr = K >> p.log2_G, k = p.top_k;
  const int c = lane & 15, lg = lane >> 4, khalf = lg >> 1, qh = lg & 1;
  const int col = 16 * (b16 & 1) + c;  // column within the 32-column packed block
  // LDS: xs = the h rows of a chunk [kDownChunk][K] (operand order); red
  // (at red_off) = row 0 of each wave's partial per choice [wave][k][16]
  half_t* xs = reinterpret_cast<half_t*>(dsm);
  float* red = reinterpret_cast<float*>(dsm + p.red_off);
  // the token's choices (expert, slot and combine weight) and every
  // expert's 2^-c and dequantisation form, read in one round trip with
  // clamped indices, no branches (a malformed id is replaced by 0 and a
  // malformed slot skipped, never used out of bounds); blockDim.x >= 128 and
  // E <= 256
  float ut[2];
  int gt[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int x = min(tid + i * (int)blockDim.x, p.E - 1);
    ut[i] = p.t0.unscale[x];
    gt[i] = p.t0.general[x] != 0;
  }
  const int pair = t * k + min(tid, k - 1);
  const int e = ids[pair], slot = pair_slot[pair];
  const float wt = topk_w[pair];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int x = tid + i * blockDim.x;
    if (x < p.E) {
      us_s[x] = ut[i];
      genx_s[x] = gt[i];
    }
  }
  if (tid < k) {
    e_s[tid] = (e >= 0 && e < p.E) ? e : 0;
    slot_s[tid] = (slot >= 0 && slot < p.P) ? slot : -1;
    w_s[tid] = wt;
  }
  if (tid < 8) reinterpret_cast<uint32_t*>(zrow)[tid] = 0u;
  __syncthreads();
  // lane j < k of every wave holds choice j's expert, slot and 2^-c, read
  // once; choice j's values are taken from lane j (uniform), its
  // dequantisation form is bit j of gmask
  const int jl = lane < k ? lane : 0;
  const int e_l = e_s[jl], slot_l = max(slot_s[jl], 0);
  const float us_l = us_s[e_l];
  const uint64_t gmask = __ballot(lane < k && genx_s[e_l] != 0);
  // this wave's slabs wave * SPW + i (nwaves * SPW == S) and their groups
  int sl_[SPW], g_[SPW];
#pragma unroll
  for (int i = 0; i < SPW; i++) {
    sl_[i] = wave * SPW + i;
    g_[i] = (64 * sl_[i] + 32 * khalf) >> p.log2_G;
  }
  int done_old = -1;  // WAIT: the done count before this workgroup's (thread 0)
  for (int j0 = 0; j0 < k; j0 += kDownChunk) {
    const int nj = min(kDownChunk, k - j0);
    // 1. the chunk's h rows, 16 bytes per thread (nj * K / 8 <= 64 * S
    //    threads), requested first: their LDS write then waits for them
    //    alone, not for the weights requested after them
    const int c8n = K / 8;
    bool stager[SPW];
    int hm[SPW], hc8[SPW];
    uint4 hv[SPW];
#pragma unroll
    for (int u = 0; u < SPW; u++) {  // nj * K / 8 <= SPW * blockDim.x pieces
      const int idx = tid + u * (int)blockDim.x;
      stager[u] = idx < nj * c8n;
      hm[u] = stager[u] ? idx / c8n : 0;
      hc8[u] = stager[u] ? idx % c8n : 0;
      hv[u] = make_uint4(0, 0, 0, 0);
      if (!WAIT && stager[u])
        hv[u] = *reinterpret_cast<const uint4*>(p.a + (size_t)max(slot_s[j0 + hm[u]], 0) * K + 8 * hc8[u]);
    }
    // 2. codes (two words) and (scale, bias) word of every choice of the
    //    chunk, and the exponents of the slab's four 16-column blocks of its
    //    h row (one word: a scalar load)
    uint2 q[kDownChunk][SPW];
    uint32_t sb[kDownChunk][SPW], hx[kDownChunk][SPW];
#pragma unroll
    for (int j = 0; j < kDownChunk; j++) {
      const int jj = min(j0 + j, k - 1);
      const int ej = __builtin_amdgcn_readlane(e_l, jj);
      const int sl = __builtin_amdgcn_readlane(slot_l, jj);
      const size_t bidx = (size_t)ej * nbl + (b16 >> 1);
#pragma unroll
      for (int i = 0; i < SPW; i++) {
        q[j][i] = *reinterpret_cast<const uint2*>(p.b0.words + ((bidx >> 2) * S * 4 + (bidx & 3)) * 256 +
                                                  4 * (2 * col + khalf) + 2 * qh + (size_t)sl_[i] * 1024);
        sb[j][i] = p.b0.sb[(bidx >> 2) * gpr * 128 + (bidx & 3) * 32 + col + (size_t)g_[i] * 128];
        if (!WAIT) hx[j][i] = reinterpret_cast<const uint32_t*>(p.hexp + (size_t)sl * (K / 16))[sl_[i]];
      }
    }
    if constexpr (WAIT) {
      // the chunk's experts: lane j of wave 0 polls expert j's count (a
      // malformed choice reads expert 0's, whose wait then gives up)
      if (tid < nj) {
        const int32_t* rp = ready + e_s[j0 + tid];
        int polls = 0;
        while (__hip_atomic_load(rp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
          if (++polls > kSpinLimit) {
            __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      __syncthreads();
      // after its last wait, the workgroup counts itself done; the last down
      // workgroup to do so returns the counts to zero (every count it
      // clears has reached its final value: each touched expert's producers
      // finished before its consumers' waits ended, and every consumer has
      // passed its waits)
      // (the count's old value is read at the end, so its round trip
      // overlaps the multiplies)
      if (j0 + kDownChunk >= k && tid == 0)
        done_old = __hip_atomic_fetch_add(ready + kSyncDone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // h rows and exponents with device-scope loads: they miss any stale
      // line another XCD's L2 may hold
#pragma unroll
      for (int u = 0; u < SPW; u++)
        if (stager[u]) {
          const uint64_t* hs =
              reinterpret_cast<const uint64_t*>(p.a + (size_t)max(slot_s[j0 + hm[u]], 0) * K + 8 * hc8[u]);
          const uint64_t lo = __hip_atomic_load(hs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t hi = __hip_atomic_load(hs + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          hv[u] = make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
        }
#pragma unroll
      for (int j = 0; j < kDownChunk; j++) {
        const int sl = __builtin_amdgcn_readlane(slot_l, min(j0 + j, k - 1));
#pragma unroll
        for (int i = 0; i < SPW; i++)
          hx[j][i] = __hip_atomic_load(reinterpret_cast<const uint32_t*>(p.hexp + (size_t)sl * (K / 16)) + sl_[i],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int u = 0; u < SPW; u++)
      if (stager[u]) *reinterpret_cast<uint4*>(xs + hm[u] * K + 8 * hc8[u]) = hv[u];
    __syncthreads();
    // 3. per choice: dequantise, multiply, keep row 0 (lanes with c == 0
    //    read the h fragment, the others the zero row).  The slab's blocks
    //    are brought to their largest exponent es (skipped when all four are
    //    0, the usual case) and the partial scaled by 2^es and the expert's
    //    2^-c (powers of two: exact in fp32 short of its range)
    const int xstride = c == 0 ? K : 0;
    auto run = [&](auto gen_tag) {
      constexpr bool ANY_GEN = decltype(gen_tag)::value;
#pragma unroll
      for (int j = 0; j < kDownChunk; j++) {
        if (j >= nj) break;
        const float us = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(us_l), j0 + j));
#pragma unroll
        for (int i = 0; i < SPW; i++) {
          const half_t* xrow = c == 0 ? xs + 64 * sl_[i] + 32 * khalf + 16 * qh : zrow;
          u32x4 xf[2];
#pragma unroll
          for (int m = 0; m < 2; m++) xf[m] = *reinterpret_cast<const u32x4*>(xrow + j * xstride + 8 * m);
          const uint32_t hw = hx[j][i];
          int es = 0;
          if (hw) {
            es = max_i8x4(hw);
            // the exponent of the block this lane's h values come from
            const int d = (int)(int8_t)(hw >> (8 * (2 * khalf + qh))) - es;
#pragma unroll
            for (int m = 0; m < 2; m++)
              xf[m] = __builtin_bit_cast(u32x4, scale_half8(__builtin_bit_cast(uint4, xf[m]), d));
          }
          floatx4_t acc = floatx4_t{};
          auto multiply = [&](auto g_tag) {
            constexpr bool GEN = decltype(g_tag)::value;
            const SbPair sp = sb_unpack(sb[j][i], GEN);
#pragma unroll
            for (int m = 0; m < 2; m++) {
              const uint32_t w = m == 0 ? q[j][i].x : q[j][i].y;
              const uint4 dq = GEN ? dequant_word_gen(w, sp.s2, sp.c2, sp.b2) : dequant_word(w, sp.s2, sp.c2);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, xf[m]),
                                                           __builtin_bit_cast(half8_t, dq), acc, 0, 0, 0);
            }
          };
          if constexpr (ANY_GEN) {
            if ((gmask >> (j0 + j)) & 1) multiply(std::true_type{});
            else multiply(std::false_type{});
          } else {
            multiply(std::false_type{});
          }
          // one partial per slab, so the sum below adds them in slab order
          // whatever the slabs per wave
          if (lane < 16) red[(sl_[i] * k + j0 + j) * 16 + lane] = ldexpf(acc[0] * us, es);
        }
      }
    };
    if ((gmask >> j0) & ((1ull << nj) - 1)) run(std::true_type{});
    else run(std::false_type{});
    __syncthreads();  // the next chunk overwrites xs
  }
  // 4. the weighted rows (one thread per choice and column), then their sum
  //    in choice order
  {
#pragma clang fp contract(off)
    for (int i = tid; i < k * 16; i += blockDim.x) {
      const int j = i >> 4, cc = i & 15;
      float d = red[j * 16 + cc];
      for (int s2 = 1; s2 < S; s2++) d += red[(s2 * k + j) * 16 + cc];
      const float v = w_s[j] * d;
      v_s[i] = v;
      if (slot_s[j] >= 0) reinterpret_cast<float*>(p.out)[(size_t)slot_s[j] * p.N + b16 * 16 + cc] = v;
    }
    __syncthreads();
    if (tid < 16) {
      float acc = 0.0f;
      for (int j = 0; j < k; j++) acc = acc + v_s[j * 16 + tid];
      y[(size_t)t * p.N + b16 * 16 + tid] = acc;
      if (out) {
        const size_t at = (size_t)t * p.N + b16 * 16 + tid;
        out[at] = (uint16_t)f32_to_bf16_rne(__uint_as_float((uint32_t)residual[at] << 16) + acc);
      }
    }
  }
  if constexpr (WAIT) {
    // the last down workgroup clears the counts, one per thread
    __shared__ int last_s;
    if (tid == 0) last_s = done_old == done_target - 1;
    __syncthreads();
    if (last_s) {
      for (int e2 = tid; e2 < p.E; e2 += blockDim.x)
        __hip_atomic_store(ready + e2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (tid == 0) __hip_atomic_store(ready + kSyncDone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int SPW>
__global__ __launch_bounds__(64 * kDecWavesMax) void decode_down_kernel(
    const DecParams p, const int32_t* __restrict__ ids, const int32_t* __restrict__ pair_slot,
    float* __restrict__ y, const uint16_t* __restrict__ residual, uint16_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  const int nb16 = p.N / 16;
  decode_down_body<false, SPW>(p, blockIdx.x / nb16, blockIdx.x % nb16, ids, pair_slot, p.topk_weights, y,
                               residual, out, dsm, nullptr, 0, nullptr, 0);
}

// The routing of the batch into rl, as every gate/up workgroup computes it
// (same loads, same order of the partial sums, same top-k and build), for a
// workgroup that runs the down half; lg: T * E floats of LDS.
template <int NK>
__device__ __forceinline__ void decode_route_only(const DecRouteParams& r, const DecParams& p, float* lg,
                                                  DecRouteLds& rl) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), nwaves = blockDim.x >> 6;
  const int T = r.T, E = p.E, k = p.top_k;
  const size_t part = (size_t)T * E;
  for (int i = tid; i < T * E; i += blockDim.x) {
    float v = r.logits[i];
    for (int z = 1; z < r.ksplit; z++) v += r.logits[z * part + i];
    lg[i] = v;
  }
  for (int i = tid; i < E; i += blockDim.x) {
    rl.cnt[i] = 0;
    rl.tokmask[i] = 0u;
  }
  __syncthreads();
  for (int t = wave; t < T; t += nwaves) topk_token<NK>(lg + t * E, E, k, rl.ids + t * k, rl.w + t * k, rl.cnt);
  __syncthreads();
  decode_build_wg(rl.ids, rl.cnt, rl.tokmask, rl.wsc, p.P, E, k, rl.off, rl.sp, rl.ps, rl.blk, rl.nb,
                  min(p.max_blocks, kSmallMaxBlocks));
  __syncthreads();
}

// Decode sizes, the whole layer (S1-S8) in one launch.  Workgroups [0, G1)
// run the gate/up half (decode_gate_up_body with ready counts), the
// workgroups after them the down half of (token, 16-column block)
// (decode_down_body, waiting on the counts of the token's experts), after
// routing the batch themselves.  Workgroups are dispatched in index order
// on each XCD, so every gate/up workgroup holds a slot before a down
// workgroup that waits on it does, and the gate/up half waits on nothing:
// the waits end.  h crosses XCDs through device-scope stores and loads, no
// cache writeback or invalidation.  Each down workgroup counts itself done
// after its last wait; the last returns the counts to zero, so sync is zero
// again for the next call.
template <int NK, int SPW>
__global__ __launch_bounds__(64 * kDecWavesMax) void decode_layer_kernel(
    const DecRouteParams r, const DecParams pg, const DecParams pd, float* __restrict__ y,
    const uint16_t* __restrict__ residual, uint16_t* __restrict__ out, int32_t* __restrict__ sync, int G1) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  __shared__ DecRouteLds rl;
  const int bid = blockIdx.x;
  if (bid < G1) {
    decode_gate_up_body<NK, SPW, true>(r, pg, bid, G1, dsm, rl, sync);
  } else {
    decode_route_only<NK>(r, pg, reinterpret_cast<float*>(dsm), rl);
    const int nb16 = pd.N / 16, item = bid - G1;
    decode_down_body<true>(pd, item / nb16, item % nb16, rl.ids, rl.ps, rl.w, y, residual, out, dsm, sync,
                           pg.N / 16, sync + kSyncErr, (int)gridDim.x - G1);
  }
}

// Slabs per wave and waves per workgroup for a launch of `grid` workgroups
// over reduction length K: four slabs per wave when the grid fills the chip
// twice over (two 8-wave workgroups per CU overlap one's loads with the
// other's MFMAs); otherwise two (up to 16 waves, as many bytes in flight per
// workgroup as possible).
struct GemvShape {
  int spw, waves;
};
GemvShape gemv_shape(int K, int64_t grid) {
  const bool wide = K >= 1024 && grid >= 1024;
  const int spw = wide ? 4 : 2;
  const int waves = (int)std::max<int64_t>(1, std::min<int64_t>(kDecWavesMax, K / (64 * spw)));
  return GemvShape{spw, waves};
}

DecParams dec_params(const GemmArgs& a, int64_t P, int64_t max_blocks, int xs_bytes) {
  const int log2_G = a.G == 32 ? 5 : a.G == 64 ? 6 : 7;  // G in {32, 64, 128}
  return DecParams{a.a, a.b0, a.b1, a.sorted_pairs, a.topk_weights, a.blocks, a.num_blocks, a.out,
                   a.t0, a.t1, a.hexp, a.tflags, a.N, a.K, log2_G, a.top_k, a.E, (int)P, (int)max_blocks,
                   xs_bytes};
}

}  // namespace

hipError_t launch_w4_gemv(const GemmArgs& a, hipStream_t s) {
  const int64_t P = (int64_t)a.T * a.top_k;
  const int64_t max_blocks = P / a.block_m + (P < a.E ? P : a.E);
  const int64_t grid = max_blocks * (a.N / 32);
  const GemvShape sh = gemv_shape(a.K, grid);
  const bool wide = sh.spw == 4;
  const int nb = a.mode == MOE_GEMM_GATE_UP_SWIGLU ? 2 : 1;
  // LDS: activation rows of one pass + the waves' partial sums
  const int xs_bytes = kGemvMaxTokens * sh.waves * sh.spw * 64 * 2;
  const size_t lds = (size_t)xs_bytes + (size_t)sh.waves * nb * 4 * 64 * 4;
  const DecParams p = dec_params(a, P, max_blocks, xs_bytes);
  const int waves = sh.waves;
  if (a.mode == MOE_GEMM_GATE_UP_SWIGLU) {
    if (wide) w4_gemv_kernel<MOE_GEMM_GATE_UP_SWIGLU, 4><<<grid, 64 * waves, lds, s>>>(p);
    else w4_gemv_kernel<MOE_GEMM_GATE_UP_SWIGLU, 2><<<grid, 64 * waves, lds, s>>>(p);
  } else if (a.y16e) {
    return hipErrorInvalidValue;  // the decode path keeps the weighted outputs in fp32
  } else {
    if (wide) w4_gemv_kernel<MOE_GEMM_DOWN, 4><<<grid, 64 * waves, lds, s>>>(p);
    else w4_gemv_kernel<MOE_GEMM_DOWN, 2><<<grid, 64 * waves, lds, s>>>(p);
  }
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int NK>
static void launch_decode_nk(const DecRouteParams& r, const DecParams& p, bool wide, int64_t grid,
                             int threads, size_t lds, hipStream_t s) {
  if (p.gamma) {
    if (wide) decode_gate_up_kernel<NK, 4, true><<<grid, threads, lds, s>>>(r, p);
    else decode_gate_up_kernel<NK, 2, true><<<grid, threads, lds, s>>>(r, p);
  } else {
    if (wide) decode_gate_up_kernel<NK, 4, false><<<grid, threads, lds, s>>>(r, p);
    else decode_gate_up_kernel<NK, 2, false><<<grid, threads, lds, s>>>(r, p);
  }
}

// Launch shape of the gate/up half at decode sizes.
namespace {
struct DecGateUpPlan {
  DecParams p;
  bool wide;
  int threads;
  size_t lds;     // dynamic LDS
  int64_t items;  // (tile, 16-column block) items at most
};
}  // namespace
static bool decode_gate_up_plan(const GemmArgs& a, DecGateUpPlan& pl) {
  if (a.T > kGemvMaxTokens || a.block_m != kGemvMaxTokens || a.E > 256 ||
      (int64_t)a.T * a.top_k > kSmallPairs)
    return false;
  const int64_t P = (int64_t)a.T * a.top_k;
  const int64_t max_blocks = P / a.block_m + (P < a.E ? P : a.E);
  pl.items = max_blocks * (a.N / 16);
  // four slabs per wave (8 waves cover K = 2048 in one pass, two workgroups
  // per CU) when K allows it: fewer waves to launch, the same bytes in flight
  const int spw = a.K >= 1024 ? 4 : 2;
  const GemvShape sh{spw, std::max(1, std::min(kDecWavesMax, a.K / (64 * spw)))};
  // LDS, one pass with every x row resident (x_res): the T x rows, the
  // logits, the waves' partial sums of both banks (rows 0..7 of 16 columns);
  // otherwise the logits, then (reused) the activation rows of one pass, and
  // the partial sums
  const int red_bytes = 2 * sh.waves * 2 * 4 * 32 * 4;  // two halves (alternating items, x_res)
  const int lg_bytes = (a.T * a.E * 4 + 15) & ~15;
  const int xres_bytes = (a.T * a.K * 2 + 15) & ~15;
  const bool one_pass = a.K <= sh.waves * sh.spw * 64;
  const bool x_res = one_pass && xres_bytes + lg_bytes + red_bytes <= 64 * 1024;
  int red_off, lg_off;
  if (x_res) {
    lg_off = xres_bytes;
    red_off = xres_bytes + lg_bytes;
  } else {
    const int xs_bytes = std::max(kGemvMaxTokens * sh.waves * sh.spw * 64 * 2, a.T * a.E * 4);
    lg_off = 0;
    red_off = (xs_bytes + 15) & ~15;
  }
  pl.lds = (size_t)red_off + red_bytes;
  pl.p = dec_params(a, P, max_blocks, red_off);
  pl.p.lg_off = lg_off;
  pl.p.x_res = x_res;
  pl.wide = sh.spw == 4;
  pl.threads = 64 * sh.waves;
  return true;
}

// Workgroups of `threads` threads with `lds` bytes of dynamic LDS (plus
// about `static_kib` KiB of static LDS) that one CU holds at once, at most
// 4 waves per SIMD.
static int decode_per_cu(int threads, size_t lds, int static_kib) {
  return std::max(1, std::min<int>(16 / (threads / 64), (int)((160 * 1024) / (lds + static_kib * 1024))));
}

bool decode_norm_fits(const GemmArgs& a) {
  DecGateUpPlan pl;
  return decode_gate_up_plan(a, pl) && pl.p.x_res;
}

hipError_t launch_decode_gate_up(const DecodeRouting& dr, const GemmArgs& a, hipStream_t s,
                                 const uint16_t* gamma, float eps) {
  if (a.T <= 0) return hipSuccess;
  DecGateUpPlan pl;
  if (!decode_gate_up_plan(a, pl)) return hipErrorInvalidValue;
  if (gamma && !pl.p.x_res) return hipErrorInvalidValue;
  pl.p.gamma = gamma;
  pl.p.eps = eps;
  const DecRouteParams r{dr.logits, dr.logits_out, dr.ksplit, a.T,
                         dr.ids, dr.w, dr.counts, dr.offsets, dr.sorted_pairs, dr.pair_slot,
                         dr.blocks, dr.num_blocks};
  // at most one round of workgroups: the routing then runs once per
  // workgroup
  const int64_t grid = std::min<int64_t>(pl.items, (int64_t)device_cus() * decode_per_cu(pl.threads, pl.lds, 12));
  switch ((a.E + 63) / 64) {
    case 1: launch_decode_nk<1>(r, pl.p, pl.wide, grid, pl.threads, pl.lds, s); break;
    case 2: launch_decode_nk<2>(r, pl.p, pl.wide, grid, pl.threads, pl.lds, s); break;
    case 3: launch_decode_nk<3>(r, pl.p, pl.wide, grid, pl.threads, pl.lds, s); break;
    default: launch_decode_nk<4>(r, pl.p, pl.wide, grid, pl.threads, pl.lds, s); break;
  }
  return hipGetLastError();
}

bool decode_down_fused(int K) { return K % 64 == 0 && K / 64 <= kDecWavesMax; }

hipError_t launch_decode_down(const GemmArgs& a, const int32_t* ids, const int32_t* pair_slot,
                              float* y, hipStream_t s, const uint16_t* residual, uint16_t* out) {
  if (a.T <= 0) return hipSuccess;
  if (a.T > kGemvMaxTokens || !decode_down_fused(a.K)) return hipErrorInvalidValue;
  const int64_t P = (int64_t)a.T * a.top_k;
  const int64_t grid = (int64_t)a.T * (a.N / 16);
  // one wave per slab; two slabs per wave when the grid would otherwise
  // need more than one round of three 8-wave workgroups per CU (half the
  // waves, so four workgroups share a CU: at H = 2048 and T = 8 the 1,024
  // workgroups then run in one round)
  const int S = a.K / 64;
  const int spw = (S % 2 == 0 && S >= 4 && grid > 3 * (int64_t)device_cus()) ? 2 : 1;
  const int waves = S / spw;
  const int xs_bytes = kDownChunk * a.K * 2;
  const size_t lds = (size_t)xs_bytes + (size_t)S * a.top_k * 16 * 4;  // one partial per slab and choice
  const DecParams p = dec_params(a, P, 0, xs_bytes);
  if (spw == 2) decode_down_kernel<2><<<grid, 64 * waves, lds, s>>>(p, ids, pair_slot, y, residual, out);
  else decode_down_kernel<1><<<grid, 64 * waves, lds, s>>>(p, ids, pair_slot, y, residual, out);
  return hipGetLastError();
}

template <int NK>
static void launch_layer_nk(const DecRouteParams& r, const DecParams& pg, const DecParams& pd, bool wide,
                            int64_t grid, int threads, size_t lds, float* y, const uint16_t* residual,
                            uint16_t* out, int32_t* sync, int G1, hipStream_t s) {
  if (wide) decode_layer_kernel<NK, 4><<<grid, threads, lds, s>>>(r, pg, pd, y, residual, out, sync, G1);
  else decode_layer_kernel<NK, 2><<<grid, threads, lds, s>>>(r, pg, pd, y, residual, out, sync, G1);
}

bool decode_layer_supported(const GemmArgs& g, const GemmArgs& d) {
  DecGateUpPlan pl;
  return decode_gate_up_plan(g, pl) && decode_down_fused(d.K) && pl.threads == 64 * (d.K / 64);
}

hipError_t launch_decode_layer(const DecodeRouting& dr, const GemmArgs& g, const GemmArgs& d, float* y,
                               int32_t* sync, hipStream_t s, const uint16_t* residual, uint16_t* out) {
  if (g.T <= 0) return hipSuccess;
  DecGateUpPlan pl;
  if (!decode_gate_up_plan(g, pl) || !decode_down_fused(d.K) || pl.threads != 64 * (d.K / 64))
    return hipErrorInvalidValue;
  const int64_t P = (int64_t)d.T * d.top_k;
  const int xs_bytes = kDownChunk * d.K * 2;
  const size_t lds_d = (size_t)xs_bytes + (size_t)(d.K / 64) * d.top_k * 16 * 4;
  const size_t lds = std::max({pl.lds, lds_d, (size_t)g.T * g.E * 4});
  const DecParams pd = dec_params(d, P, 0, xs_bytes);
  const DecRouteParams r{dr.logits, dr.logits_out, dr.ksplit, g.T,
                         dr.ids, dr.w, dr.counts, dr.offsets, dr.sorted_pairs, dr.pair_slot,
                         dr.blocks, dr.num_blocks};
  // gate/up workgroups: what the chip holds at once, less the down
  // workgroups when those take at most half of it, so the down half starts
  // with the gate/up half (routing, its first weights in flight) instead of
  // after it
  const int64_t slots = (int64_t)device_cus() * decode_per_cu(pl.threads, lds, 16);
  const int64_t G2 = (int64_t)d.T * (d.N / 16);
  const int64_t G1 = std::min<int64_t>(pl.items, 2 * G2 <= slots ? slots - G2 : slots);
  const int64_t grid = G1 + G2;
  switch ((g.E + 63) / 64) {
    case 1: launch_layer_nk<1>(r, pl.p, pd, pl.wide, grid, pl.threads, lds, y, residual, out, sync, (int)G1, s); break;
    case 2: launch_layer_nk<2>(r, pl.p, pd, pl.wide, grid, pl.threads, lds, y, residual, out, sync, (int)G1, s); break;
    case 3: launch_layer_nk<3>(r, pl.p, pd, pl.wide, grid, pl.threads, lds, y, residual, out, sync, (int)G1, s); break;
    default: launch_layer_nk<4>(r, pl.p, pd, pl.wide, grid, pl.threads, lds, y, residual, out, sync, (int)G1, s); break;
  }
  return hipGetLastError();
}

}  // namespace moe
