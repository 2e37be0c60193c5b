// attn.hip -- a second workload: decode attention over a block-paged KV
// cache with grouped query heads.  Page "Perplexity's Lily engine beats MLX
// by 35% on M5 Max", architecture paragraph: the decode gains come from
// coalesced key-cache reads, packing the query heads that share a KV head,
// and a fixed-block cache layout.  Here:
//  - keys are [block][KV head][BLK positions][D] bf16 and values
//    [block][KV head][D][BLK] bf16 (element-major), blocks found through a
//    block table (scattered blocks cost nothing extra);
//  - a workgroup owns (sequence, KV head, range of positions) and all GQ
//    query heads of that KV head, so every key and value is read once and
//    used GQ times; its 4 waves take steps of 32 positions in turn;
//  - both contractions run on v_mfma_f32_16x16x32_bf16, with the heads as
//    the 16 columns (padded): scores as K q^T (rows = positions, in an order
//    chosen so that each lane ends with 8 consecutive positions of one head),
//    and the output as V^T P^T, whose operand of V is one 16-byte load of 8
//    consecutive positions of one element in the element-major layout;
//  - softmax in base 2 with a running maximum per head (the scores scaled
//    by log2(e) / sqrt(D)); the probabilities enter the second product as a
//    bf16 pair hi + lo (hi = the upper half of the fp32 bits, lo = the
//    remainder rounded), so the weights keep about 16 bits and the sums stay
//    fp32;
//  - the 4 waves are merged in LDS in fixed order into one partial result
//    per range, and a second launch merges the ranges in fixed order, so the
//    output does not depend on timing.
#include "internal.h"

namespace moe {
namespace {

constexpr int kAttnD = 128;
constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kAttnGroups = 128;   // runs of 8 positions in a range (ranges are at most 1024 long)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));

struct AttnParams {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* table;
  const int32_t* lens;
  float* part_m;    // [B][Hq][nsplit]
  float* part_l;    // [B][Hq][nsplit]
  float* part_acc;  // [B][Hq][nsplit][D]
  int Hq, Hkv, block, max_blocks, num_blocks, nsplit, chunk;
  float qscale;     // log2(e) / sqrt(D)
  int max_len;      // positions at or past it are never visited
};

template <int GQ>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_split_kernel(const AttnParams p) {
  constexpr int kWaves = kAttnThreads / 64;
  constexpr int kRow = kAttnD + 4;  // LDS row of the merge (padded against bank conflicts)
  __shared__ int gslab[kAttnGroups], goff[kAttnGroups];
  __shared__ float sm[kWaves][GQ], sl[kWaves][GQ];
  __shared__ __attribute__((aligned(16))) float sacc[kWaves][GQ][kRow];
  const int tid = threadIdx.x, r = tid & 15, g = (tid >> 4) & 3;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t0 = s * p.chunk;
  // each run of 8 positions of the range (t0 and the block length are
  // multiples of 8, so a run lies in one block): its block and KV head as
  // one index (-1: skipped block) and its offset in the block, once, in LDS.
  // The whole range's entries are read without waiting for the sequence
  // length (entries past it are never used).
  const int ngr = p.chunk / 8;  // <= kAttnGroups (host plan)
  for (int i = tid; i < ngr; i += kAttnThreads) {
    const int t = t0 + 8 * i, bi = t / p.block;
    const int blk = bi < p.max_blocks ? p.table[(size_t)b * p.max_blocks + bi] : -1;
    gslab[i] = (blk >= 0 && blk < p.num_blocks) ? blk * p.Hkv + h : -1;
    goff[i] = t % p.block;
  }
  const int t1 = min(min(p.lens[b], p.max_len), t0 + p.chunk);
  // second operand of the scores: lane (r, g) holds elements 32c + 8g .. +7
  // of query head r (zero for the padding heads r >= GQ)
  u32x4 qop[4];
#pragma unroll
  for (int c = 0; c < 4; c++)
    qop[c] = r < GQ ? *reinterpret_cast<const u32x4*>(p.q + ((size_t)b * p.Hq + h * GQ + r) * kAttnD + 32 * c + 8 * g)
                    : u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  // a step covers positions tb .. tb + 31 (runs tb + 8i, i < 4).  Keys: row
  // r of the first score product is position tb + 8 (r / 4) + r % 4, of the
  // second the same + 4; lane (r, g) loads elements 32c + 8g .. of that
  // row.  Values: lane (r, g) loads element 16c + r of positions tb + 8g ..
  // tb + 8g + 7.  Positions past the range or in a skipped block read block
  // 0 and count as absent (nv = the lane's present positions).
  auto load_step = [&](int tb, u32x4 (&kv)[8], u32x4 (&vv)[8], int& nv) {
    const int gk = (tb - t0) / 8 + (r >> 2);
    const int sk = tb + 8 * (r >> 2) < t1 ? gslab[gk] : -1;
    const size_t krow = sk >= 0 ? (size_t)sk * p.block + goff[gk] + (r & 3) : (size_t)(r & 3);
#pragma unroll
    for (int hf = 0; hf < 2; hf++)
#pragma unroll
      for (int c = 0; c < 4; c++)
        kv[4 * hf + c] = *reinterpret_cast<const u32x4*>(p.kc + (krow + 4 * hf) * kAttnD + 32 * c + 8 * g);
    const int gv = (tb - t0) / 8 + g, tv = tb + 8 * g;
    const int sv = tv < t1 ? gslab[gv] : -1;
    nv = sv >= 0 ? min(8, t1 - tv) : 0;
    const size_t vrow = sv >= 0 ? (size_t)sv * kAttnD * p.block + goff[gv] : 0;
#pragma unroll
    for (int c = 0; c < 8; c++)
      vv[c] = *reinterpret_cast<const u32x4*>(p.vc + vrow + (size_t)(16 * c + r) * p.block);
  };
  // running state of head r: maximum m (scaled), this lane's share l of the
  // denominator, and acc[c][i] = output element 16c + 4g + i
  float m = -INFINITY, l = 0.0f;
  floatx4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; c++) acc[c] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto compute_step = [&](const u32x4 (&kv)[8], u32x4 (&vv)[8], int nv) {
    floatx4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv[c]),
                                                   __builtin_bit_cast(bf16x8_t, qop[c]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv[4 + c]),
                                                   __builtin_bit_cast(bf16x8_t, qop[c]), s1, 0, 0, 0);
    }
    // lane (r, g): scores of head r at positions tb + 8g + k, k = 0..7
    float sc[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sc[i] = i < nv ? s0[i] : -INFINITY;
      sc[4 + i] = 4 + i < nv ? s1[i] : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int k = 1; k < 8; k++) mx = fmaxf(mx, sc[k]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx * p.qscale);
    if (__all(mn == -INFINITY)) return;  // nothing present so far (the same in every lane)
    const float cf = exp2f(m - mn);
    float pr[8], ps = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      pr[k] = exp2f(fmaf(sc[k], p.qscale, -mn));  // 0 when absent
      ps += pr[k];
    }
    l = l * cf + ps;
    m = mn;
    if (__any(cf != 1.0f))
#pragma unroll
      for (int c = 0; c < 8; c++) acc[c] *= cf;
    // absent positions: zero their values too (the slot may hold anything)
    if (__any(nv < 8)) {
      u32x4 keep;
#pragma unroll
      for (int i = 0; i < 4; i++) keep[i] = (2 * i < nv ? 0xFFFFu : 0u) | (2 * i + 1 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int c = 0; c < 8; c++) vv[c] &= keep;
    }
    // probabilities as hi + lo bf16 pairs, position order 0..7
    u32x4 phi, plo;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t a = __float_as_uint(pr[2 * i]), bb = __float_as_uint(pr[2 * i + 1]);
      phi[i] = (a >> 16) | (bb & 0xFFFF0000u);
      const float ra = pr[2 * i] - __uint_as_float(a & 0xFFFF0000u);
      const float rb = pr[2 * i + 1] - __uint_as_float(bb & 0xFFFF0000u);
      plo[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2_t{ra, rb}), bf16x2_t));
    }
#pragma unroll
    for (int c = 0; c < 8; c++) {
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv[c]),
                                                       __builtin_bit_cast(bf16x8_t, phi), acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv[c]),
                                                       __builtin_bit_cast(bf16x8_t, plo), acc[c], 0, 0, 0);
    }
  };
  // two register sets per wave: the next step's loads are in flight while
  // this one is computed (every step issues the same 16 loads, so one
  // count-based wait leaves exactly the newer set outstanding); the wave's
  // step count is known up front, so the loop has one exit
  u32x4 ka[8], va[8], kb[8], vb[8];
  int na, nb;
  constexpr int kStride = 32 * kWaves;
  int tb = t0 + 32 * w;
  const int nsteps = tb < t1 ? (t1 - tb + kStride - 1) / kStride : 0;
  if (nsteps > 0) {
    load_step(tb, ka, va, na);
    int k = 0;
    for (; k + 2 < nsteps; k += 2) {
      load_step(tb + kStride, kb, vb, nb);
      wait_vm<16>();
      compute_step(ka, va, na);
      load_step(tb + 2 * kStride, ka, va, na);
      wait_vm<16>();
      compute_step(kb, vb, nb);
      tb += 2 * kStride;
    }
    // the last one or two steps, nothing more to fetch
    if (nsteps - k == 2) {
      load_step(tb + kStride, kb, vb, nb);
      wait_vm<16>();
      compute_step(ka, va, na);
      wait_vm<0>();
      compute_step(kb, vb, nb);
    } else {
      wait_vm<0>();
      compute_step(ka, va, na);
    }
  }
  // head r's denominator over the 4 lane groups, then the waves merged in
  // LDS, in wave order
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (r < GQ) {
    if (g == 0) {
      sm[w][r] = m;
      sl[w][r] = l;
    }
#pragma unroll
    for (int c = 0; c < 8; c++) *reinterpret_cast<floatx4_t*>(&sacc[w][r][16 * c + 4 * g]) = acc[c];
  }
  __syncthreads();
  const size_t base = ((size_t)b * p.Hq + h * GQ) * p.nsplit + s;
  for (int i = tid; i < GQ * kAttnD; i += kAttnThreads) {
    const int j = i / kAttnD, d = i % kAttnD;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; v++) M = fmaxf(M, sm[v][j]);
    float lt = 0.0f, at = 0.0f;
    if (M != -INFINITY)
#pragma unroll
      for (int v = 0; v < kWaves; v++) {
        const float f = exp2f(sm[v][j] - M);  // 0 for a wave with nothing present
        lt += sl[v][j] * f;
        at += sacc[v][j][d] * f;
      }
    const size_t at_idx = base + (size_t)j * p.nsplit;
    p.part_acc[at_idx * kAttnD + d] = at;
    if (d == 0) {
      p.part_m[at_idx] = M;
      p.part_l[at_idx] = lt;
    }
  }
}

// Merges the ranges of each (sequence, query head): a workgroup per
// (sequence and head, 32 output elements).  The ranges' maxima go through
// LDS as factors exp2(m_s - M); thread (y, x) sums element x over the ranges
// y, y + 8, y + 16, ... in order (16 independent loads at a time, the first
// 16 issued before the maxima are read), and the 8 sums are added in y
// order, so the result does not depend on timing.
constexpr int kMaxSplit = 4096;
constexpr int kMergeCols = 32, kMergeRows = 8;

__global__ __launch_bounds__(kMergeCols * kMergeRows) void attn_combine_kernel(
    const float* __restrict__ part_m, const float* __restrict__ part_l, const float* __restrict__ part_acc,
    int nsplit, float* __restrict__ out) {
  __shared__ float fm[kMaxSplit];
  __shared__ float wmax[kMergeCols * kMergeRows / 64];
  __shared__ float sa[kMergeRows][kMergeCols], sden[kMergeRows];
  const int bq = blockIdx.x, tid = threadIdx.x, x = tid % kMergeCols, y = tid / kMergeCols;
  const int d = blockIdx.y * kMergeCols + x;
  const float* pm = part_m + (size_t)bq * nsplit;
  const float* pl = part_l + (size_t)bq * nsplit;
  const float* pa = part_acc + (size_t)bq * nsplit * kAttnD;
  // the first U of this thread's ranges are loaded before the maxima are
  // known, so that their latency overlaps the reduction
  constexpr int U = 16;
  float v[U], lv[U];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const int sidx = y + u * kMergeRows;
    v[u] = sidx < nsplit ? pa[(size_t)sidx * kAttnD + d] : 0.0f;
    lv[u] = sidx < nsplit ? pl[sidx] : 0.0f;
  }
  float M = -INFINITY;
  for (int s = tid; s < nsplit; s += kMergeCols * kMergeRows) {
    fm[s] = pm[s];
    M = fmaxf(M, fm[s]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & 63) == 0) wmax[tid >> 6] = M;
  __syncthreads();
  M = wmax[0];
#pragma unroll
  for (int i = 1; i < kMergeCols * kMergeRows / 64; i++) M = fmaxf(M, wmax[i]);
  // factors (0 for empty ranges)
  for (int s = tid; s < nsplit; s += kMergeCols * kMergeRows) fm[s] = M == -INFINITY ? 0.0f : exp2f(fm[s] - M);
  __syncthreads();
  float lt = 0.0f, at = 0.0f;
  for (int s0 = y;; s0 += U * kMergeRows) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int sidx = s0 + u * kMergeRows;
      if (sidx < nsplit) {
        lt += lv[u] * fm[sidx];
        at += v[u] * fm[sidx];
      }
    }
    const int next = s0 + U * kMergeRows;
    if (next >= nsplit) break;
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int sidx = next + u * kMergeRows;
      v[u] = sidx < nsplit ? pa[(size_t)sidx * kAttnD + d] : 0.0f;
      lv[u] = sidx < nsplit ? pl[sidx] : 0.0f;
    }
  }
  sa[y][x] = at;
  if (x == 0) sden[y] = lt;
  __syncthreads();
  if (y == 0) {
    float a = 0.0f, l = 0.0f;
#pragma unroll
    for (int i = 0; i < kMergeRows; i++) {
      a += sa[i][x];
      l += sden[i];
    }
    out[(size_t)bq * kAttnD + d] = l > 0.0f ? a / l : 0.0f;
  }
}

}  // namespace

AttnPlan attn_plan(int B, int Hkv, int max_len) {
  // about 512 workgroups over (sequence, KV head, range); ranges of 64 to
  // 1024 positions, a multiple of 64 (so a range spans at most 1024 / block
  // + 2 table entries)
  const int64_t want = std::max<int64_t>(1, 512 / std::max(1, B * Hkv));
  int64_t chunk = (std::max(max_len, 1) + want - 1) / want;
  chunk = std::min<int64_t>(1024, std::max<int64_t>(64, (chunk + 63) / 64 * 64));
  const int nsplit = (int)((std::max(max_len, 1) + chunk - 1) / chunk);
  return AttnPlan{nsplit, (int)chunk};
}

hipError_t launch_decode_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                                   const int32_t* table, const int32_t* lens, int B, int Hq,
                                   int Hkv, int block, int max_blocks, int num_blocks,
                                   int max_len, float* out, float* ws, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const AttnPlan pl = attn_plan(B, Hkv, max_len);
  const size_t nq = (size_t)B * Hq * pl.nsplit;
  AttnParams p{q, kc, vc, table, lens, ws, ws + nq, ws + 2 * nq, Hq, Hkv, block, max_blocks,
               num_blocks, pl.nsplit, pl.chunk, 1.4426950408889634f / sqrtf((float)kAttnD), max_len};
  const dim3 grid(pl.nsplit, Hkv, B);
  switch (Hq / Hkv) {
    case 1: attn_split_kernel<1><<<grid, kAttnThreads, 0, s>>>(p); break;
    case 2: attn_split_kernel<2><<<grid, kAttnThreads, 0, s>>>(p); break;
    case 4: attn_split_kernel<4><<<grid, kAttnThreads, 0, s>>>(p); break;
    case 8: attn_split_kernel<8><<<grid, kAttnThreads, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  attn_combine_kernel<<<dim3(B * Hq, kAttnD / kMergeCols), kMergeCols * kMergeRows, 0, s>>>(
      ws, ws + nq, ws + 2 * nq, pl.nsplit, out);
  return hipGetLastError();
}

}  // namespace moe
