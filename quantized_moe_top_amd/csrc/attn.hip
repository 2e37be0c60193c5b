// attn.hip -- a second workload: decode attention over a block-paged KV
// cache with grouped query heads.  Page "Perplexity's Lily engine beats MLX
// by 35% on M5 Max", architecture paragraph: the decode gains come from
// coalesced key-cache reads, packing the query heads that share a KV head,
// and a fixed-block cache layout.  Here:
//  - the cache is [block][KV head][BLK positions][D] bf16, so the positions
//    of one block and head are one contiguous run, found through a block
//    table (scattered blocks cost nothing extra);
//  - a workgroup owns (sequence, KV head, range of positions) and all GQ
//    query heads of that KV head, so every key and value is read once and
//    used GQ times;
//  - 16 lanes share a position: lane i holds elements 8i..8i+7 of the 128,
//    one 16-byte load, and the 16 lane groups of a workgroup read 16
//    consecutive positions, 4 KiB contiguous per step;
//  - scores are reduced over the 16 lanes on DPP moves (each step adds the
//    same two values in both partners), and each lane group keeps a running
//    maximum, denominator and weighted sum (softmax in base 2, the scores
//    scaled by log2(e) / sqrt(D)), rescaled once per step of four positions;
//    the dot products take bf16 pairs straight from the loads
//    (v_dot2_f32_bf16, fp32 sums);
//  - the 16 lane groups are merged in LDS in fixed order into one partial
//    result per range, and a second launch merges the ranges in fixed order,
//    so the output does not depend on timing.
#include "internal.h"

namespace moe {
namespace {

constexpr int kAttnD = 128;
constexpr int kAttnThreads = 256;  // 16 lane groups of 16
constexpr int kAttnUnroll = 4;     // positions per lane group issued together
constexpr int kAttnTable = 1026;   // block-table entries of one range held in LDS (1024 / block + 2)

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
};

__device__ __forceinline__ float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Sum over the 16 lanes of a row, on DPP: partners lane ^ 1 and lane ^ 2 (quad
// permutations), then the mirrors within 8 and within 16 lanes; each step
// adds the same two values in both partners, so every lane ends with the
// same total.
__device__ __forceinline__ float row16_sum(float v) {
#define MOE_DPP_ADD(ctrl) \
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false))
  MOE_DPP_ADD(0xB1);   // quad_perm 1,0,3,2
  MOE_DPP_ADD(0x4E);   // quad_perm 2,3,0,1
  MOE_DPP_ADD(0x141);  // row_half_mirror
  MOE_DPP_ADD(0x140);  // row_mirror
#undef MOE_DPP_ADD
  return v;
}

template <int GQ>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(const AttnParams p) {
  __shared__ float sm[16][GQ], sl[16][GQ];
  __shared__ float sacc[16][GQ][kAttnD];
  const int tid = threadIdx.x, grp = tid >> 4, sub = tid & 15;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int L = p.lens[b];
  const int t0 = s * p.chunk, t1 = min(L, t0 + p.chunk);
  // this lane's 8 query elements of each of the GQ heads, as bf16 pairs
  uint4 qp[GQ];
#pragma unroll
  for (int j = 0; j < GQ; j++)
    qp[j] = *reinterpret_cast<const uint4*>(p.q + ((size_t)b * p.Hq + h * GQ + j) * kAttnD + 8 * sub);
  float m[GQ], l[GQ], acc[GQ][8];
#pragma unroll
  for (int j = 0; j < GQ; j++) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++) acc[j][e] = 0.0f;
  }
  // the block-table entries of this range, once, in LDS (the loads below
  // then depend on nothing but LDS)
  __shared__ int tbl[kAttnTable];
  const int bi0 = t0 / p.block;
  const int nbi = t1 > t0 ? (t1 - 1) / p.block - bi0 + 1 : 0;  // <= kAttnTable (host plan)
  for (int i = tid; i < nbi; i += kAttnThreads) {
    const int bi = bi0 + i;
    const int blk = bi < p.max_blocks ? p.table[(size_t)b * p.max_blocks + bi] : -1;
    tbl[i] = (blk >= 0 && blk < p.num_blocks) ? blk : -1;
  }
  __syncthreads();
  // one step: positions tb + 16 u of this lane group; past the range or in
  // a malformed block: a valid row is read and not used
  auto load_step = [&](int tb, uint4 (&kv)[kAttnUnroll], uint4 (&vv)[kAttnUnroll], bool (&ok)[kAttnUnroll]) {
#pragma unroll
    for (int u = 0; u < kAttnUnroll; u++) {
      const int t = tb + 16 * u;
      const int blk = t < t1 ? tbl[t / p.block - bi0] : -1;
      ok[u] = blk >= 0;  // uniform over the lane group
      const size_t row = ((size_t)(ok[u] ? blk : 0) * p.Hkv + h) * p.block + (ok[u] ? t % p.block : 0);
      kv[u] = *reinterpret_cast<const uint4*>(p.kc + row * kAttnD + 8 * sub);
      vv[u] = *reinterpret_cast<const uint4*>(p.vc + row * kAttnD + 8 * sub);
    }
  };
  auto compute_step = [&](const uint4 (&kv)[kAttnUnroll], const uint4 (&vv)[kAttnUnroll], const bool (&ok)[kAttnUnroll]) {
    // scores of the step's positions (skipped ones: -inf), then per head one
    // rescale of the running sums for the whole step
    float sc[kAttnUnroll][GQ];
#pragma unroll
    for (int u = 0; u < kAttnUnroll; u++) {
#pragma unroll
      for (int j = 0; j < GQ; j++) {
        // products of bf16 pairs summed in fp32 (v_dot2_f32_bf16)
        float d = dot2_bf16(qp[j].x, kv[u].x, 0.0f);
        d = dot2_bf16(qp[j].y, kv[u].y, d);
        d = dot2_bf16(qp[j].z, kv[u].z, d);
        d = dot2_bf16(qp[j].w, kv[u].w, d);
        sc[u][j] = ok[u] ? row16_sum(d) * p.qscale : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < GQ; j++) {
      float mn = m[j];
#pragma unroll
      for (int u = 0; u < kAttnUnroll; u++) mn = fmaxf(mn, sc[u][j]);
      if (mn == -INFINITY) continue;  // nothing yet (uniform over the lane group)
      const float c = exp2f(m[j] - mn);
      l[j] *= c;
#pragma unroll
      for (int e = 0; e < 8; e++) acc[j][e] *= c;
      m[j] = mn;
#pragma unroll
      for (int u = 0; u < kAttnUnroll; u++) sc[u][j] = exp2f(sc[u][j] - mn);  // 0 when skipped
    }
#pragma unroll
    for (int u = 0; u < kAttnUnroll; u++) {
      const uint32_t vw[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
      float vf[8];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        vf[2 * i] = bf16f(vw[i] & 0xFFFFu);
        vf[2 * i + 1] = bf16f(vw[i] >> 16);
      }
#pragma unroll
      for (int j = 0; j < GQ; j++) {
        if (m[j] == -INFINITY) continue;
        const float pr = sc[u][j];
        l[j] += pr;
#pragma unroll
        for (int e = 0; e < 8; e++) acc[j][e] += pr * vf[e];
      }
    }
  };
  // two register sets: the next step's loads are in flight while this one
  // is computed (every step issues the same 2 * kAttnUnroll loads, so one
  // count-based wait leaves exactly the newer set outstanding)
  uint4 ka[kAttnUnroll], va[kAttnUnroll], kb[kAttnUnroll], vb[kAttnUnroll];
  bool oa[kAttnUnroll], ob[kAttnUnroll];
  constexpr int kStep = 16 * kAttnUnroll;
  int tb = t0 + grp;
  if (t1 > t0) {
    load_step(tb, ka, va, oa);
    while (true) {
      load_step(tb + kStep, kb, vb, ob);
      wait_vm<2 * kAttnUnroll>();
      compute_step(ka, va, oa);
      tb += kStep;
      if (tb - grp >= t1) break;
      load_step(tb + kStep, ka, va, oa);
      wait_vm<2 * kAttnUnroll>();
      compute_step(kb, vb, ob);
      tb += kStep;
      if (tb - grp >= t1) break;
    }
  }
  // merge the 16 lane groups, in group order
  if (sub == 0)
#pragma unroll
    for (int j = 0; j < GQ; j++) {
      sm[grp][j] = m[j];
      sl[grp][j] = l[j];
    }
#pragma unroll
  for (int j = 0; j < GQ; j++)
#pragma unroll
    for (int e = 0; e < 8; e++) sacc[grp][j][8 * sub + e] = acc[j][e];
  __syncthreads();
  const size_t base = ((size_t)b * p.Hq + h * GQ) * p.nsplit + s;
  for (int i = tid; i < GQ * kAttnD; i += kAttnThreads) {
    const int j = i / kAttnD, d = i % kAttnD;
    float M = -INFINITY;
    for (int g = 0; g < 16; g++) M = fmaxf(M, sm[g][j]);
    float lt = 0.0f, at = 0.0f;
    if (M != -INFINITY)
      for (int g = 0; g < 16; g++) {
        const float f = exp2f(sm[g][j] - M);  // 0 for an empty group
        lt += sl[g][j] * f;
        at += sacc[g][j][d] * f;
      }
    const size_t at_idx = base + (size_t)j * p.nsplit;
    p.part_acc[at_idx * kAttnD + d] = at;
    if (d == 0) {
      p.part_m[at_idx] = M;
      p.part_l[at_idx] = lt;
    }
  }
}

// Merges the ranges of each (sequence, query head), in range order: the
// ranges' maxima and denominators go through LDS (loaded in parallel), then
// each thread sums its output element over the ranges with independent loads.
constexpr int kMaxSplit = 4096;

__global__ __launch_bounds__(kAttnD) void attn_combine_kernel(const float* __restrict__ part_m,
                                                              const float* __restrict__ part_l,
                                                              const float* __restrict__ part_acc,
                                                              int nsplit, float* __restrict__ out) {
  __shared__ float fm[kMaxSplit];
  __shared__ float red[kAttnD];
  const int bq = blockIdx.x, d = threadIdx.x;
  const float* pm = part_m + (size_t)bq * nsplit;
  const float* pl = part_l + (size_t)bq * nsplit;
  const float* pa = part_acc + (size_t)bq * nsplit * kAttnD;
  float M = -INFINITY;
  for (int s = d; s < nsplit; s += kAttnD) {
    fm[s] = pm[s];
    M = fmaxf(M, fm[s]);
  }
  red[d] = M;
  __syncthreads();
  M = -INFINITY;
  for (int i = 0; i < kAttnD; i++) M = fmaxf(M, red[i]);
  // factors exp2(m_s - M) (0 for empty ranges), and the denominator in range order
  for (int s = d; s < nsplit; s += kAttnD) fm[s] = M == -INFINITY ? 0.0f : exp2f(fm[s] - M);
  __syncthreads();
  float lt = 0.0f, at = 0.0f;
  constexpr int U = 8;
  for (int s0 = 0; s0 < nsplit; s0 += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = s0 + u < nsplit ? pa[(size_t)(s0 + u) * kAttnD + d] : 0.0f;
#pragma unroll
    for (int u = 0; u < U; u++)
      if (s0 + u < nsplit) {
        lt += pl[s0 + u] * fm[s0 + u];
        at += v[u] * fm[s0 + u];
      }
  }
  out[(size_t)bq * kAttnD + d] = lt > 0.0f ? at / lt : 0.0f;
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
               num_blocks, pl.nsplit, pl.chunk, 1.4426950408889634f / sqrtf((float)kAttnD)};
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
  attn_combine_kernel<<<B * Hq, kAttnD, 0, s>>>(ws, ws + nq, ws + 2 * nq, pl.nsplit, out);
  return hipGetLastError();
}

}  // namespace moe
