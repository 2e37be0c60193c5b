// route.hip -- S0 router linear layer and S1 top-k routing with combine
// weights, fused with the first half of S2 (per-chunk expert histogram) and
// with the fp16 operand staging of the activations.  Page "Perplexity's
// Lily engine beats MLX by 35% on M5 Max", architecture paragraph: expert
// routing runs on the GPU in the same submission as the rest of the layer.
//
// S0 (only when a router weight is given) is its own kernel (router_kernel):
// LDS-staged bf16 MFMA tiles whose shape follows T, deterministic sums, and
// the fp16 operand copy of x written from the staged slabs, so the routing
// kernel then skips it.
//
// The routing kernel: one workgroup (8 waves) owns a chunk of consecutive
// tokens and walks it in passes of 8, 32 or 64 tokens (64, 16 or 8 lanes
// per token):
//   1. the pass's logits into LDS;
//   2. top-k per token, in (logit descending, index ascending) order: for
//      chunks of at most 8 tokens a wave per token runs a radix select
//      (topk_token); for larger chunks a group of 16 or 8 lanes per token
//      keeps per-lane sorted lists of 64-bit keys (logit image, inverted
//      index) and merges them across the group by bitonic merges
//      (topk_group), all on the VALU, so many tokens proceed at once;
//   3. (whole-layer mode) the chunk's expert histogram (LDS atomics: counts
//      do not depend on order), and x bf16 -> fp16 in the interleaved order
//      the grouped GEMM reads.
#include "scan_scatter.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kLgFloats = 16384;  // LDS logits of one pass (64 KiB)
constexpr int kRouteThreads = 512;

// ------------------------------------------------------------------ S0 ---
// logits[t][e] = sum_h x[t][h] * wr[e][h], fp32 accumulation of the bf16
// products on v_mfma_f32_32x32x16_bf16, and (optionally) the fp16 operand
// copy of x.  A workgroup of 4 waves owns TMB x TEB blocks of 32 tokens x 32
// experts over the whole of H, in slabs of 64.  Per slab its x rows and
// router rows reach LDS by global_load_lds_dwordx4 through a ring of R
// stages (R - 1 slabs in flight, R = 4..16: as deep as 128 KiB of LDS
// allows, since with few workgroups per CU the copies are latency-bound);
// each wave instruction moves 8 rows x 128
// contiguous bytes, the 16-byte chunk c of row r landing at position
// c ^ (r % 8), so the loads are coalesced and the fragment reads free of
// bank conflicts.  With one block the 4 waves take one 16-wide k step of
// every slab each and add their partial tiles in wave order at the end
// (deterministic); with 4 or more blocks each wave owns blocks that share
// its x rows.  The workgroups of expert tile 0 also convert every staged x
// slab to fp16 in operand order for the grouped GEMM, so x is read from
// HBM once.

struct RouterParams {
  const uint16_t* x;   // bf16 [T][H]
  const uint16_t* wr;  // bf16 [E][H]
  const uint16_t* gamma;  // bf16 [H]: the A operand is bf16(x * gamma) (NORM), or nullptr
  float* logits;       // fp32 [ksplit][T][E]: the logits, or partial sums over H / ksplit
  half_t* xh;          // fp16 [T][H] operand copy, or nullptr
  int T, H, E, n_et;   // n_et: expert tiles
  int ksplit;          // H ranges (the grid is token tiles x n_et x ksplit)
};

// Elementwise bf16(a * g) of eight bf16 pairs, rounded to nearest even.
__device__ __forceinline__ u32x4 bf16x8_mul(u32x4 a, u32x4 g) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  typedef float float2_v __attribute__((ext_vector_type(2)));
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float2_v v = {__uint_as_float(a[i] << 16) * __uint_as_float(g[i] << 16),
                        __uint_as_float(a[i] & 0xFFFF0000u) * __uint_as_float(g[i] & 0xFFFF0000u)};
    o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
  }
  return o;
}

// Gamma values one workgroup of the router stages (its range of H).
constexpr int kRouterGamma = 4096;

template <int TMB, int TEB, int R, bool NORM>
__global__ __launch_bounds__(256) void router_kernel(const RouterParams p) {
  constexpr int NBLK = TMB * TEB;
  static_assert(NBLK == 1 || ((TMB == 2 || TMB == 4) && (TEB == 2 || TEB == 4)), "block split");
  constexpr bool KSPLIT = NBLK == 1;            // 4 waves share one block
  // otherwise wave (wm, we) = (w % 2, w / 2) owns block rows MW wm .. and
  // block columns EW we .. (a 2 x 2 grid of waves over the tile)
  constexpr int MW = KSPLIT ? 1 : TMB / 2, EW = KSPLIT ? 1 : TEB / 2;
  constexpr int NBW = MW * EW;                  // blocks per wave
  constexpr int RX = 32 * TMB, RW = 32 * TEB;   // x rows, router rows per stage
  constexpr int STAGE = (RX + RW) * 128;        // bytes per slab
  constexpr int D = (RX + RW) / 32;             // load instructions per wave and slab
  constexpr int X = TMB;                        // operand-copy stores per thread and slab
  static_assert(R >= 3 && (R - 1) * (D + X) < 64, "ring depth within the vmcnt range");
  __shared__ __attribute__((aligned(16))) char ring[R * STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t gam[NORM ? kRouterGamma : 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kz = blockIdx.x % p.ksplit, tile = blockIdx.x / p.ksplit;
  const int tt = tile / p.n_et, et = tile % p.n_et;
  const int t0 = tt * RX, e0 = et * RW;
  const int S = p.H / 64 / p.ksplit, s0 = kz * S;  // this workgroup's slabs s0 .. s0 + S - 1
  float* const out = p.logits + (size_t)kz * p.T * p.E;
  const bool stage_x = p.xh != nullptr && et == 0;  // uniform over the workgroup

  // Load instruction q of this wave moves 8-row group g = wave + 4 q of the
  // stage (x rows first, then router rows; rows past T or E repeat the last
  // valid row and are never stored); lane l moves chunk (l % 8) ^ (l / 8) of
  // row 8 g + l / 8, which lands at position l % 8 of that row.
  const int cl = (lane & 7) ^ (lane >> 3);
  const uint16_t* src[D];
#pragma unroll
  for (int q = 0; q < D; q++) {
    const int r = 8 * (wave + 4 * q) + (lane >> 3);
    src[q] = r < RX ? p.x + (size_t)min(t0 + r, p.T - 1) * p.H + 8 * cl
                    : p.wr + (size_t)min(e0 + r - RX, p.E - 1) * p.H + 8 * cl;
  }
  auto issue = [&](int s, int st) {
    char* base = ring + st * STAGE;
#pragma unroll
    for (int q = 0; q < D; q++) lds_load16(src[q] + 64 * (s0 + s), base + (wave + 4 * q) * 1024);
  };
  // MFMA fragment of the 32 rows from row0 of a stage, k step j of the slab:
  // lane (i, half) holds row row0 + i, elements 16 j + 8 half .. + 7 (usable
  // after lds_wait)
  auto frag = [&](const char* base, int row0, int j) {
    const int r = row0 + (lane & 31), c = 2 * j + (lane >> 5);
    return lds_read16(base + r * 128 + 16 * (c ^ (r & 7)));
  };
  auto mfma = [](u32x4 a, u32x4 b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  };

  floatx16_t acc[NBW];
#pragma unroll
  for (int b = 0; b < NBW; b++) acc[b] = floatx16_t{};
  if constexpr (NORM) {
    // gamma over this workgroup's slabs (128 S bytes <= sizeof gam) into LDS
    // ahead of the ring: every wave's wait for slab 0 also covers these
    // copies, since loads complete in issue order
    const int nb = 128 * S;
    for (int q = wave; 1024 * q < nb; q += 4)
      lds_load16(reinterpret_cast<const char*>(p.gamma + 64 * s0) + min(1024 * q + 16 * lane, nb - 16),
                 reinterpret_cast<char*>(gam) + 1024 * q);
  }
  // NORM: the gamma fragment matching frag(.., j): columns 16 j + 8 half .. + 7
  // of slab s
  auto gfrag = [&](int s, int j) { return lds_read16(gam + 64 * s + 16 * j + 8 * (lane >> 5)); };
#pragma unroll
  for (int j = 0; j < R - 1; j++) issue(min(j, S - 1), j);
  for (int s = 0; s < S; s++) {
    // Slab s has landed once at most the loads (and copy stores) issued after
    // it are outstanding: every load and store completes in issue order.
    // Issued after slab s's loads: the loads of slabs s + 1 .. s + R - 2 and
    // the copy stores of the min(s, R - 1) slabs before s.
    wait_vm_barrier_n<(R - 2) * D, X, R - 1>(stage_x ? min(s, R - 1) : 0);
    issue(min(s + R - 1, S - 1), (s + R - 1) % R);
    const char* base = ring + (s % R) * STAGE;
    if constexpr (KSPLIT) {
      u32x4 a = frag(base, 0, wave), b = frag(base, RX, wave);
      if constexpr (NORM) {
        u32x4 g = gfrag(s, wave);
        lds_wait(a, b);
        lds_tie(g);
        a = bf16x8_mul(a, g);
      } else {
        lds_wait(a, b);
      }
      acc[0] = mfma(a, b, acc[0]);
    } else {
      // every fragment of the slab first, one wait, then the MFMAs
      u32x4 a[4][MW], b[4][EW];
#pragma unroll
      for (int j = 0; j < 4; j++) {
#pragma unroll
        for (int m = 0; m < MW; m++) a[j][m] = frag(base, 32 * (MW * (wave & 1) + m), j);
#pragma unroll
        for (int e = 0; e < EW; e++) b[j][e] = frag(base, RX + 32 * (EW * (wave >> 1) + e), j);
      }
      u32x4 g[4];
      if constexpr (NORM)
#pragma unroll
        for (int j = 0; j < 4; j++) g[j] = gfrag(s, j);
#pragma unroll
      for (int j = 0; j < 4; j++) {
#pragma unroll
        for (int m = 0; m < MW; m++) lds_wait(a[j][m]);
#pragma unroll
        for (int e = 0; e < EW; e++) lds_wait(b[j][e]);
        if constexpr (NORM) lds_wait(g[j]);
      }
      if constexpr (NORM)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
          for (int m = 0; m < MW; m++) a[j][m] = bf16x8_mul(a[j][m], g[j]);
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int m = 0; m < MW; m++)
#pragma unroll
          for (int e = 0; e < EW; e++) acc[m * EW + e] = mfma(a[j][m], b[j][e], acc[m * EW + e]);
    }
    if (stage_x) {
      // exactly X stores per thread, so the wait count above is exact; rows
      // past T hold row T - 1 (clamped load) and rewrite its identical bytes
      u32x4 d[X];
#pragma unroll
      for (int i = 0; i < X; i++) {
        const int r = (tid + 256 * i) >> 3, c = tid & 7;
        d[i] = lds_read16(base + r * 128 + 16 * (c ^ (r & 7)));
      }
#pragma unroll
      for (int i = 0; i < X; i++) lds_wait(d[i]);
#pragma unroll
      for (int i = 0; i < X; i++) {
        const int r = (tid + 256 * i) >> 3, c = tid & 7;
        *reinterpret_cast<uint4*>(p.xh + (size_t)min(t0 + r, p.T - 1) * p.H + 64 * (s0 + s) + 8 * c) =
            bf16x8_to_half_interleaved(make_uint4(d[i][0], d[i][1], d[i][2], d[i][3]));
      }
    }
  }
  wait_vm<0>();  // the ring's last (repeated) loads drain before the end

  // accumulator register i of lane (col, half) is row 8 (i / 4) + 4 half + i % 4
  const int col = lane & 31, half = lane >> 5;
  if constexpr (KSPLIT) {
    static_assert(R * STAGE >= 4 * 32 * 33 * 4, "the wave partials reuse the ring");
    float* red = reinterpret_cast<float*>(ring);
    __syncthreads();  // every wave is done with the ring
#pragma unroll
    for (int i = 0; i < 16; i++) red[wave * 32 * 33 + (8 * (i >> 2) + 4 * half + (i & 3)) * 33 + col] = acc[0][i];
    __syncthreads();
    for (int idx = tid; idx < 32 * 32; idx += 256) {
      const int row = idx >> 5, c2 = idx & 31;
      float v = red[row * 33 + c2];
#pragma unroll
      for (int w = 1; w < 4; w++) v += red[w * 32 * 33 + row * 33 + c2];
      if (t0 + row < p.T && e0 + c2 < p.E) out[(size_t)(t0 + row) * p.E + e0 + c2] = v;
    }
  } else {
#pragma unroll
    for (int m = 0; m < MW; m++)
#pragma unroll
      for (int e2 = 0; e2 < EW; e2++) {
        const int e = e0 + 32 * (EW * (wave >> 1) + e2) + col;
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int t = t0 + 32 * (MW * (wave & 1) + m) + 8 * (i >> 2) + 4 * half + (i & 3);
          if (t < p.T && e < p.E) out[(size_t)t * p.E + e] = acc[m * EW + e2][i];
        }
      }
  }
}

constexpr int kMaxSplit = 8;  // ranges of H the router may sum separately

struct RouterPlan {
  int tm, te, ksplit;
};

// Tile shape: the candidate whose busiest CU moves the fewest bytes
// (rounds of 256 workgroups x bytes per workgroup), more workgroups on ties.
// With the smallest tile and partial sums allowed, H is also split into up
// to 8 ranges while that keeps the grid within two rounds of the chip.
RouterPlan router_plan(int64_t T, int64_t H, int64_t E, bool split) {
  const int cand[4][2] = {{1, 1}, {2, 2}, {2, 4}, {4, 4}};
  int best = 0;
  int64_t best_cost = -1, best_wg = 0;
  for (int c = 0; c < 4; c++) {
    const int64_t wg = ((T + 32 * cand[c][0] - 1) / (32 * cand[c][0])) *
                       ((E + 32 * cand[c][1] - 1) / (32 * cand[c][1]));
    const int64_t cost = ((wg + 255) / 256) * (int64_t)(cand[c][0] + cand[c][1]);
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && wg > best_wg)) {
      best = c;
      best_cost = cost;
      best_wg = wg;
    }
  }
  int ks = 1;
  if (split && best == 0)
    while (ks < kMaxSplit && best_wg * ks * 2 <= 512 && (H / 64) % (2 * ks) == 0) ks *= 2;
  return RouterPlan{cand[best][0], cand[best][1], ks};
}

template <bool NORM>
void launch_router_plan(const RouterPlan& pl, const RouterParams& p, int64_t grid, hipStream_t s) {
  if (pl.tm == 1) router_kernel<1, 1, 9, NORM><<<grid, 256, 0, s>>>(p);  // ring depths: <= 128 KiB
  else if (pl.te == 2) router_kernel<2, 2, 8, NORM><<<grid, 256, 0, s>>>(p);
  else if (pl.tm == 2) router_kernel<2, 4, 5, NORM><<<grid, 256, 0, s>>>(p);
  else router_kernel<4, 4, 4, NORM><<<grid, 256, 0, s>>>(p);
}

// gamma (bf16 [H], or nullptr): the router multiplies bf16(x * gamma); its
// range of H per workgroup must fit kRouterGamma (router_gamma_fits).
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, float* logits, half_t* xh, int T,
                         int H, int E, int ksplit, hipStream_t s, const uint16_t* gamma = nullptr) {
  const RouterPlan pl = router_plan(T, H, E, ksplit > 1);
  if (pl.ksplit != ksplit) return hipErrorInvalidValue;  // the caller sized its buffer for ksplit
  if (gamma && H / ksplit > kRouterGamma) return hipErrorInvalidValue;
  RouterParams p{x, wr, gamma, logits, xh, T, H, E, (E + 32 * pl.te - 1) / (32 * pl.te), ksplit};
  const int64_t grid = (int64_t)((T + 32 * pl.tm - 1) / (32 * pl.tm)) * p.n_et * ksplit;
  if (gamma) launch_router_plan<true>(pl, p, grid, s);
  else launch_router_plan<false>(pl, p, grid, s);
  return hipGetLastError();
}

// -------------------------------------------------------------- S1, S2 ---
struct RouteParams {
  const uint16_t* x;    // bf16 [T][H] (staging)
  const float* logits;  // fp32 [ksplit][T][E]: logits, or partial sums added here
  float* logits_out;    // fp32 [T][E]: the summed logits (ksplit > 1)
  int ksplit;
  int32_t* ids;         // [T][k]
  float* w;             // [T][k]
  half_t* xh;           // fp16 [T][H] staged activations (whole-layer mode)
  int32_t* chunk_hist;  // [nchunks][E] (whole-layer mode)
  int T, H, E, k, chunk_tokens;
  int lpt_log2;         // lanes per token in the top-k (log2)
  bool stage_x;         // write xh here (false when the router kernel did)
  // RMSNorm in front (gamma != nullptr): xh holds the normalised rows, and
  // with scale_logits the logits (the router's sums over bf16(x * gamma))
  // are multiplied by each row's 1 / rms
  const uint16_t* gamma;
  float eps;
  bool scale_logits;
};


// Selection key of expert e with logit v: the order-preserving image of v
// in the high word and ~e in the low word, so a larger key is a larger logit
// or, between equal logits, the lower expert index (the tie rule).  Every
// key of a real expert is above 0, the key of an empty slot.
__device__ __forceinline__ uint64_t sel_key(float v, int e) {
  return ((uint64_t)ordered_bits(v) << 32) | (uint32_t)~e;
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Partner value for butterfly round m of a lane group: lanes 0..m-1 and
// m..2m-1 of every 2m-lane block are paired up.  Up to 8 the pairing runs
// on DPP lane moves inside the VALU (quad permutations for 1 and 2, the
// 8- and 16-lane mirrors for 4 and 8, which pair lane i with 2m - 1 - i);
// beyond, a ds_bpermute exchange with lane ^ m.
template <int M>
__device__ __forceinline__ uint32_t partner32(uint32_t v) {
  const int x = (int)v;
  if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);   // quad_perm 1,0,3,2
  else if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);   // quad_perm 2,3,0,1
  else if constexpr (M == 4) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);  // row_half_mirror
  else if constexpr (M == 8) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true);  // row_mirror
  else return (uint32_t)__shfl_xor(x, M);
}
template <int M>
__device__ __forceinline__ uint64_t partner64(uint64_t v) {
  return ((uint64_t)partner32<M>((uint32_t)(v >> 32)) << 32) | partner32<M>((uint32_t)v);
}


// Compare-exchange: K[i] gets the larger key, K[j] the smaller.
__device__ __forceinline__ void cex(uint64_t& a, uint64_t& b) {
  const uint64_t x = a, y = b;
  const bool gt = x > y;
  a = gt ? x : y;
  b = gt ? y : x;
}

// Sorts a bitonic sequence of L keys into descending order.
template <int L>
__device__ __forceinline__ void bitonic_merge_desc(uint64_t (&K)[L]) {
#pragma unroll
  for (int d = L / 2; d >= 1; d >>= 1)
#pragma unroll
    for (int i = 0; i < L; i++)
      if ((i & d) == 0) cex(K[i], K[i + d]);
}

// Sorts L arbitrary keys into descending order (bitonic sorting network).
template <int L>
__device__ __forceinline__ void bitonic_sort_desc(uint64_t (&K)[L]) {
#pragma unroll
  for (int size = 2; size <= L; size <<= 1)
#pragma unroll
    for (int d = size / 2; d >= 1; d >>= 1)
#pragma unroll
      for (int i = 0; i < L; i++)
        if ((i & d) == 0) {
          if ((i & size) == 0) cex(K[i], K[i + d]);
          else cex(K[i + d], K[i]);
        }
}

// K = the L largest of K and P, both sorted descending: the elementwise
// larger of K and reversed P is a bitonic sequence holding them.
template <int L>
__device__ __forceinline__ void merge_top(uint64_t (&K)[L], const uint64_t (&P)[L]) {
#pragma unroll
  for (int i = 0; i < L; i++) K[i] = K[i] > P[L - 1 - i] ? K[i] : P[L - 1 - i];
  bitonic_merge_desc<L>(K);
}

// Butterfly rounds M, 2M, ... below LPT (unrolled at compile time).
template <int L, int LPT, int M>
__device__ __forceinline__ void butterfly(uint64_t (&K)[L]) {
  if constexpr (M < LPT) {
    uint64_t P[L];
#pragma unroll
    for (int i = 0; i < L; i++) P[i] = partner64<M>(K[i]);
    merge_top<L>(K, P);
    butterfly<L, LPT, 2 * M>(K);
  }
}

// Top-k of one token by a group of LPT consecutive lanes (LPT in {8, 16,
// 64}), sub = lane within the group, l = the token's E logits.
//  1. Lane sub keeps the L largest keys (L >= k) of experts sub, sub + lpt,
//     ..., sorted in descending order: blocks of L keys are sorted by a
//     bitonic network and merged into the list.
//  2. log2(lpt) butterfly rounds: a lane and its partner hold the sorted top
//     L of disjoint expert sets and both merge them into the top L of the
//     union, so after the last round every lane holds the token's top L in
//     (logit descending, index ascending) order: rank j is entry j.
//  3. Softmax over the first k logits, max-subtracted, the denominator
//     summed in rank order; lane sub writes ranks sub, sub + lpt, ... < k
//     and, when hist != nullptr, counts the chosen experts.
// All branches are uniform over the group, so a group never diverges.
template <int L, int LPT>
__device__ __forceinline__ void topk_group(const float* l, int E, int k, int sub, int32_t* ids,
                                           float* w, int* hist) {
  constexpr int lpt = LPT;
  uint64_t K[L];
  for (int base = 0; base < E; base += L * lpt) {
    uint64_t B[L];
#pragma unroll
    for (int i = 0; i < L; i++) {
      const int e = base + sub + lpt * i;
      B[i] = e < E ? sel_key(l[e], e) : 0;
    }
    bitonic_sort_desc<L>(B);
    if (base == 0) {
#pragma unroll
      for (int i = 0; i < L; i++) K[i] = B[i];
    } else {
      merge_top<L>(K, B);
    }
  }
  butterfly<L, LPT, 1>(K);
  const float mx = key_logit(K[0]);
  float a[L];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < L; j++) {
    a[j] = j < k ? expf(key_logit(K[j]) - mx) : 0.0f;
    sum += a[j];  // rank order; the terms past k are 0
  }
#pragma unroll
  for (int j = 0; j < L; j++) {
    if (j < k && (j & (lpt - 1)) == sub) {
      const int e = key_expert(K[j]);
      ids[j] = e;
      w[j] = a[j] / sum;
      if (hist) atomicAdd(&hist[e], 1);
    }
  }
}

// bf16(x * r * gamma), nearest even, of eight bf16 pairs (the normalised
// values, in moe_rmsnorm's order of operations).
__device__ __forceinline__ uint4 norm_bf16x8(uint4 v, uint4 g, float r) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w}, gw[4] = {g.x, g.y, g.z, g.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; i++)
    o[i] = f32_to_bf16_rne(__uint_as_float(w[i] << 16) * r * __uint_as_float(gw[i] << 16)) |
           (f32_to_bf16_rne(__uint_as_float(w[i] & 0xFFFF0000u) * r * __uint_as_float(gw[i] & 0xFFFF0000u))
            << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// The RMSNorm of the RMSNorm step's definition, row by row: 1 / rms of
// tokens [t0, t0 + nt) into rn[0 .. nt), a wave per row.  The same
// arithmetic as moe_rmsnorm (fp32 squares of each lane's 16-byte pieces in
// order, a butterfly over the lanes, 1 / sqrt(mean + eps)), so the
// normalised rows equal its output bit for bit.
// Each wave takes two rows at a time and requests up to 8 pieces per lane
// of both before adding (H <= 4096 in one round trip per row pair).  With
// stage (and H <= 4096), the wave also writes the pair's normalised rows
// to xh from the pieces it holds, so x is read once.
// The calling wave is wave w of NW taking part.
__device__ void norm_rows(const RouteParams& p, int t0, int nt, float* rn, bool stage, int w, int NW) {
  constexpr int B = 8;
  const int lane = threadIdx.x & 63, H8 = p.H / 8;
  const uint4* gam = reinterpret_cast<const uint4*>(p.gamma);
  for (int r = w; r < nt; r += 2 * NW) {
    const int r2 = min(r + NW, nt - 1);  // the pair's second row (a repeat past the pass)
    const uint4* xa = reinterpret_cast<const uint4*>(p.x + (size_t)(t0 + r) * p.H);
    const uint4* xb = reinterpret_cast<const uint4*>(p.x + (size_t)(t0 + r2) * p.H);
    float ss[2] = {0.0f, 0.0f};
    uint4 v[2][B], g[B];
    for (int c0 = 0; c0 < H8; c0 += 64 * B) {
#pragma unroll
      for (int i = 0; i < B; i++) {
        const int c = min(c0 + lane + 64 * i, H8 - 1);
        v[0][i] = xa[c];
        v[1][i] = xb[c];
        if (stage) g[i] = gam[c];
      }
#pragma unroll
      for (int q = 0; q < 2; q++)
#pragma unroll
        for (int i = 0; i < B; i++) {
          if (c0 + lane + 64 * i >= H8) break;
          const uint32_t w[4] = {v[q][i].x, v[q][i].y, v[q][i].z, v[q][i].w};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const float a = __uint_as_float(w[e] << 16), b = __uint_as_float(w[e] & 0xFFFF0000u);
            ss[q] += a * a;
            ss[q] += b * b;
          }
        }
    }
#pragma unroll
    for (int q = 0; q < 2; q++) {
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) ss[q] += __shfl_xor(ss[q], m);
    }
    const float ra = 1.0f / sqrtf(ss[0] / (float)p.H + p.eps), rb = 1.0f / sqrtf(ss[1] / (float)p.H + p.eps);
    if (lane == 0) {
      rn[r] = ra;
      if (r + NW < nt) rn[r + NW] = rb;
    }
    if (stage) {  // H8 <= 64 B: v holds the whole pair
      uint4* oa = reinterpret_cast<uint4*>(p.xh + (size_t)(t0 + r) * p.H);
      uint4* ob = reinterpret_cast<uint4*>(p.xh + (size_t)(t0 + r2) * p.H);
#pragma unroll
      for (int i = 0; i < B; i++) {
        const int c = lane + 64 * i;
        if (c >= H8) break;
        oa[c] = bf16x8_to_half_interleaved(norm_bf16x8(v[0][i], g[i], ra));
        if (r + NW < nt) ob[c] = bf16x8_to_half_interleaved(norm_bf16x8(v[1][i], g[i], rb));
      }
    }
  }
}

// bf16 -> fp16 of tokens [t0, t0 + nt), each 8-element chunk reordered to
// (0,4,1,5,2,6,3,7); with gamma, of the normalised rows (rn: each row's
// 1 / rms).  Loads use clamped indices so that each batch of U is issued
// together.
// Threads [0, nth) take part; the caller's index is tid.
__device__ void stage_rows(const RouteParams& p, int t0, int nt, const float* rn, int tid, int nth) {
  const int H8 = p.H / 8, n = nt * H8;
  const uint4* in = reinterpret_cast<const uint4*>(p.x + (size_t)t0 * p.H);
  const uint4* gam = reinterpret_cast<const uint4*>(p.gamma);
  uint4* out = reinterpret_cast<uint4*>(p.xh + (size_t)t0 * p.H);
  constexpr int U = 8;
  for (int i0 = tid; i0 < n; i0 += nth * U) {
    uint4 v[U], g[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = min(i0 + u * nth, n - 1);
      v[u] = in[i];
      if (gam) g[u] = gam[i % H8];
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = i0 + u * nth;
      if (i < n) out[i] = bf16x8_to_half_interleaved(gam ? norm_bf16x8(v[u], g[u], rn[i / H8]) : v[u]);
    }
  }
}

// Logits of tokens [t0, t0 + nt) into lg[nt][stride] (rows padded so that
// the lane groups of a wave read different LDS banks).  With partial sums
// over ranges of H, they are added in range order (deterministic) and the
// sums also written to logits_out.
// Threads [0, nth) take part; the caller's index is tid.  With
// scale_logits the sums are left unscaled (scale_logits_pass follows).
__device__ void load_logits(const RouteParams& p, int t0, int nt, float* lg, int stride, int tid, int nth) {
  const int n = nt * p.E;
  const size_t part = (size_t)p.T * p.E;
  const float* src = p.logits + (size_t)t0 * p.E;
  // U values per thread and range in one batch: the smallest of 1, 2, 4, 8
  // that covers the pass (batches of 8 beyond), so no thread issues loads
  // past the pass's last value
  auto batches = [&](auto utag) {
    constexpr int U = decltype(utag)::value;
    for (int i0 = tid; i0 < n; i0 += nth * U) {
      // every partial of the batch is loaded before the first add (one round
      // trip); at most kMaxSplit ranges
      float v[kMaxSplit][U];
#pragma unroll
      for (int z = 0; z < kMaxSplit; z++)
        if (z < p.ksplit)
#pragma unroll
          for (int u = 0; u < U; u++) v[z][u] = src[z * part + min(i0 + u * nth, n - 1)];
#pragma unroll
      for (int z = 1; z < kMaxSplit; z++)
        if (z < p.ksplit)
#pragma unroll
          for (int u = 0; u < U; u++) v[0][u] += v[z][u];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int i = i0 + u * nth;
        if (i < n) {
          const int r = i / p.E;
          lg[r * stride + (i - r * p.E)] = v[0][u];
          if (p.ksplit > 1 && !p.scale_logits) p.logits_out[(size_t)t0 * p.E + i] = v[0][u];
        }
      }
    }
  };
  if (n <= nth) batches(std::integral_constant<int, 1>{});
  else if (n <= 2 * nth) batches(std::integral_constant<int, 2>{});
  else if (n <= 4 * nth) batches(std::integral_constant<int, 4>{});
  else batches(std::integral_constant<int, 8>{});
}

// The pass's logits times each row's 1 / rms, in LDS and to logits_out.
__device__ void scale_logits_pass(const RouteParams& p, int t0, int nt, float* lg, int stride, const float* rn) {
  const int n = nt * p.E;
  for (int i = threadIdx.x; i < n; i += kRouteThreads) {
    const int r = i / p.E;
    float& l = lg[r * stride + (i - r * p.E)];
    l = l * rn[r];
    p.logits_out[(size_t)t0 * p.E + i] = l;
  }
}

// One chunk of tokens, in passes of kRouteThreads / LPT tokens (one group of
// LPT lanes per token).  LPT = 64: radix select by a wave, A = ceil(E / 64)
// keys per lane; LPT = 8 or 16: sort-merge top-k, A = L, the list length.
template <bool FULL, int A, int LPT>
__device__ __forceinline__ void route_chunk(const RouteParams& p, int chunk) {
  __shared__ float lg[kLgFloats];
  __shared__ int hist[256];
  __shared__ float rn[kRouteThreads / 8];  // 1 / rms of the pass's rows (gamma)
  const int tid = threadIdx.x;
  constexpr int tp = kRouteThreads / LPT;
  const int stride = p.E + LPT;
  const int grp = tid / LPT, sub = tid % LPT;
  if (FULL && tid < 256) hist[tid] = 0;
  const int c0 = chunk * p.chunk_tokens;
  const int c1 = min(p.T, c0 + p.chunk_tokens);
  for (int t0 = c0; t0 < c1; t0 += tp) {
    const int nt = min(tp, c1 - t0);
    // with rows to stage or normalise, waves 0-3 load the logits while
    // waves 4-7 stage the rows, or (RMSNorm) take the rows' 1 / rms and, for
    // H <= 4096, stage the normalised rows from the same loads; then (with
    // a router weight) the logits are scaled by 1 / rms
    const int wave = tid >> 6;
    const bool stage = FULL && p.stage_x;
    const bool fused_stage = stage && p.gamma && p.H <= 64 * 8 * 8;
    if (!stage && !p.gamma) load_logits(p, t0, nt, lg, stride, tid, kRouteThreads);
    else if (wave < 4) load_logits(p, t0, nt, lg, stride, tid, 256);
    else if (p.gamma) norm_rows(p, t0, nt, rn, fused_stage, wave - 4, 4);
    else stage_rows(p, t0, nt, rn, tid - 256, 256);
    __syncthreads();
    if (p.gamma) {
      if (p.scale_logits) scale_logits_pass(p, t0, nt, lg, stride, rn);
      if (stage && !fused_stage) stage_rows(p, t0, nt, rn, tid, kRouteThreads);
      __syncthreads();
    }
    if (grp < nt)
    {
      int32_t* ids = p.ids + (size_t)(t0 + grp) * p.k;
      float* w = p.w + (size_t)(t0 + grp) * p.k;
      if constexpr (LPT == 64) topk_token<A>(lg + grp * stride, p.E, p.k, ids, w, FULL ? hist : nullptr);
      else topk_group<A, LPT>(lg + grp * stride, p.E, p.k, sub, ids, w, FULL ? hist : nullptr);
    }
    __syncthreads();
  }
  if (FULL && tid < p.E) p.chunk_hist[(size_t)chunk * p.E + tid] = hist[tid];
}

template <bool FULL, int A, int LPT>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const RouteParams p) {
  route_chunk<FULL, A, LPT>(p, blockIdx.x);
}

// Outputs of S2-S5 for the fused single-chunk kernel.
// List length L of the top-k: the power of two in {2, 4, 8, 16} at or above k.
template <bool FULL, int L>
void launch_route_group(const RouteParams& p, int nchunks, hipStream_t s) {
  if (p.lpt_log2 == 3) route_kernel<FULL, L, 8><<<nchunks, kRouteThreads, 0, s>>>(p);
  else route_kernel<FULL, L, 16><<<nchunks, kRouteThreads, 0, s>>>(p);
}

template <bool FULL>
hipError_t launch_route_l(const RouteParams& p, int nchunks, hipStream_t s) {
  if (p.lpt_log2 == 6) {
    switch ((p.E + 63) / 64) {
      case 1: route_kernel<FULL, 1, 64><<<nchunks, kRouteThreads, 0, s>>>(p); break;
      case 2: route_kernel<FULL, 2, 64><<<nchunks, kRouteThreads, 0, s>>>(p); break;
      case 3: route_kernel<FULL, 3, 64><<<nchunks, kRouteThreads, 0, s>>>(p); break;
      default: route_kernel<FULL, 4, 64><<<nchunks, kRouteThreads, 0, s>>>(p); break;
    }
  } else if (p.k <= 2) launch_route_group<FULL, 2>(p, nchunks, s);
  else if (p.k <= 4) launch_route_group<FULL, 4>(p, nchunks, s);
  else if (p.k <= 8) launch_route_group<FULL, 8>(p, nchunks, s);
  else launch_route_group<FULL, 16>(p, nchunks, s);
  return hipGetLastError();
}

// Lanes per token (log2): a wave per token (radix select) for chunks of at
// most 8 tokens; 16 lanes for chunks of up to 32 tokens; otherwise 8
// (passes of 64 tokens) when their logits fit the LDS rows.
int route_lpt_log2(int chunk_tokens, int E) {
  if (chunk_tokens <= 8) return 6;
  if (chunk_tokens <= 32 || (kRouteThreads / 8) * (E + 8) > kLgFloats) return 4;
  return 3;
}

}  // namespace

int route_chunk_tokens(int64_t T) {
  // at least 8 tokens, at most 256 chunks, a multiple of 8
  const int64_t per = (T + 8 * 256 - 1) / (8 * 256);
  return (int)(8 * (per > 1 ? per : 1));
}

int route_chunks(int64_t T) {
  const int ct = route_chunk_tokens(T);
  return (int)((T + ct - 1) / ct);
}

int router_ksplit(int64_t T, int64_t H, int64_t E) { return router_plan(T, H, E, true).ksplit; }

bool route_norm_fits(int64_t T, int64_t H, int64_t E, bool has_router, bool split) {
  return !has_router || H / router_plan(T, H, E, split).ksplit <= kRouterGamma;
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, float* logits, int T, int H, int E,
                        int k, int32_t* ids, float* w, half_t* xh, int32_t* chunk_hist,
                        float* part, hipStream_t s, const uint16_t* gamma, float eps) {
  if (T <= 0) return hipSuccess;
  if (gamma && !xh) return hipErrorInvalidValue;  // the normalised rows exist only as xh
  const int ks = wr && part ? router_ksplit(T, H, E) : 1;
  if (wr) {
    // with RMSNorm the routing kernel writes xh (it knows each row's rms);
    // otherwise the router does, from the slabs it stages anyway
    const hipError_t err = launch_router(x, wr, ks > 1 ? part : logits, gamma ? nullptr : xh, T, H, E, ks,
                                         s, gamma);
    if (err != hipSuccess) return err;
  }
  const int ct = route_chunk_tokens(T);
  RouteParams p{x, ks > 1 ? part : logits, logits, ks, ids, w, xh, chunk_hist, T, H, E, k, ct,
                route_lpt_log2(ct, E), wr == nullptr || gamma != nullptr, gamma, eps,
                wr != nullptr && gamma != nullptr};
  const int n = route_chunks(T);
  return xh ? launch_route_l<true>(p, n, s) : launch_route_l<false>(p, n, s);
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, float* out, int T, int H,
                                int E, int ksplit, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  return launch_router(x, wr, out, nullptr, T, H, E, ksplit, s);
}

}  // namespace moe
