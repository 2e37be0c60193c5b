/*
 * moe_oracle.c -- plain CPU oracle for the 4-bit-weight mixture-of-experts
 * layer.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the CPU
 * baseline leg of the benchmark may call it; the library never does.
 *
 * What it computes (page "Perplexity's Lily engine beats MLX by 35% on M5
 * Max", the architecture paragraph: expert routing, prefix scan, scatter and
 * block map on the GPU, then a grouped GEMM with the 4-bit dequantisation
 * fused in), written as the plain definition of an MoE layer, one step per
 * function, in the order the layer runs:
 *
 *   oracle_router_logits  l[t,e] = sum_h x[t,h] * Wr[e,h]   (fp64 sum, one
 *                         rounding to fp32)
 *   oracle_route          top-k of l[t,:] ranked by (value desc, index asc);
 *                         combine weights = fp32 softmax over the k logits
 *   oracle_build_blocks   expert histogram, exclusive prefix scan, stable
 *                         scatter of (token, choice) pairs into expert order,
 *                         tile block map of at most BM rows per tile
 *   oracle_dequant        w = q * scale + bias, in fp32, one code at a time
 *   oracle_expert_hidden  h = silu(Wg x) * (Wu x)  (SwiGLU), fp64
 *   oracle_expert_down    Wd h, fp64
 *   oracle_ffn            per token, per selected expert:
 *                         y[t] = sum_j w[t,j] * Wd_e (silu(Wg_e x) * Wu_e x)
 *
 * and the two steps an engine runs on either side of the layer (the pages
 * give neither; these are their textbook definitions):
 *
 *   oracle_rmsnorm        x_n[t,h] = bf16(x[t,h] * gamma[h] / sqrt(mean_h x[t,h]^2 + eps)),
 *                         fp64, rounded once to bf16 (nearest, ties to even)
 *   oracle_residual_out   out = bf16(residual + y), fp64 sum rounded once
 *
 * and a second workload the pages' decode gains come from (their
 * architecture paragraph: coalesced key-cache reads, grouped-query packing,
 * a fixed-block cache layout), defined plainly:
 *
 *   oracle_decode_attention  one query token per sequence against its cached
 *                         keys and values: o = softmax(q K^T / sqrt(D)) V per
 *                         query head, the KV head shared by Hq / Hkv query
 *                         heads, keys and values found through a block table
 *                         of fixed-size blocks; fp64
 *
 * Nothing is blocked, fused or reordered beyond those definitions; every
 * weight is dequantised scalar by scalar each time it is used.  Shares no
 * code, header or table with the HIP library.
 *
 * Weight format: a bank is qweight uint32 [E][N][K/8] (code 8w+j of a row in
 * bits 4j..4j+3 of word w), scales and biases bf16 [E][N][K/G]; gate and up
 * have N = I, K = H; down has N = H, K = I.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the parallel loops below will use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static float bf16_bits_to_float(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Router linear layer: l[t,e] = sum_h x[t,h] Wr[e,h], no bias.  bf16 inputs;
 * the products are exact in fp64 and the 2048-term sum is kept in fp64, then
 * rounded once to fp32. */
void oracle_router_logits(const uint16_t* x, const uint16_t* wr, int64_t T, int64_t H,
                          int64_t E, float* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++) {
    for (int64_t e = 0; e < E; e++) {
      double acc = 0.0;
      for (int64_t h = 0; h < H; h++)
        acc += (double)bf16_bits_to_float(x[t * H + h]) * (double)bf16_bits_to_float(wr[e * H + h]);
      logits[t * E + e] = (float)acc;
    }
  }
}

/* Top-k routing.  For each token the k experts with the largest fp32 logit,
 * in order of (logit descending, expert index ascending): k rounds of a
 * selection over every not-yet-taken expert, where a later expert replaces
 * the current best only if its logit is strictly larger (so equal logits
 * keep the lower index).  -inf logits rank last.
 * Combine weights: softmax over the k selected logits in fp32,
 *   m = l[ids[0]],  a_j = expf(l[ids[j]] - m),  S = a_0 + ... + a_{k-1}
 *   (summed in j order),  w_j = a_j / S. */
void oracle_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids,
                  float* weights) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++) {
    const float* l = logits + t * E;
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    float* a = (float*)malloc(sizeof(float) * (size_t)k);
    for (int64_t j = 0; j < k; j++) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; e++) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      ids[t * k + j] = (int32_t)best;
    }
    float m = l[ids[t * k]];
    float s = 0.0f;
    for (int64_t j = 0; j < k; j++) {
      a[j] = expf(l[ids[t * k + j]] - m);
      s += a[j];
    }
    for (int64_t j = 0; j < k; j++) weights[t * k + j] = a[j] / s;
    free(a);
    free(taken);
  }
}

/* Histogram, prefix scan, scatter and block map over the P = T*k pairs
 * p = t*k + j (expert ids[p]).
 *   counts[e]      = #{p : ids[p] = e}
 *   offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e]   (E+1 entries)
 *   scatter: a cursor per expert starts at offsets[e]; pairs are visited in
 *            increasing p and each takes the next slot of its expert, so
 *            sorted_pairs[slot] = p and pair_slot[p] = slot, and within an
 *            expert the slots are in increasing pair (hence token) order.
 *   block map: for e = 0..E-1 with counts[e] > 0, tiles of at most BM rows:
 *            (e, offsets[e] + r, min(BM, counts[e] - r)) for r = 0, BM, 2BM..;
 *            blocks is [num_blocks][3]. */
void oracle_build_blocks(const int32_t* ids, int64_t T, int64_t k, int64_t E, int64_t BM,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                         int32_t* pair_slot, int32_t* blocks, int32_t* num_blocks) {
  const int64_t P = T * k;
  for (int64_t e = 0; e < E; e++) counts[e] = 0;
  for (int64_t p = 0; p < P; p++) counts[ids[p]] += 1;
  offsets[0] = 0;
  for (int64_t e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  for (int64_t e = 0; e < E; e++) cursor[e] = offsets[e];
  for (int64_t p = 0; p < P; p++) {
    int32_t s = cursor[ids[p]]++;
    sorted_pairs[s] = (int32_t)p;
    pair_slot[p] = s;
  }
  free(cursor);
  int32_t nb = 0;
  for (int64_t e = 0; e < E; e++) {
    for (int64_t r = 0; r < counts[e]; r += BM) {
      int64_t rows = counts[e] - r < BM ? counts[e] - r : BM;
      blocks[3 * nb + 0] = (int32_t)e;
      blocks[3 * nb + 1] = (int32_t)(offsets[e] + r);
      blocks[3 * nb + 2] = (int32_t)rows;
      nb++;
    }
  }
  *num_blocks = nb;
}

/* One weight of bank row n, reduction index kk:
 *   q = (qweight[n][kk/8] >> 4*(kk%8)) & 15,  w = q * scale[n][kk/G] + bias[n][kk/G]
 * in fp32 (a single fused multiply-add).  `qrow`, `srow`, `brow` point at
 * row n of one expert. */
float oracle_dequant(const uint32_t* qrow, const uint16_t* srow, const uint16_t* brow,
                     int64_t kk, int64_t G) {
  uint32_t q = (qrow[kk / 8] >> (4 * (kk % 8))) & 15u;
  return fmaf((float)q, bf16_bits_to_float(srow[kk / G]), bf16_bits_to_float(brow[kk / G]));
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU hidden vector of expert e for one activation row xrow (bf16, H):
 *   g_i = sum_h Wg[e][i][h] x[h],  u_i = sum_h Wu[e][i][h] x[h]   (fp64)
 *   h_i = silu(g_i) * u_i,  silu(z) = z / (1 + e^-z). */
static void expert_hidden_row(const uint16_t* xrow, int64_t e, int64_t H, int64_t I, int64_t G,
                              const uint32_t* gq, const uint16_t* gs, const uint16_t* gb,
                              const uint32_t* uq, const uint16_t* us, const uint16_t* ub,
                              double* hout) {
  for (int64_t i = 0; i < I; i++) {
    const int64_t row = e * I + i;
    double g = 0.0, u = 0.0;
    for (int64_t h = 0; h < H; h++) {
      double xv = (double)bf16_bits_to_float(xrow[h]);
      g += (double)oracle_dequant(gq + row * (H / 8), gs + row * (H / G), gb + row * (H / G), h, G) * xv;
      u += (double)oracle_dequant(uq + row * (H / 8), us + row * (H / G), ub + row * (H / G), h, G) * xv;
    }
    hout[i] = silu(g) * u;
  }
}

/* Down projection of expert e: out_n = sum_i Wd[e][n][i] h_i (fp64). */
static void expert_down_row(const double* h, int64_t e, int64_t H, int64_t I, int64_t G,
                            const uint32_t* dq, const uint16_t* ds, const uint16_t* db,
                            double* out) {
  for (int64_t n = 0; n < H; n++) {
    const int64_t row = e * H + n;
    double acc = 0.0;
    for (int64_t i = 0; i < I; i++)
      acc += (double)oracle_dequant(dq + row * (I / 8), ds + row * (I / G), db + row * (I / G), i, G) * h[i];
    out[n] = acc;
  }
}

/* h for a list of (token, expert) pairs: hout[p][i] for p < npairs. */
void oracle_expert_hidden(const uint16_t* x, const int32_t* tokens, const int32_t* experts,
                          int64_t npairs, int64_t H, int64_t I, int64_t G,
                          const uint32_t* gq, const uint16_t* gs, const uint16_t* gb,
                          const uint32_t* uq, const uint16_t* us, const uint16_t* ub,
                          double* hout) {
#pragma omp parallel for schedule(dynamic)
  for (int64_t p = 0; p < npairs; p++)
    expert_hidden_row(x + (int64_t)tokens[p] * H, experts[p], H, I, G, gq, gs, gb, uq, us, ub,
                      hout + p * I);
}

/* Down projection for a list of (hidden row, expert) pairs: out[p][n]. */
void oracle_expert_down(const double* h, const int32_t* experts, int64_t npairs, int64_t H,
                        int64_t I, int64_t G, const uint32_t* dq, const uint16_t* ds,
                        const uint16_t* db, double* out) {
#pragma omp parallel for schedule(dynamic)
  for (int64_t p = 0; p < npairs; p++)
    expert_down_row(h + p * I, experts[p], H, I, G, dq, ds, db, out + p * H);
}

/* The layer output for the tokens listed in `tokens` (ntok of them):
 *   y[r] = sum_{j<k} w[t,j] * Wd_e (silu(Wg_e x_t) * (Wu_e x_t)),  e = ids[t,j],
 * accumulated in fp64 in j order and rounded once to fp32; y is [ntok][H]. */
void oracle_ffn(const uint16_t* x, const int32_t* ids, const float* weights, const int32_t* tokens,
                int64_t ntok, int64_t H, int64_t I, int64_t k, int64_t G,
                const uint32_t* gq, const uint16_t* gs, const uint16_t* gb,
                const uint32_t* uq, const uint16_t* us, const uint16_t* ub,
                const uint32_t* dq, const uint16_t* ds, const uint16_t* db, float* y) {
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < ntok; r++) {
    const int64_t t = tokens[r];
    double* acc = (double*)calloc((size_t)H, sizeof(double));
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    double* o = (double*)malloc(sizeof(double) * (size_t)H);
    for (int64_t j = 0; j < k; j++) {
      const int64_t e = ids[t * k + j];
      expert_hidden_row(x + t * H, e, H, I, G, gq, gs, gb, uq, us, ub, h);
      expert_down_row(h, e, H, I, G, dq, ds, db, o);
      const double w = (double)weights[t * k + j];
      for (int64_t n = 0; n < H; n++) acc[n] += w * o[n];
    }
    for (int64_t n = 0; n < H; n++) y[r * H + n] = (float)acc[n];
    free(o);
    free(h);
    free(acc);
  }
}

/* fp64 -> bf16 bits, round to nearest, ties to even, in one step (no
 * intermediate fp32 rounding).  Finite normal inputs only (zero allowed). */
static uint16_t double_to_bf16_bits(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
  int e;
  frexp(v, &e);                      /* |v| in [2^(e-1), 2^e) */
  const double ulp = ldexp(1.0, e - 8);  /* bf16 keeps 8 significant bits */
  const double r = nearbyint(v / ulp) * ulp;  /* default rounding: nearest even */
  const float f = (float)r;          /* exact: r has at most 9 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* RMSNorm of each row of x (bf16 [T][H]) with gain gamma (bf16 [H]):
 *   r_t = 1 / sqrt(sum_h x[t,h]^2 / H + eps),  x_n[t,h] = x[t,h] * r_t * gamma[h],
 * all in fp64, rounded once to bf16 into out [T][H]. */
void oracle_rmsnorm(const uint16_t* x, const uint16_t* gamma, double eps, int64_t T, int64_t H,
                    uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++) {
    double ss = 0.0;
    for (int64_t h = 0; h < H; h++) {
      const double v = (double)bf16_bits_to_float(x[t * H + h]);
      ss += v * v;
    }
    const double r = 1.0 / sqrt(ss / (double)H + eps);
    for (int64_t h = 0; h < H; h++)
      out[t * H + h] = double_to_bf16_bits((double)bf16_bits_to_float(x[t * H + h]) * r *
                                           (double)bf16_bits_to_float(gamma[h]));
  }
}

/* out[i] = bf16(residual[i] + y[i]) for n values: the bf16 residual and the
 * fp32 layer output added in fp64 and rounded once. */
void oracle_residual_out(const uint16_t* residual, const float* y, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++)
    out[i] = double_to_bf16_bits((double)bf16_bits_to_float(residual[i]) + (double)y[i]);
}

/* Decode attention.  q: bf16 [B][Hq][D]; kc: bf16 [NB][Hkv][BLK][D] and vc:
 * bf16 [NB][Hkv][D][BLK] (block n holds BLK cache positions of one sequence;
 * keys position-major, values element-major); table: int32
 * [B][MB], table[b][i] = the block holding positions i*BLK .. i*BLK+BLK-1 of
 * sequence b; lens: int32 [B].  For each sequence b and query head j (KV head
 * j / (Hq / Hkv)):
 *   s_t = sum_d q[b][j][d] * K_t[d] / sqrt(D)   for t < lens[b],
 *   o[b][j][d] = sum_t exp(s_t - max s) V_t[d] / sum_t exp(s_t - max s),
 * in fp64, rounded once to fp32; a sequence of length 0 gives o = 0. */
void oracle_decode_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                             const int32_t* table, const int32_t* lens, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t D, int64_t BLK, int64_t MB, float* out) {
  const int64_t group = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < B; b++) {
    for (int64_t j = 0; j < Hq; j++) {
      const int64_t h = j / group, L = lens[b];
      double* sc = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
      double mx = -INFINITY;
      for (int64_t t = 0; t < L; t++) {
        const int64_t blk = table[b * MB + t / BLK];
        const uint16_t* krow = kc + ((blk * Hkv + h) * BLK + t % BLK) * D;
        double acc = 0.0;
        for (int64_t d = 0; d < D; d++)
          acc += (double)bf16_bits_to_float(q[(b * Hq + j) * D + d]) * (double)bf16_bits_to_float(krow[d]);
        sc[t] = acc / sqrt((double)D);
        if (sc[t] > mx) mx = sc[t];
      }
      double den = 0.0;
      for (int64_t t = 0; t < L; t++) {
        sc[t] = exp(sc[t] - mx);
        den += sc[t];
      }
      for (int64_t d = 0; d < D; d++) {
        double o = 0.0;
        for (int64_t t = 0; t < L; t++) {
          const int64_t blk = table[b * MB + t / BLK];
          o += sc[t] * (double)bf16_bits_to_float(vc[((blk * Hkv + h) * D + d) * BLK + t % BLK]);
        }
        out[(b * Hq + j) * D + d] = L > 0 ? (float)(o / den) : 0.0f;
      }
      free(sc);
    }
  }
}
