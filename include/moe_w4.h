/*
 * moe_w4.h -- C ABI of libmoe_w4.so: the mixture-of-experts layer of a
 * single-model inference engine with 4-bit weights, for one AMD Instinct
 * MI355X (gfx950).
 *
 * The layer follows the page "Perplexity's Lily engine beats MLX by 35% on
 * M5 Max" (the architecture paragraph): expert routing, a prefix scan over
 * the expert histogram, a scatter of tokens into expert order and a tile
 * block map are built on the GPU in one submission, then a grouped expert
 * GEMM dequantises the 4-bit weights inside the kernel so that expanded
 * 16-bit weights never reach memory.  SwiGLU and a routing-weighted combine
 * finish the layer.
 *
 * Conventions (every entry point):
 *  - Pointers named as device pointers must be device memory of the current
 *    HIP device; everything is contiguous and row-major.  The caller owns
 *    every buffer, workspaces included; the library allocates nothing, frees
 *    nothing, never synchronises and never reads device memory on the host.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls only
 *    enqueue work on it and return; results are ready when the stream is.
 *  - Errors: a negative moe_status.  Argument errors are detected on the host
 *    before anything is enqueued, and leave every output untouched; a failed
 *    launch returns MOE_ERR_HIP.  moe_last_error() gives a thread-local
 *    message for the last failing call of the calling thread.  Device faults
 *    surface at the caller's next synchronisation.
 *  - T = 0 is valid and enqueues nothing.
 *  - Supported sizes: 1 <= E <= 256, 1 <= top_k <= min(E, 16), group size
 *    G in {32, 64, 128}; H % 256 == 0, I % 128 == 0, H % G == 0, I % G == 0;
 *    T * top_k < 2^31.  Pointers to packed weights, activations, h, outputs
 *    and workspaces must be 16-byte aligned.
 *  - Logits may contain -inf (never selected while top_k finite logits
 *    exist); NaN logits give unspecified routing.
 *  - Activations x are carried in fp16 inside the grouped GEMM: |x| must
 *    stay below 65504 (bf16 values beyond it have no fp16 form), and values
 *    below 2^-14 in magnitude keep fewer bits (fp16 subnormals).  The hidden
 *    vector h between the two GEMMs carries a power-of-two exponent per row
 *    and 16 columns (moe_w4_h_exp_bytes), so it has no such limit.
 *
 * Notation: T tokens, H hidden size, I expert intermediate size, E experts,
 * top_k experts per token, G quantisation group size, P = T * top_k
 * (token, choice) pairs, pair p = t * top_k + j.
 */
#ifndef MOE_W4_H
#define MOE_W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* sizes negative or inconsistent */
  MOE_ERR_UNSUPPORTED = -3, /* valid but outside the supported sizes above */
  MOE_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = -5,   /* workspace smaller than the query returns */
  MOE_ERR_HIP = -6          /* a HIP launch failed */
} moe_status;

/* Static description of a status code (never NULL). */
const char* moe_status_string(int status);
/* Thread-local detail of the calling thread's last failed call ("" if none). */
const char* moe_last_error(void);
/* Library version string. */
const char* moe_version(void);

/* Layer sizes. */
typedef struct {
  int32_t T, H, I, E, top_k, group_size;
} moe_dims;

/* One bank of 4-bit weights for all E experts, device pointers.
 *  qweight: uint32 [E][N][K/8]; code k' = 8w + j of row n is bits 4j..4j+3
 *           of word w (lowest nibble first), an unsigned value q in 0..15.
 *  scales, biases: bf16 bits [E][N][K/G]; group g covers k' in [gG, gG+G).
 *  Weight W[e][n][k'] = q * scale[e][n][k'/G] + bias[e][n][k'/G].
 * gate and up banks have N = I, K = H; the down bank has N = H, K = I. */
typedef struct {
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint16_t* biases;
} moe_w4_bank;

/* ------------------------------------------------------------ weight pack --
 * The compute kernels read each bank in a tile-major layout, made once from
 * the row-major bank above by moe_w4_pack (load time, not part of a layer
 * call; page "Perplexity's Lily beats MLX by 1.35x by doing one thing:
 * single-model Rust/Metal engines", section "Why one model on one chip is
 * faster": the weights are laid out in the order the kernels read fastest).
 *  words: uint32 [E][N/128][K/64][4 blocks][32 columns][2 halves][4 words]:
 *         for column 128c + 32u + cc (chunk c, block u) and half h of slab s,
 *         the four row-major words holding codes 64s + 32h .. 64s + 32h + 31
 *         (same nibble order), each word rotated left by 5 bits; each chunk
 *         is one contiguous 4 KiB run per slab.
 *  sb:    uint32 [E][N/128][K/G][128 columns], then a tail.  Each expert's
 *         scales and biases are first multiplied by a power of two 2^c
 *         (exact), the one that puts the expert's largest |bias| +
 *         32 |scale| in [2^13, 2^14) (|c| <= 100): every fp16 value of the
 *         dequantisation is then a normal number well below overflow,
 *         whatever the range of the bank.  Word: s' = 2^c scale as fp16 in
 *         the low 16 bits; in the high 16 bits b' - 32 s' (b' = 2^c bias)
 *         when that is an fp16 value for every group of the expert (an
 *         "exact" expert, e.g. bias = -8 * scale: the kernels form
 *         q s' + b' with one rounding), else b' itself (a "general" expert:
 *         q s' is rounded, then b' added and rounded).  Tail, after the
 *         E * N * K/G words: float 2^-c [E], then uint32 general [E] (1 for
 *         a general expert), zero-padded to 16 bytes.  The kernels multiply
 *         their fp32 sums by 2^-c.  Scales and biases must be finite.
 * Requires N % 128 == 0, K % 128 == 0, G in {32, 64, 128}, K % G == 0. */
typedef struct {
  const uint32_t* words;
  const uint32_t* sb;
} moe_w4_packed;

/* Byte sizes of the two packed buffers of one bank, sb with its tail
 * (host-only; 0 for unsupported sizes). */
size_t moe_w4_packed_words_bytes(int32_t E, int32_t N, int32_t K);
size_t moe_w4_packed_sb_bytes(int32_t E, int32_t N, int32_t K, int32_t group_size);
/* Packs `src` (device, row-major) into words / sb (device buffers of the
 * sizes above, 16-byte aligned, owned by the caller) on `stream`. */
int moe_w4_pack(const moe_w4_bank* src, int32_t E, int32_t N, int32_t K, int32_t group_size,
                uint32_t* words, uint32_t* sb, void* stream);

/* One layer's weights (device pointers), banks packed by moe_w4_pack. */
typedef struct {
  moe_dims dims;
  const uint16_t* router_weight; /* bf16 [E][H], or NULL when logits are given */
  moe_w4_packed gate, up, down;
} moe_layer;

/* ------------------------------------------------------------------ S0, S1 --
 * Expert routing.
 * If router_weight != NULL, first computes the router linear layer
 *   logits[t][e] = sum_h x[t][h] * router_weight[e][h]
 * (bf16 inputs, fp32 accumulation, no bias) into `logits`; otherwise `logits`
 * is an input and `x` may be NULL.  Then, per token, selects the top_k
 * experts by (logit descending, expert index ascending) into
 * topk_ids[t][j] (j = 0 is the largest) and writes the combine weights
 *   topk_weights[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0)   (fp32),
 * the softmax over the top_k selected logits.
 * Device pointers: x bf16 [T][H]; router_weight bf16 [E][H]; logits fp32
 * [T][E]; topk_ids int32 [T][top_k]; topk_weights fp32 [T][top_k].
 * With a router weight, H must be a positive multiple of 128.  The caller
 * owns every buffer; nothing is allocated.  Errors (before anything is
 * enqueued): MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGN;
 * MOE_ERR_HIP for a failed launch.
 * Source: page "Perplexity's Lily engine beats MLX by 35% on M5 Max",
 * architecture paragraph (expert routing runs on the GPU in the layer's one
 * submission), and page "Perplexity's Lily beats MLX by 1.35x by doing one
 * thing: single-model Rust/Metal engines", section "Why one model on one
 * chip is faster" (the routing of one MoE model, hardcoded).  The pages do
 * not define the selection itself; top-k with the lower index on ties and a
 * softmax over the chosen logits is the plainest reading. */
int moe_route(const uint16_t* x, const uint16_t* router_weight, float* logits, int32_t T,
              int32_t H, int32_t E, int32_t top_k, int32_t* topk_ids, float* topk_weights,
              void* stream);

/* ----------------------------------------------------------------- S2 - S5 --
 * Upper bound on the number of tiles of the block map (host-only):
 *   floor(P / block_m) + min(E, P). */
int64_t moe_max_blocks(int32_t T, int32_t top_k, int32_t E, int32_t block_m);
/* Bytes of workspace moe_build_blocks needs (host-only). */
size_t moe_build_blocks_workspace_bytes(int32_t T, int32_t top_k, int32_t E);

/* Expert histogram, prefix scan, scatter and tile block map, all on the GPU
 * with no host round trip.  Input topk_ids int32 [T][top_k] (values < E).
 * Outputs (device, int32):
 *   counts[E]          number of pairs routed to each expert
 *   offsets[E + 1]     exclusive prefix sum of counts; offsets[E] = P
 *   sorted_pairs[P]    slot -> pair; the slots of expert e are
 *                      [offsets[e], offsets[e+1]) in increasing pair order
 *                      (a stable counting sort, deterministic)
 *   pair_slot[P]       pair -> slot (the inverse permutation)
 *   blocks[max][3]     tiles (expert, first slot, rows), experts ascending,
 *                      rows <= block_m, none for empty experts; entries past
 *                      num_blocks are unspecified
 *   num_blocks[1]      number of tiles written
 * block_m >= 1.  workspace: device, >= moe_build_blocks_workspace_bytes,
 * owned by the caller.  Ids outside [0, E) are not counted and get no slot.
 * Errors (before anything is enqueued): MOE_ERR_NULL, MOE_ERR_SHAPE,
 * MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE; MOE_ERR_HIP for a failed launch.
 * Source: page "Perplexity's Lily engine beats MLX by 35% on M5 Max",
 * architecture paragraph: the prefix scan, the scatter and the block map
 * stay on the GPU inside the one submission of the layer (credited there
 * with +89% at 512 tokens). */
int moe_build_blocks(const int32_t* topk_ids, int32_t T, int32_t top_k, int32_t E,
                     int32_t block_m, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                     int32_t* pair_slot, int32_t* blocks, int32_t* num_blocks, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ S6, S7 --
 * Grouped W4 GEMM over the block map, dequantisation fused (the packed codes
 * are expanded in registers only).
 *
 * MOE_GEMM_GATE_UP_SWIGLU: for every slot s of every tile (expert e), with
 *   token t = sorted_pairs[s] / top_k,
 *     g = W_gate[e] x[t],  u = W_up[e] x[t],  h[s][n] = silu(g_n) * u_n
 *   silu(z) = z / (1 + exp(-z)); a = x bf16 [T][K]; N = I, K = H; bank0 =
 *   gate, bank1 = up.  h is written as out = h16 fp16 [P][N] and h_exp:
 *     h[s][n] = h16[s][n] * 2^h_exp[s][n / 16]
 *   h16 in operand order: within every run of 8 columns 8c..8c+7 the stored
 *   order is (8c+0, 8c+4, 8c+1, 8c+5, 8c+2, 8c+6, 8c+3, 8c+7).  h_exp is
 *   int8 [P][N / 16] (16-byte padded), then one int32 per tile of the block
 *   map, nonzero when a row of the tile has a nonzero exponent.  An exponent
 *   is 0 unless the 16-column block's largest |h| is at least 2^15, or below
 *   2^-10 and not 0: then the block is scaled so that its largest |h| lies in
 *   [2^14, 2^15).
 * MOE_GEMM_DOWN: for every slot s of every tile (expert e), pair
 *   p = sorted_pairs[s],
 *     out[s][n] = topk_weights[p] * (W_down[e] h[s])_n
 *   a = h16 fp16 [P][K] (slot order, operand order) and h_exp as written by
 *   the gate/up mode with the same block map; out = y_sorted fp32 [P][N];
 *   N = H, K = I; bank0 = down; bank1 unused.
 * T <= 8 runs a bandwidth-bound GEMV-style kernel that reads each touched
 * expert's packed rows once; larger T runs fp16 MFMA tiles of block_m rows
 * (block_m in {32, 64, 128}, equal to the block map's).  K % 128 == 0.
 * Slots outside every tile are not written.  workspace: device, >=
 * moe_w4_grouped_gemm_workspace_bytes(args).  h_exp: device, 16-byte
 * aligned, >= moe_w4_h_exp_bytes(T, top_k, E, I, block_m) bytes (both
 * modes).  All buffers are the caller's.  Errors (before anything is
 * enqueued): MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGN,
 * MOE_ERR_WORKSPACE; MOE_ERR_HIP for a failed launch.
 * Source: page "Perplexity's Lily engine beats MLX by 35% on M5 Max",
 * architecture paragraph: the grouped expert GEMM with the 4-bit
 * dequantisation fused in, so expanded 16-bit weights never reach memory
 * (credited there with +77.4% prefill); page "Perplexity's Lily beats MLX by
 * 1.35x by doing one thing: single-model Rust/Metal engines", section "Why
 * one model on one chip is faster": tiles picked for the model's exact
 * shapes. */
typedef enum { MOE_GEMM_GATE_UP_SWIGLU = 0, MOE_GEMM_DOWN = 1 } moe_gemm_mode;

typedef struct {
  int32_t mode;                /* moe_gemm_mode */
  int32_t T, top_k, E;         /* P = T * top_k rows */
  int32_t N, K, group_size;
  int32_t block_m;
  const void* a;               /* see the modes above */
  moe_w4_packed bank0, bank1;  /* packed by moe_w4_pack */
  const int32_t* sorted_pairs; /* [P] */
  const float* topk_weights;   /* [P], MOE_GEMM_DOWN only */
  const int32_t* blocks;       /* [max_blocks][3] */
  const int32_t* num_blocks;   /* [1] */
  void* out;
  void* workspace;
  size_t workspace_bytes;
  void* h_exp;                 /* h's exponents and tile flags (see the modes); device */
  size_t h_exp_bytes;
} moe_w4_gemm_args;

size_t moe_w4_grouped_gemm_workspace_bytes(const moe_w4_gemm_args* args);
/* Bytes of h_exp for P = T * top_k slots, I = h's columns and the block map
 * of block_m rows per tile: round16(P * I / 16) + 4 * moe_max_blocks(...). */
size_t moe_w4_h_exp_bytes(int32_t T, int32_t top_k, int32_t E, int32_t I, int32_t block_m);
int moe_w4_grouped_gemm(const moe_w4_gemm_args* args, void* stream);

/* -------------------------------------------------------------- whole layer --
 * y[t] = sum_j topk_weights[t][j] * W_down[e] (silu(W_gate[e] x[t]) * W_up[e] x[t]),
 * e = topk_ids[t][j], summed in j order in fp32 (S8, deterministic).
 * Runs S0 (when layer->router_weight != NULL; router_logits must then be
 * NULL) or takes router_logits fp32 [T][E], then S1 - S8 on one stream with
 * no host round trip.  x bf16 [T][H]; y fp32 [T][H] (overwritten).
 * info (host struct, may be NULL) receives the block size used and device
 * pointers into the workspace where the routing structures were written.
 * workspace: device, 256-byte aligned, >= moe_ffn_workspace_bytes(&layer->dims,
 * has_router), owned by the caller (its contents are valid until it is
 * reused).  Errors (before anything is enqueued): MOE_ERR_NULL,
 * MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE;
 * MOE_ERR_HIP for a failed launch.
 * Source: page "Perplexity's Lily engine beats MLX by 35% on M5 Max",
 * architecture paragraph: routing, prefix scan, scatter and block map, then
 * the grouped GEMMs with fused dequantisation, all in one GPU submission.
 * SwiGLU and the routing-weighted sum are the standard MoE expert and
 * combine; the pages name the model family, not these formulas. */
typedef struct {
  int32_t block_m;
  int32_t path;                 /* 0 = MFMA tiles, 1 = GEMV (T <= 8) */
  const float* logits;          /* [T][E] (the input, or the router output) */
  const int32_t* topk_ids;      /* [T][top_k] */
  const float* topk_weights;    /* [T][top_k] */
  const int32_t* counts;        /* [E] */
  const int32_t* offsets;       /* [E + 1] */
  const int32_t* sorted_pairs;  /* [P] */
  const int32_t* pair_slot;     /* [P] */
  const int32_t* blocks;        /* [max_blocks][3] */
  const int32_t* num_blocks;    /* [1] */
  const uint16_t* h;            /* h16 fp16 [P][I], slot order, operand order */
  const uint8_t* y_sorted;      /* [P][H] weighted, slot order, y_sorted_bytes
                                   per value: 4 = fp32 (path 1); 2 = int16
                                   mantissas q (path 0), value = q * 2^E with E
                                   = y_sorted_exp[s][n / 16]: block floating
                                   point, each block's largest |value| in
                                   [2^14, 2^15) * 2^E (relative error <= 2^-16
                                   for it, absolute <= 2^(E-1) for every value;
                                   E = -128 for an all-zero block) */
  int32_t y_sorted_bytes;
  const int8_t* h_exp;          /* [P][I / 16]: h = h16 * 2^h_exp (see S6 above) */
  const int8_t* y_sorted_exp;   /* [P][H / 16] on path 0, NULL on path 1 */
} moe_route_info;

/* Tile rows moe_ffn_forward uses for these sizes (host-only). */
int32_t moe_ffn_block_m(const moe_dims* dims);
size_t moe_ffn_workspace_bytes(const moe_dims* dims, int32_t has_router);
int moe_ffn_forward(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                    float* y, moe_route_info* info, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ------------------------------------------- either side of the layer --
 * The steps a decoder block runs around the MoE layer, so that the layer
 * drops into an engine (the pages describe the layer only; these are the
 * textbook definitions).
 *
 * moe_rmsnorm: RMSNorm of the activations,
 *   out[t][h] = bf16(x[t][h] * gamma[h] / sqrt(mean_h x[t][h]^2 + eps)),
 * computed in fp32 and rounded to nearest even (an fp64 reference rounded
 * once agrees except, rarely, by one bf16 unit).  x, out: device bf16 [T][H],
 * 16-byte aligned, out not overlapping x; gamma: device bf16 [H], 16-byte
 * aligned; H % 8 == 0, H > 0; T >= 0 (T = 0: nothing enqueued).  Enqueued on
 * stream, nothing allocated.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE,
 * MOE_ERR_UNSUPPORTED (H % 8), MOE_ERR_ALIGN, MOE_ERR_HIP. */
int moe_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int32_t T, int32_t H,
                uint16_t* out, void* stream);

/* moe_ffn_forward_io: moe_ffn_forward with the steps around it.
 *  - io->norm_weight (bf16 [H], or NULL): the layer runs on the RMS-
 *    normalised rows x_n = bf16(x * r * gamma), r = 1 / sqrt(mean x^2 +
 *    io->norm_eps), computed as moe_rmsnorm computes them.  Where x is
 *    staged anyway the normalisation is folded in (no launch of its own): at
 *    T > 8 in the routing kernel, and at T <= 8 with logits given in the
 *    gate/up launch; otherwise moe_rmsnorm runs first into the workspace.
 *    At T > 8 with a router weight, the router sums r * bf16(x * gamma) * wr
 *    (r applied after the sum), which is within 1.5 bf16 units of x_n per
 *    term; the logits it returns in `info` are the ones routed;
 *  - io->out (bf16 [T][H], or NULL; needs io->residual, bf16 [T][H]): also
 *    out = bf16(residual + y), fp32 sum rounded to nearest even, written by
 *    the same launch that writes y.  y (fp32) is always written.
 * All device pointers, 16-byte aligned.  io == NULL behaves as
 * moe_ffn_forward.  workspace: >= moe_ffn_io_workspace_bytes (room for the
 * normalised activations after moe_ffn_forward's workspace).  Errors as
 * moe_ffn_forward, plus MOE_ERR_NULL (out without residual) and MOE_ERR_ALIGN. */
typedef struct {
  const uint16_t* norm_weight;
  float norm_eps;
  const uint16_t* residual;
  uint16_t* out;
} moe_ffn_io;
size_t moe_ffn_io_workspace_bytes(const moe_dims* dims, int32_t has_router);
int moe_ffn_forward_io(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                       float* y, const moe_ffn_io* io, moe_route_info* info, void* workspace,
                       size_t workspace_bytes, void* stream);

/* -------------------------------------------------- decode attention --
 * A second workload, the one the pages' decode gains come from (page
 * "Perplexity's Lily engine beats MLX by 35% on M5 Max", architecture
 * paragraph: coalesced key-cache reads, grouped-query packing, a
 * fixed-block cache layout).  One query token per sequence:
 *   o[b][j] = softmax_t(q[b][j] . K_t / sqrt(D)) V  over t < seq_lens[b],
 * the KV head of query head j being j / (Hq / Hkv); a sequence of length 0
 * gives o = 0.  Products of bf16 values summed in fp32 (the softmax
 * weights enter the value sums within 2^-16 of their fp32 value); ranges of
 * positions merged in fixed order (deterministic).
 *   q:           device bf16 [B][Hq][D]
 *   kcache:      device bf16 [num_blocks][Hkv][block][D] (position-major)
 *   vcache:      device bf16 [num_blocks][Hkv][D][block] (element-major);
 *                block n of either holds block positions of one sequence
 *   block_table: device int32 [B][max_blocks]: entry i of sequence b is the
 *                block holding its positions i*block .. i*block+block-1;
 *                entries outside [0, num_blocks) are skipped, never read
 *                through
 *   seq_lens:    device int32 [B], each <= max_blocks*block; a length
 *                above max_len is taken as max_len (positions at or past
 *                max_len are never visited)
 *   out:         device fp32 [B][Hq][D]
 *   workspace:   device, >= moe_decode_attention_workspace_bytes(B, Hq,
 *                Hkv, max_len), 16-byte aligned
 * Supported: D == 128; Hq % Hkv == 0 with Hq / Hkv in {1, 2, 4, 8}; block a
 * multiple of 8; all pointers 16-byte aligned.  Enqueued on stream; nothing allocated.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGN,
 * MOE_ERR_WORKSPACE, MOE_ERR_HIP. */
size_t moe_decode_attention_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_len);
int moe_decode_attention(const uint16_t* q, const uint16_t* kcache, const uint16_t* vcache,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t block, int32_t max_blocks,
                         int32_t num_blocks, int32_t max_len, float* out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ------------------------------------------------------ per-stage timing --
 * The same layer as moe_ffn_forward (identical kernels and results), with a
 * timing event recorded on `stream` at every stage boundary, so that a
 * caller can measure each kernel on the stream it runs on.
 * stage_events: host array of MOE_NUM_STAGES + 1 hipEvent_t handles created
 * by the caller (NULL entries are skipped); events[i] is recorded just
 * before stage i is enqueued and events[MOE_NUM_STAGES] after the last.
 * The elapsed time between events[i] and events[i+1] is stage i.  The
 * library only records the events; the caller owns, synchronises and
 * destroys them.  A NULL stage_events returns MOE_ERR_NULL. */
typedef enum {
  MOE_STAGE_ROUTE = 0,        /* S0 router linear layer (when present), S1 top-k, per-chunk
                                 expert histograms, activations to the fp16 operand layout */
  MOE_STAGE_BUILD_BLOCKS = 1, /* S2 - S5 totals, scan, block map, stable scatter */
  MOE_STAGE_GATE_UP = 2,      /* S6 gate/up grouped GEMM + SwiGLU (S9 at T <= 8) */
  MOE_STAGE_DOWN = 3,         /* S7 down grouped GEMM x routing weight (S9 at T <= 8) */
  MOE_STAGE_COMBINE = 4,      /* S8 combine */
  MOE_NUM_STAGES = 5
} moe_stage;

int moe_ffn_forward_timed(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                          float* y, moe_route_info* info, void* workspace, size_t workspace_bytes,
                          void* const* stage_events, void* stream);

/* ------------------------------------------- ablation: host block map --
 * The same layer as moe_ffn_forward (same kernels, same results, bit for
 * bit), except that S2-S5 take a host round trip, the design the pages'
 * single-submission pipeline replaces (page "Perplexity's Lily engine
 * beats MLX by 35% on M5 Max", architecture paragraph): after S1 the
 * per-chunk expert histograms are copied to host_pinned and the stream is
 * synchronised; the host computes the counts, the offsets, each chunk's
 * first slot per expert and the block map, and uploads them; the device
 * then only runs the stable scatter, and the GEMMs are launched with the
 * exact tile count.  For measuring that design only; it blocks the calling
 * thread and cannot be captured in a graph.
 * host_pinned: pinned host memory (hipHostMalloc) of at least
 * moe_ffn_host_blockmap_ints(&layer->dims) int32; it is read by the uploads
 * until the stream passes them, so the caller leaves it alone until then.
 * T <= 8 (the GEMV path) returns MOE_ERR_UNSUPPORTED. */
size_t moe_ffn_host_blockmap_ints(const moe_dims* dims);  /* 0 if unsupported */
int moe_ffn_forward_host_blockmap(const moe_layer* layer, const uint16_t* x,
                                  const float* router_logits, float* y, moe_route_info* info,
                                  void* workspace, size_t workspace_bytes, int32_t* host_pinned,
                                  size_t host_ints, void* stream);

/* ------------------------------------------- ablation: unfused dequant --
 * The same layer with the 4-bit dequantisation taken out of the grouped
 * GEMMs, the design the pages' fused GEMM replaces (page "Perplexity's Lily
 * engine beats MLX by 35% on M5 Max", architecture paragraph): every call
 * first expands all experts' gate, up and down banks to fp16 weights in
 * `expanded` (HBM), then runs the grouped GEMMs on those, streaming 4 times
 * the weight bytes.  Same values, same products in the same order: the output
 * is bit-identical to moe_ffn_forward.  For measuring that design only.
 * expanded: device, 16-byte aligned, at least moe_ffn_unfused_bytes(dims)
 * bytes (E * 3 * H * I * 2).  T <= 8 returns MOE_ERR_UNSUPPORTED. */
size_t moe_ffn_unfused_bytes(const moe_dims* dims);  /* 0 if unsupported */
int moe_ffn_forward_unfused(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                            float* y, moe_route_info* info, void* workspace,
                            size_t workspace_bytes, void* expanded, size_t expanded_bytes,
                            void* stream);

/* ------------------------------------- single-launch decode layer --
 * The decode-size layer (T <= 8) as one kernel launch instead of two: the
 * gate/up workgroups and the down workgroups run side by side in one grid,
 * and each down workgroup waits on per-expert device counters until every
 * gate/up item of the experts its token chose has stored its h columns.
 * Page "Perplexity Lily: 1.35x Faster Local AI Than MLX on Mac", section
 * "Why MLX Falls Behind", sets decode apart as a latency-bound workload of
 * its own; page "Perplexity's Lily engine beats MLX by 35% on M5 Max",
 * architecture paragraph, keeps the whole MoE step in one GPU submission.
 * Same kernels' arithmetic, same results as moe_ffn_forward, bit for bit.
 * sync: device int32 [moe_ffn_single_sync_ints()], 4-byte aligned, all
 * zero before its first use; every call leaves the counters at zero again,
 * so a sync buffer is reusable without clearing.  Calls that share a sync
 * buffer must be ordered (one stream, or synchronised): overlapping calls
 * race on it.  sync[257] is set to 1 if a wait ever gave up (each wait is
 * bounded, about a second; never reached in a correct run, and the layer's
 * results are then undefined); it is never cleared by the library.  T > 8 returns MOE_ERR_UNSUPPORTED, and
 * so do shapes whose two halves need workgroups of different sizes
 * (H >= 1024 needs I = H / 4, smaller H needs I = H / 2).  Arguments and
 * other errors as moe_ffn_forward; MOE_ERR_NULL for a NULL sync. */
size_t moe_ffn_single_sync_ints(void);
int moe_ffn_forward_single(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                           float* y, moe_route_info* info, void* workspace, size_t workspace_bytes,
                           int32_t* sync, void* stream);

/* --------------------------------------------- no-allocation variant --
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as moe_ffn_forward (same kernels, same results, bit for bit), with
 * its workspace in a fixed device area of the library instead of a caller's
 * buffer.  The area is moe_ffn_noalloc_max_bytes() (40 MiB) per GPU, held
 * by the library from the first call on that GPU until the process ends; a
 * layer whose workspace (moe_ffn_workspace_bytes) is larger returns
 * MOE_ERR_UNSUPPORTED before anything is enqueued.  Nothing in it needs to
 * start cleared: every piece the layer reads is written earlier in the same
 * call.  The call allocates nothing; its first call on a GPU looks up the
 * area's device address (hipGetSymbolAddress) and fails with MOE_ERR_HIP if
 * that fails.  Every call on one GPU shares the one area: calls that overlap
 * on a GPU (on different streams, or from different threads without ordering)
 * race and give undefined results, and the device pointers `info` receives
 * stay valid only until the next call on that GPU.  Arguments and errors
 * otherwise as moe_ffn_forward. */
size_t moe_ffn_noalloc_max_bytes(void);
int moe_ffn_forward_noalloc(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                            float* y, moe_route_info* info, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4_H */
