// api.hip -- host side of libmoe_w4.so: the C entry points declared in
// include/moe_w4.h.  Every argument is checked on the host before anything
// is enqueued; kernels are then enqueued on the caller's stream, in order,
// with no synchronisation and no device-to-host copy (page "Perplexity's
// Lily engine beats MLX by 35% on M5 Max", architecture paragraph: the
// routing steps stay in one GPU submission).
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "internal.h"

namespace {

thread_local char g_error[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_error[0] = 0;
  return MOE_OK;
}

int hip_status(hipError_t err, const char* where) {
  if (err == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(err));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t max_blocks(int64_t P, int E, int block_m) {
  if (P <= 0 || block_m <= 0) return 0;
  return P / block_m + (P < E ? P : E);
}

// Checks shared by every entry point: counts and routing sizes.
int check_routing(int64_t T, int64_t E, int64_t k) {
  if (T < 0 || E < 1 || k < 1) return fail(MOE_ERR_SHAPE, "need T >= 0, E >= 1, top_k >= 1");
  if (E > 256) return fail(MOE_ERR_UNSUPPORTED, "E = %lld > 256", (long long)E);
  if (k > E || k > 16) return fail(MOE_ERR_UNSUPPORTED, "top_k = %lld exceeds min(E, 16)", (long long)k);
  if (T * k >= (int64_t)1 << 31) return fail(MOE_ERR_UNSUPPORTED, "T * top_k >= 2^31");
  return MOE_OK;
}

int check_bank(const moe_w4_packed& b, const char* name) {
  if (!b.words || !b.sb) return fail(MOE_ERR_NULL, "%s packed bank has a NULL pointer", name);
  if (!aligned16(b.words) || !aligned16(b.sb))
    return fail(MOE_ERR_ALIGN, "%s packed bank not 16-byte aligned", name);
  return MOE_OK;
}

bool pack_sizes_ok(int64_t E, int64_t N, int64_t K, int64_t G) {
  return E >= 1 && E <= 256 && N > 0 && N % 128 == 0 && K > 0 && K % 128 == 0 &&
         (G == 32 || G == 64 || G == 128) && K % G == 0;
}

int check_group(int64_t G, int64_t K, const char* what) {
  if (G != 32 && G != 64 && G != 128) return fail(MOE_ERR_UNSUPPORTED, "group size %lld not in {32, 64, 128}", (long long)G);
  if (K % G) return fail(MOE_ERR_SHAPE, "%s = %lld not a multiple of the group size", what, (long long)K);
  return MOE_OK;
}

int gemm_block_ok(int T, int block_m) {
  if (block_m < 1) return fail(MOE_ERR_SHAPE, "block_m must be >= 1");
  if (T > moe::kGemvMaxTokens && block_m != 32 && block_m != 64 && block_m != 128)
    return fail(MOE_ERR_UNSUPPORTED, "block_m = %d not in {32, 64, 128}", block_m);
  return MOE_OK;
}

size_t gemm_workspace(int mode, int64_t T, int64_t K) {
  return mode == MOE_GEMM_GATE_UP_SWIGLU ? round_up((size_t)T * K * 2) : 0;
}

// h's exponents [P][I / 16] (16-byte padded), then one flag per tile.
size_t hexp_part(int64_t P, int64_t I) { return ((size_t)P * (I / 16) + 15) & ~(size_t)15; }
size_t hexp_bytes(int64_t T, int k, int E, int64_t I, int block_m) {
  const int64_t P = T * k;
  return hexp_part(P, I) + 4 * (size_t)max_blocks(P, E, block_m);
}

// Workspace layout of moe_ffn_forward.
struct FfnLayout {
  size_t logits, logits_part, ids, w, counts, offsets, sorted_pairs, pair_slot, blocks,
      num_blocks, scratch, xh, h, hexp, tflags, y_sorted, yexp, total;
  int router_ks;  // ranges of H the router sums separately (1: no partial sums)
};

FfnLayout ffn_layout(const moe_dims& d, bool has_router, int block_m) {
  const size_t T = d.T, H = d.H, I = d.I, E = d.E, P = (size_t)d.T * d.top_k;
  FfnLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes);
    return at;
  };
  L.logits = take(has_router ? T * E * 4 : 0);
  L.router_ks = has_router ? moe::router_ksplit(d.T, d.H, d.E) : 1;
  L.logits_part = take(L.router_ks > 1 ? (size_t)L.router_ks * T * E * 4 : 0);
  L.ids = take(P * 4);
  L.w = take(P * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted_pairs = take(P * 4);
  L.pair_slot = take(P * 4);
  L.blocks = take((size_t)max_blocks((int64_t)P, d.E, block_m) * 12);
  L.num_blocks = take(4);
  L.scratch = take((size_t)moe::route_chunks(d.T) * E * 4);
  L.xh = take(T * H * 2);
  L.h = take(P * I * 2);
  L.hexp = take(P * (I / 16));                                          // h's exponents
  L.tflags = take((size_t)max_blocks((int64_t)P, d.E, block_m) * 4);  // per-tile flags
  // weighted expert outputs: fp32 (decode path), or int16 mantissas with an
  // exponent per 16 values (MFMA path)
  const bool gemv = d.T <= moe::kGemvMaxTokens;
  L.y_sorted = take(P * H * (gemv ? 4 : 2));
  L.yexp = take(gemv ? 0 : P * (H / 16));
  L.total = o;
  return L;
}

bool gemv_path(const moe_dims& d) { return d.T <= moe::kGemvMaxTokens; }

int check_dims(const moe_dims* d) {
  if (!d) return fail(MOE_ERR_NULL, "dims is NULL");
  int st = check_routing(d->T, d->E, d->top_k);
  if (st) return st;
  if (d->H <= 0 || d->I <= 0) return fail(MOE_ERR_SHAPE, "H and I must be positive");
  if (d->H % 256) return fail(MOE_ERR_UNSUPPORTED, "H = %d not a multiple of 256", d->H);
  if (d->I % 128) return fail(MOE_ERR_UNSUPPORTED, "I = %d not a multiple of 128", d->I);
  if ((st = check_group(d->group_size, d->H, "H"))) return st;
  if ((st = check_group(d->group_size, d->I, "I"))) return st;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "sizes negative or inconsistent";
    case MOE_ERR_UNSUPPORTED: return "sizes outside the supported range";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_error; }

const char* moe_version(void) { return "moe_w4 0.1 gfx950"; }

int moe_route(const uint16_t* x, const uint16_t* router_weight, float* logits, int32_t T,
              int32_t H, int32_t E, int32_t top_k, int32_t* topk_ids, float* topk_weights,
              void* stream) {
  int st = check_routing(T, E, top_k);
  if (st) return st;
  if (T == 0) return ok();  // empty tensors may carry NULL data pointers
  if (!logits || !topk_ids || !topk_weights) return fail(MOE_ERR_NULL, "logits/topk_ids/topk_weights NULL");
  if (router_weight) {
    if (!x) return fail(MOE_ERR_NULL, "x is NULL while router_weight is given");
    if (H <= 0 || H % 128) return fail(MOE_ERR_UNSUPPORTED, "H = %d not a positive multiple of 128", H);
    if (!aligned16(x) || !aligned16(router_weight)) return fail(MOE_ERR_ALIGN, "x or router_weight not 16-byte aligned");
  }
  return hip_status(moe::launch_route(x, router_weight, logits, T, H, E, top_k, topk_ids,
                                      topk_weights, nullptr, nullptr, nullptr, (hipStream_t)stream),
                    "route");
}

size_t moe_w4_packed_words_bytes(int32_t E, int32_t N, int32_t K) {
  if (!pack_sizes_ok(E, N, K, 128)) return 0;  // any supported G divides K % 128 == 0
  return (size_t)E * N * K / 2;
}

size_t moe_w4_packed_sb_bytes(int32_t E, int32_t N, int32_t K, int32_t group_size) {
  if (!pack_sizes_ok(E, N, K, group_size)) return 0;
  // the words, then per expert 2^-c and the dequantisation form (16-byte padded)
  return (size_t)E * N * (K / group_size) * 4 + (((size_t)E * 8 + 15) & ~(size_t)15);
}

int moe_w4_pack(const moe_w4_bank* src, int32_t E, int32_t N, int32_t K, int32_t group_size,
                uint32_t* words, uint32_t* sb, void* stream) {
  if (!src || !words || !sb) return fail(MOE_ERR_NULL, "src, words or sb is NULL");
  if (!src->qweight || !src->scales || !src->biases) return fail(MOE_ERR_NULL, "src bank has a NULL pointer");
  if (E < 1 || N <= 0 || K <= 0) return fail(MOE_ERR_SHAPE, "need E >= 1, N > 0, K > 0");
  if (!pack_sizes_ok(E, N, K, group_size))
    return fail(MOE_ERR_UNSUPPORTED, "pack needs E <= 256, N %% 128 == 0, K %% 128 == 0, G in {32, 64, 128}");
  if (!aligned16(src->qweight) || !aligned16(words) || !aligned16(sb))
    return fail(MOE_ERR_ALIGN, "qweight, words or sb not 16-byte aligned");
  return hip_status(moe::launch_pack(*src, E, N, K, group_size, words, sb, (hipStream_t)stream), "pack");
}

int64_t moe_max_blocks(int32_t T, int32_t top_k, int32_t E, int32_t block_m) {
  return max_blocks((int64_t)T * top_k, E, block_m);
}

size_t moe_build_blocks_workspace_bytes(int32_t T, int32_t top_k, int32_t E) {
  if (T <= 0 || top_k <= 0 || E <= 0) return 0;
  return round_up((size_t)moe::route_chunks(T) * (size_t)E * 4);
}

int moe_build_blocks(const int32_t* topk_ids, int32_t T, int32_t top_k, int32_t E,
                     int32_t block_m, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                     int32_t* pair_slot, int32_t* blocks, int32_t* num_blocks, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_routing(T, E, top_k);
  if (st) return st;
  if (block_m < 1) return fail(MOE_ERR_SHAPE, "block_m must be >= 1");
  if (T == 0) return ok();
  if (!topk_ids || !counts || !offsets || !sorted_pairs || !pair_slot || !blocks || !num_blocks)
    return fail(MOE_ERR_NULL, "an input or output pointer is NULL");
  const size_t need = moe_build_blocks_workspace_bytes(T, top_k, E);
  if (need && !workspace) return fail(MOE_ERR_NULL, "workspace is NULL");
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = moe::launch_chunk_hist(topk_ids, T, top_k, E, (int32_t*)workspace, s);
  if (err != hipSuccess) return hip_status(err, "chunk_hist");
  return hip_status(moe::launch_scan_scatter(topk_ids, T, top_k, E, (const int32_t*)workspace,
                                             block_m, counts, offsets, sorted_pairs, pair_slot,
                                             blocks, num_blocks, s),
                    "scan_scatter");
}

size_t moe_w4_grouped_gemm_workspace_bytes(const moe_w4_gemm_args* a) {
  if (!a || a->T <= 0 || a->K <= 0) return 0;
  return gemm_workspace(a->mode, a->T, a->K);
}

int moe_w4_grouped_gemm(const moe_w4_gemm_args* a, void* stream) {
  if (!a) return fail(MOE_ERR_NULL, "args is NULL");
  if (a->mode != MOE_GEMM_GATE_UP_SWIGLU && a->mode != MOE_GEMM_DOWN)
    return fail(MOE_ERR_SHAPE, "unknown mode %d", a->mode);
  const bool gate_up = a->mode == MOE_GEMM_GATE_UP_SWIGLU;
  int st = check_routing(a->T, a->E, a->top_k);
  if (st) return st;
  if (a->N <= 0 || a->K <= 0) return fail(MOE_ERR_SHAPE, "N and K must be positive");
  if ((st = check_group(a->group_size, a->K, "K"))) return st;
  if (a->K % 128) return fail(MOE_ERR_UNSUPPORTED, "K = %d not a multiple of 128", a->K);
  if (a->N % (gate_up ? 128 : 256))
    return fail(MOE_ERR_UNSUPPORTED, "N = %d not a multiple of %d", a->N, gate_up ? 128 : 256);
  if ((st = gemm_block_ok(a->T, a->block_m))) return st;
  if (a->T == 0) return ok();
  const int64_t hI = gate_up ? a->N : a->K;  // h's columns
  const size_t hneed = hexp_bytes(a->T, a->top_k, a->E, hI, a->block_m);
  if (!a->h_exp) return fail(MOE_ERR_NULL, "h_exp is NULL");
  if (!aligned16(a->h_exp)) return fail(MOE_ERR_ALIGN, "h_exp not 16-byte aligned");
  if (a->h_exp_bytes < hneed) return fail(MOE_ERR_WORKSPACE, "h_exp %zu < %zu bytes", a->h_exp_bytes, hneed);
  if (!a->a || !a->sorted_pairs || !a->blocks || !a->num_blocks || !a->out)
    return fail(MOE_ERR_NULL, "a/sorted_pairs/blocks/num_blocks/out NULL");
  if (!gate_up && !a->topk_weights) return fail(MOE_ERR_NULL, "topk_weights NULL");
  if ((st = check_bank(a->bank0, gate_up ? "gate" : "down"))) return st;
  if (gate_up && (st = check_bank(a->bank1, "up"))) return st;
  if (!aligned16(a->a) || !aligned16(a->out)) return fail(MOE_ERR_ALIGN, "a or out not 16-byte aligned");
  const size_t need = gemm_workspace(a->mode, a->T, a->K);
  if (need && (!a->workspace || !aligned16(a->workspace)))
    return fail(a->workspace ? MOE_ERR_ALIGN : MOE_ERR_NULL, "workspace NULL or misaligned");
  if (a->workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", a->workspace_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  moe::GemmArgs g{a->mode, a->T, a->top_k, a->E, a->N, a->K, a->group_size, a->block_m,
                  (const moe::half_t*)a->a, a->bank0, a->bank1, a->sorted_pairs,
                  a->topk_weights, a->blocks, a->num_blocks, a->out};
  g.t0 = moe::bank_tail(a->bank0, a->E, a->N, a->K, a->group_size);
  g.t1 = gate_up ? moe::bank_tail(a->bank1, a->E, a->N, a->K, a->group_size) : g.t0;
  g.hexp = (int8_t*)a->h_exp;
  g.tflags = (int32_t*)((char*)a->h_exp + hexp_part((int64_t)a->T * a->top_k, hI));
  if (gate_up) {
    // the fp16 operand copy of x; the tile flags the kernel sets start cleared
    hipError_t err = moe::launch_stage_x((const uint16_t*)a->a, (moe::half_t*)a->workspace,
                                         (int64_t)a->T * a->K, g.tflags,
                                         max_blocks((int64_t)a->T * a->top_k, a->E, a->block_m), s);
    if (err != hipSuccess) return hip_status(err, "stage_x");
    g.a = (const moe::half_t*)a->workspace;
  }
  const hipError_t err = a->T <= moe::kGemvMaxTokens ? moe::launch_w4_gemv(g, s) : moe::launch_w4_mfma(g, s);
  return hip_status(err, "w4_grouped_gemm");
}

size_t moe_w4_h_exp_bytes(int32_t T, int32_t top_k, int32_t E, int32_t I, int32_t block_m) {
  if (T <= 0 || top_k <= 0 || E <= 0 || I <= 0 || I % 16 || block_m <= 0) return 0;
  return hexp_bytes(T, top_k, E, I, block_m);
}

int32_t moe_ffn_block_m(const moe_dims* d) {
  if (!d || d->E <= 0) return 0;
  if (d->T <= moe::kGemvMaxTokens) return moe::kGemvMaxTokens;
  const int64_t avg = (int64_t)d->T * d->top_k / d->E;
  return avg <= 16 ? 32 : avg <= 64 ? 64 : 128;
}

size_t moe_ffn_workspace_bytes(const moe_dims* d, int32_t has_router) {
  if (!d || check_dims(d) != MOE_OK) return 0;
  return ffn_layout(*d, has_router != 0, moe_ffn_block_m(d)).total;
}

}  // extern "C"

namespace {

// Records stage event i (when given) on the stream before stage i runs.
hipError_t mark(void* const* events, int i, hipStream_t s) {
  if (!events || !events[i]) return hipSuccess;
  return hipEventRecord((hipEvent_t)events[i], s);
}

// The host round trip of the S2-S5 ablation: the per-chunk histograms come
// to the host (the stream is synchronised), the host computes counts,
// offsets, each chunk's first slot per expert and the block map, and uploads
// them (first slots over the histograms); the device then only scatters,
// and the GEMMs are launched with the exact tile count.  host stays in use
// by the uploads until the stream passes them.
hipError_t host_block_map(const moe_dims& d, int block_m, int32_t* host, int32_t* chunk_hist,
                          int32_t* counts, int32_t* offsets, int32_t* blocks, int32_t* num_blocks,
                          int64_t* tiles_out, hipStream_t s) {
  const int E = d.E, nch = moe::route_chunks(d.T);
  const int64_t P = (int64_t)d.T * d.top_k;
  int32_t* hist = host;  // [nch][E], then first slots
  int32_t* hc = hist + (size_t)nch * E;
  int32_t* ho = hc + E;
  int32_t* hb = ho + E + 1;
  int32_t* hn = hb + 3 * max_blocks(P, E, block_m);
  hipError_t err = hipMemcpyAsync(hist, chunk_hist, sizeof(int32_t) * nch * E, hipMemcpyDeviceToHost, s);
  if (err != hipSuccess) return err;
  if ((err = hipStreamSynchronize(s)) != hipSuccess) return err;
  int64_t off = 0, tiles = 0;
  for (int e = 0; e < E; e++) {
    int64_t run = off;
    for (int c = 0; c < nch; c++) {
      const int32_t n = hist[(size_t)c * E + e];
      hist[(size_t)c * E + e] = (int32_t)run;
      run += n;
    }
    hc[e] = (int32_t)(run - off);
    ho[e] = (int32_t)off;
    for (int64_t i = 0; i * block_m < run - off; i++, tiles++) {
      hb[3 * tiles] = e;
      hb[3 * tiles + 1] = (int32_t)(off + i * block_m);
      hb[3 * tiles + 2] = (int32_t)std::min<int64_t>(block_m, run - off - i * block_m);
    }
    off = run;
  }
  ho[E] = (int32_t)P;
  *hn = (int32_t)tiles;
  const struct { void* dst; const void* src; size_t n; } up[] = {
      {chunk_hist, hist, sizeof(int32_t) * nch * E}, {counts, hc, sizeof(int32_t) * E},
      {offsets, ho, sizeof(int32_t) * (E + 1)}, {blocks, hb, sizeof(int32_t) * 3 * tiles},
      {num_blocks, hn, sizeof(int32_t)}};
  for (const auto& u : up)
    if (u.n && (err = hipMemcpyAsync(u.dst, u.src, u.n, hipMemcpyHostToDevice, s)) != hipSuccess) return err;
  *tiles_out = tiles;
  return hipSuccess;
}

// Bytes of the fp16 weights the unfused ablation expands: gate, up and down
// of every expert.
size_t unfused_bytes(const moe_dims& d) { return (size_t)d.E * 3 * d.H * d.I * 2; }

// Ints of the pinned host buffer the host-block-map path uses: per-chunk
// histograms (then first slots), counts, offsets, the block map and its size.
size_t host_blockmap_ints(const moe_dims& d, int block_m) {
  const int64_t P = (int64_t)d.T * d.top_k;
  return (size_t)moe::route_chunks(d.T) * d.E + d.E + (d.E + 1) +
         3 * (size_t)max_blocks(P, d.E, block_m) + 1;
}

// host (or nullptr): pinned host buffer of host_blockmap_ints ints; when
// given, S2-S5 take the host round trip (see moe_ffn_forward_host_blockmap).
int ffn_forward_impl(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                     float* y, moe_route_info* info, void* workspace, size_t workspace_bytes,
                     void* const* events, hipStream_t s, int32_t* host = nullptr,
                     size_t host_ints = 0, uint32_t* expanded = nullptr,
                     size_t expanded_bytes = 0, const moe_ffn_io* io = nullptr,
                     int32_t* sync = nullptr) {
  if (!layer) return fail(MOE_ERR_NULL, "layer is NULL");
  const moe_dims& d = layer->dims;
  int st = check_dims(&d);
  if (st) return st;
  const bool has_router = layer->router_weight != nullptr;
  const int block_m = moe_ffn_block_m(&d);
  if (d.T == 0) {  // empty tensors may carry NULL data pointers
    if (info) *info = moe_route_info{block_m, 1, router_logits, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 4, nullptr,
                                     nullptr};
    return ok();
  }
  if (has_router == (router_logits != nullptr))
    return fail(MOE_ERR_SHAPE, "give exactly one of layer->router_weight and router_logits");
  if (!x || !y) return fail(MOE_ERR_NULL, "x or y is NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(MOE_ERR_ALIGN, "x or y not 16-byte aligned");
  if (has_router && !aligned16(layer->router_weight)) return fail(MOE_ERR_ALIGN, "router_weight not 16-byte aligned");
  if ((st = check_bank(layer->gate, "gate")) || (st = check_bank(layer->up, "up")) ||
      (st = check_bank(layer->down, "down")))
    return st;
  const FfnLayout L = ffn_layout(d, has_router, block_m);
  const bool norm = io && io->norm_weight;
  const size_t need = L.total + (norm ? round_up((size_t)d.T * d.H * 2) : 0);
  if (io) {
    if (io->out && !io->residual) return fail(MOE_ERR_NULL, "io->out given without io->residual");
    if ((norm && !aligned16(io->norm_weight)) || (io->out && (!aligned16(io->out) || !aligned16(io->residual))))
      return fail(MOE_ERR_ALIGN, "io->norm_weight, residual or out not 16-byte aligned");
  }
  if (!workspace) return fail(MOE_ERR_NULL, "workspace is NULL");
  if ((uintptr_t)workspace & 255u) return fail(MOE_ERR_ALIGN, "workspace not 256-byte aligned");
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (expanded) {
    if (d.T <= moe::kGemvMaxTokens)
      return fail(MOE_ERR_UNSUPPORTED, "the unfused path needs T > %d", moe::kGemvMaxTokens);
    if (!aligned16(expanded)) return fail(MOE_ERR_ALIGN, "expanded weights not 16-byte aligned");
    if (expanded_bytes < unfused_bytes(d))
      return fail(MOE_ERR_WORKSPACE, "expanded buffer %zu < %zu bytes", expanded_bytes, unfused_bytes(d));
  }
  if (sync) {
    if (d.T > moe::kGemvMaxTokens)
      return fail(MOE_ERR_UNSUPPORTED, "the single-launch layer needs T <= %d", moe::kGemvMaxTokens);
    if ((uintptr_t)sync & 3u) return fail(MOE_ERR_ALIGN, "sync not 4-byte aligned");
  }
  if (host) {
    if (d.T <= moe::kGemvMaxTokens)
      return fail(MOE_ERR_UNSUPPORTED, "the host block map path needs T > %d", moe::kGemvMaxTokens);
    if (host_ints < host_blockmap_ints(d, block_m))
      return fail(MOE_ERR_WORKSPACE, "host buffer %zu < %zu ints", host_ints, host_blockmap_ints(d, block_m));
  }

  char* ws = (char*)workspace;
  float* logits = has_router ? (float*)(ws + L.logits) : (float*)router_logits;
  int32_t* ids = (int32_t*)(ws + L.ids);
  float* w = (float*)(ws + L.w);
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* sorted_pairs = (int32_t*)(ws + L.sorted_pairs);
  int32_t* pair_slot = (int32_t*)(ws + L.pair_slot);
  int32_t* blocks = (int32_t*)(ws + L.blocks);
  int32_t* num_blocks = (int32_t*)(ws + L.num_blocks);
  moe::half_t* xh = (moe::half_t*)(ws + L.xh);
  moe::half_t* h = (moe::half_t*)(ws + L.h);
  uint8_t* y_sorted = (uint8_t*)(ws + L.y_sorted);
  int8_t* hexp = (int8_t*)(ws + L.hexp);
  int8_t* yexp = gemv_path(d) ? nullptr : (int8_t*)(ws + L.yexp);
  int32_t* tflags = (int32_t*)(ws + L.tflags);
  const int64_t nflags = max_blocks((int64_t)d.T * d.top_k, d.E, block_m);
  const bool gemv = d.T <= moe::kGemvMaxTokens;
  if (info) {
    *info = moe_route_info{block_m, gemv ? 1 : 0, logits, ids, w, counts, offsets, sorted_pairs,
                           pair_slot, blocks, num_blocks, (const uint16_t*)h, y_sorted,
                           gemv ? 4 : 2, hexp, yexp};
  }

  hipError_t err;
  int32_t* chunk_hist = (int32_t*)(ws + L.scratch);
  int64_t grid_tiles = -1;  // host-known tile count (host block map path)
  float* part = L.router_ks > 1 ? (float*)(ws + L.logits_part) : nullptr;  // router partial sums
  if ((err = mark(events, MOE_STAGE_ROUTE, s)) != hipSuccess) return hip_status(err, "event");
  // RMSNorm in front: at prefill sizes folded into the routing front end
  // (the router multiplies bf16(x * gamma), the routing kernel scales each
  // row's logits by its 1 / rms and stages the normalised rows); otherwise
  // its own launch, and the layer runs on the normalised rows
  moe::GemmArgs shape{MOE_GEMM_GATE_UP_SWIGLU, d.T, d.top_k, d.E, d.I, d.H, d.group_size, block_m,
                      nullptr, layer->gate, layer->up, nullptr, nullptr, nullptr, nullptr, nullptr};
  // at decode sizes (logits given, every x row resident in the gate/up
  // launch's LDS) folded into that launch's staging of x
  const bool norm_folded = norm && !host && !expanded && !sync &&
                           (gemv ? !has_router && moe::decode_norm_fits(shape)
                                 : moe::route_norm_fits(d.T, d.H, d.E, has_router, L.router_ks > 1));
  if (norm && !norm_folded) {
    uint16_t* xn = (uint16_t*)(ws + L.total);
    if ((err = moe::launch_rmsnorm(x, io->norm_weight, io->norm_eps, d.T, d.H, xn, s)) != hipSuccess)
      return hip_status(err, "rmsnorm");
    x = xn;
  }
  const uint16_t* residual = io && io->out ? io->residual : nullptr;
  uint16_t* out = io ? io->out : nullptr;
  if (gemv) {
    // decode sizes: the router GEMM (when given), then S1-S6 in one launch
    // (the build stage and the routing inside the gate/up stage)
    if (has_router && (err = moe::launch_router_logits(x, layer->router_weight, part ? part : logits,
                                                       d.T, d.H, d.E, L.router_ks, s)) != hipSuccess)
      return hip_status(err, "router");
    if ((err = mark(events, MOE_STAGE_BUILD_BLOCKS, s)) != hipSuccess) return hip_status(err, "event");
  } else {
    if ((err = moe::launch_route(x, layer->router_weight, logits, d.T, d.H, d.E, d.top_k, ids, w, xh,
                                 chunk_hist, part, s, norm_folded ? io->norm_weight : nullptr,
                                 norm_folded ? io->norm_eps : 0.0f)) != hipSuccess)
      return hip_status(err, "route");
    if ((err = mark(events, MOE_STAGE_BUILD_BLOCKS, s)) != hipSuccess) return hip_status(err, "event");
    if (host) {
      if ((err = host_block_map(d, block_m, host, chunk_hist, counts, offsets, blocks, num_blocks,
                                &grid_tiles, s)) != hipSuccess)
        return hip_status(err, "host block map");
    }
    if ((err = moe::launch_scan_scatter(ids, d.T, d.top_k, d.E, chunk_hist, block_m, counts, offsets,
                                        sorted_pairs, pair_slot, blocks, num_blocks, s,
                                        host ? chunk_hist : nullptr, tflags, nflags)) != hipSuccess)
      return hip_status(err, "scan_scatter");
  }
  moe::GemmArgs g1{MOE_GEMM_GATE_UP_SWIGLU, d.T, d.top_k, d.E, d.I, d.H, d.group_size, block_m,
                   xh, layer->gate, layer->up, sorted_pairs, w, blocks, num_blocks, h, false,
                   grid_tiles};
  moe::GemmArgs g2{MOE_GEMM_DOWN, d.T, d.top_k, d.E, d.H, d.I, d.group_size, block_m,
                   h, layer->down, layer->down, sorted_pairs, w, blocks, num_blocks, y_sorted,
                   !gemv, grid_tiles};
  g1.hexp = g2.hexp = hexp;
  g2.yexp = yexp;
  g1.tflags = g2.tflags = tflags;
  g1.t0 = moe::bank_tail(layer->gate, d.E, d.I, d.H, d.group_size);
  g1.t1 = moe::bank_tail(layer->up, d.E, d.I, d.H, d.group_size);
  g2.t0 = g2.t1 = moe::bank_tail(layer->down, d.E, d.H, d.I, d.group_size);
  if ((err = mark(events, MOE_STAGE_GATE_UP, s)) != hipSuccess) return hip_status(err, "event");
  if (gemv) {
    g1.a = (const moe::half_t*)x;  // bf16, converted while staged
    const moe::DecodeRouting dr{part ? part : logits, logits, L.router_ks, ids, w, counts, offsets,
                                sorted_pairs, pair_slot, blocks, num_blocks};
    if (sync) {
      // the whole layer in one launch (the down and combine stages are empty)
      if (!moe::decode_layer_supported(g1, g2))
        return fail(MOE_ERR_UNSUPPORTED, "the single-launch layer needs H and I on workgroups of one size");
      if ((err = moe::launch_decode_layer(dr, g1, g2, y, sync, s, residual, out)) != hipSuccess)
        return hip_status(err, "decode layer");
      if ((err = mark(events, MOE_STAGE_DOWN, s)) != hipSuccess ||
          (err = mark(events, MOE_STAGE_COMBINE, s)) != hipSuccess ||
          (err = mark(events, MOE_NUM_STAGES, s)) != hipSuccess)
        return hip_status(err, "event");
      return ok();
    }
    err = moe::launch_decode_gate_up(dr, g1, s, norm_folded ? io->norm_weight : nullptr,
                                     norm_folded ? io->norm_eps : 0.0f);
  } else if (expanded) {
    // unfused ablation: every expert's banks expanded to fp16 in HBM first
    uint32_t* eg = expanded;
    uint32_t* eu = eg + (size_t)d.E * d.I * d.H / 2;
    uint32_t* ed = eu + (size_t)d.E * d.I * d.H / 2;
    if ((err = moe::launch_expand(layer->gate, d.E, d.I, d.H, d.group_size, eg, s)) != hipSuccess ||
        (err = moe::launch_expand(layer->up, d.E, d.I, d.H, d.group_size, eu, s)) != hipSuccess ||
        (err = moe::launch_expand(layer->down, d.E, d.H, d.I, d.group_size, ed, s)) != hipSuccess)
      return hip_status(err, "expand");
    g1.b0 = moe_w4_packed{eg, nullptr};
    g1.b1 = moe_w4_packed{eu, nullptr};
    g2.b0 = g2.b1 = moe_w4_packed{ed, nullptr};
    g1.dense = g2.dense = true;
  }
  if (!gemv) err = moe::launch_w4_mfma(g1, s);
  if (err != hipSuccess) return hip_status(err, "gate_up");
  if ((err = mark(events, MOE_STAGE_DOWN, s)) != hipSuccess) return hip_status(err, "event");
  if (gemv && moe::decode_down_fused(d.I)) {
    // decode sizes: the down GEMV and the combine in one launch, per token
    // (the combine stage is empty)
    if ((err = moe::launch_decode_down(g2, ids, pair_slot, y, s, residual, out)) != hipSuccess)
      return hip_status(err, "down");
    if ((err = mark(events, MOE_STAGE_COMBINE, s)) != hipSuccess) return hip_status(err, "event");
  } else {
    err = gemv ? moe::launch_w4_gemv(g2, s) : moe::launch_w4_mfma(g2, s);
    if (err != hipSuccess) return hip_status(err, "down");
    if ((err = mark(events, MOE_STAGE_COMBINE, s)) != hipSuccess) return hip_status(err, "event");
    if ((err = moe::launch_combine(y_sorted, yexp, pair_slot, y, d.T, d.H, d.top_k, s, residual, out)) !=
        hipSuccess)
      return hip_status(err, "combine");
  }
  if ((err = mark(events, MOE_NUM_STAGES, s)) != hipSuccess) return hip_status(err, "event");
  return ok();
}

}  // namespace

extern "C" {

int moe_ffn_forward(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                    float* y, moe_route_info* info, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return ffn_forward_impl(layer, x, router_logits, y, info, workspace, workspace_bytes, nullptr,
                          (hipStream_t)stream);
}

size_t moe_ffn_single_sync_ints(void) { return moe::kDecodeSyncInts; }

int moe_ffn_forward_single(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                           float* y, moe_route_info* info, void* workspace, size_t workspace_bytes,
                           int32_t* sync, void* stream) {
  if (!sync) return fail(MOE_ERR_NULL, "sync is NULL");
  return ffn_forward_impl(layer, x, router_logits, y, info, workspace, workspace_bytes, nullptr,
                          (hipStream_t)stream, nullptr, 0, nullptr, 0, nullptr, sync);
}

size_t moe_ffn_unfused_bytes(const moe_dims* d) {
  if (!d || check_dims(d) != MOE_OK || d->T <= moe::kGemvMaxTokens) return 0;
  return unfused_bytes(*d);
}

int moe_ffn_forward_unfused(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                            float* y, moe_route_info* info, void* workspace,
                            size_t workspace_bytes, void* expanded, size_t expanded_bytes,
                            void* stream) {
  if (!expanded) return fail(MOE_ERR_NULL, "expanded is NULL");
  return ffn_forward_impl(layer, x, router_logits, y, info, workspace, workspace_bytes, nullptr,
                          (hipStream_t)stream, nullptr, 0, (uint32_t*)expanded, expanded_bytes);
}

size_t moe_ffn_host_blockmap_ints(const moe_dims* d) {
  if (!d || check_dims(d) != MOE_OK || d->T <= moe::kGemvMaxTokens) return 0;
  return host_blockmap_ints(*d, moe_ffn_block_m(d));
}

int moe_ffn_forward_host_blockmap(const moe_layer* layer, const uint16_t* x,
                                  const float* router_logits, float* y, moe_route_info* info,
                                  void* workspace, size_t workspace_bytes, int32_t* host_pinned,
                                  size_t host_ints, void* stream) {
  if (!host_pinned) return fail(MOE_ERR_NULL, "host_pinned is NULL");
  return ffn_forward_impl(layer, x, router_logits, y, info, workspace, workspace_bytes, nullptr,
                          (hipStream_t)stream, host_pinned, host_ints);
}

int moe_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int32_t T, int32_t H,
                uint16_t* out, void* stream) {
  if (T < 0 || H <= 0) return fail(MOE_ERR_SHAPE, "need T >= 0 and H > 0");
  if (H % 8) return fail(MOE_ERR_UNSUPPORTED, "H = %d not a multiple of 8", H);
  if (T == 0) return ok();
  if (!x || !gamma || !out) return fail(MOE_ERR_NULL, "x, gamma or out is NULL");
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(out)) return fail(MOE_ERR_ALIGN, "x, gamma or out not 16-byte aligned");
  return hip_status(moe::launch_rmsnorm(x, gamma, eps, T, H, out, (hipStream_t)stream), "rmsnorm");
}

size_t moe_decode_attention_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_len) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_len < 0) return 0;
  const moe::AttnPlan pl = moe::attn_plan(B, Hkv, max_len);
  return round_up((size_t)B * Hq * pl.nsplit * (128 + 2) * 4);
}

int moe_decode_attention(const uint16_t* q, const uint16_t* kcache, const uint16_t* vcache,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t block, int32_t max_blocks,
                         int32_t num_blocks, int32_t max_len, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || block < 1 || max_blocks < 1 || num_blocks < 1 || max_len < 0)
    return fail(MOE_ERR_SHAPE, "need B >= 0, Hq, Hkv, block, max_blocks, num_blocks >= 1, max_len >= 0");
  if (D != 128) return fail(MOE_ERR_UNSUPPORTED, "D = %d (only 128)", D);
  if (block % 8) return fail(MOE_ERR_UNSUPPORTED, "block = %d not a multiple of 8", block);
  const int g = Hq % Hkv ? 0 : Hq / Hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(MOE_ERR_UNSUPPORTED, "Hq / Hkv = %d / %d not in {1, 2, 4, 8}", Hq, Hkv);
  if (B == 0) return ok();
  if (!q || !kcache || !vcache || !block_table || !seq_lens || !out || !workspace)
    return fail(MOE_ERR_NULL, "a pointer argument is NULL");
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out) || !aligned16(workspace))
    return fail(MOE_ERR_ALIGN, "q, caches, out or workspace not 16-byte aligned");
  if (moe::attn_plan(B, Hkv, max_len).nsplit > 4096)
    return fail(MOE_ERR_UNSUPPORTED, "max_len = %d above 4194304", max_len);
  const size_t need = moe_decode_attention_workspace_bytes(B, Hq, Hkv, max_len);
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  return hip_status(moe::launch_decode_attention(q, kcache, vcache, block_table, seq_lens, B, Hq, Hkv,
                                                 block, max_blocks, num_blocks, max_len, out,
                                                 (float*)workspace, (hipStream_t)stream),
                    "decode_attention");
}

size_t moe_ffn_io_workspace_bytes(const moe_dims* d, int32_t has_router) {
  if (!d || check_dims(d) != MOE_OK) return 0;
  return ffn_layout(*d, has_router != 0, moe_ffn_block_m(d)).total + round_up((size_t)d->T * d->H * 2);
}

int moe_ffn_forward_io(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                       float* y, const moe_ffn_io* io, moe_route_info* info, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return ffn_forward_impl(layer, x, router_logits, y, info, workspace, workspace_bytes, nullptr,
                          (hipStream_t)stream, nullptr, 0, nullptr, 0, io);
}

int moe_ffn_forward_timed(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                          float* y, moe_route_info* info, void* workspace, size_t workspace_bytes,
                          void* const* stage_events, void* stream) {
  if (!stage_events) return fail(MOE_ERR_NULL, "stage_events is NULL");
  return ffn_forward_impl(layer, x, router_logits, y, info, workspace, workspace_bytes,
                          stage_events, (hipStream_t)stream);
}

}  // extern "C"

// ------------------------------------------------- no-allocation variant --
// moe_ffn_forward_noalloc runs the layer with its workspace in this fixed
// device array instead of a caller's buffer.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the device address
// hipGetSymbolAddress reports for the current device, looked up once per
// device on its first call.
namespace {

constexpr size_t kScratchBytes = (size_t)40 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on the device's
// first call, with that device current).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_status(err, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return hip_status(err, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_ffn_noalloc_max_bytes(void) { return kScratchBytes; }

int moe_ffn_forward_noalloc(const moe_layer* layer, const uint16_t* x, const float* router_logits,
                            float* y, moe_route_info* info, void* stream) {
  if (!layer) return fail(MOE_ERR_NULL, "layer is NULL");
  int st = check_dims(&layer->dims);
  if (st) return st;
  const size_t need = ffn_layout(layer->dims, layer->router_weight != nullptr,
                                 moe_ffn_block_m(&layer->dims)).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "this layer needs %zu bytes of scratch, more than the fixed %zu (use moe_ffn_forward "
                "with a workspace)", need, kScratchBytes);
  if (layer->dims.T == 0) return ffn_forward_impl(layer, x, router_logits, y, info, nullptr, 0, nullptr,
                                                  (hipStream_t)stream);
  void* ptr = nullptr;
  if ((st = scratch_address(&ptr))) return st;
  return ffn_forward_impl(layer, x, router_logits, y, info, ptr, kScratchBytes, nullptr,
                          (hipStream_t)stream);
}

}  // extern "C"
