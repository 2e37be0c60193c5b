// gemm.hip -- S6/S7 grouped W4 GEMM on fp16 MFMA with the 4-bit
// dequantisation fused into the kernel (page "Perplexity's Lily engine beats
// MLX by 35% on M5 Max", architecture paragraph: dequantising inside the
// grouped GEMM keeps expanded 16-bit weights out of memory), the activation
// staging pass of the standalone entry point, and the S8 combine.
//
// One workgroup of W waves computes a tile of BM rows (slots of one expert,
// from the block map) x 64 W weight columns: 32 W columns of the gate bank
// and the same 32 W of the up bank (S6), or 64 W columns of the down bank
// (S7), over the whole reduction dimension in slabs of 64.  Wave w owns all
// BM rows and two 32-column blocks (gate and up columns 32w.. in S6,
// columns 64w.. in S7), so every word of codes it dequantises feeds BM/32
// MFMAs per block.  W is 4, and two or three workgroups share a CU.
//
// Operands reach LDS with global_load_lds_dwordx4 (each lane's 16 bytes
// land at the instruction's LDS base + 16 * lane, no registers involved)
// into a ring of R stages (R = 4 for 32-row tiles, 3 otherwise); the loads
// for slab s + R - 1 are issued while slab s is computed, so R - 1 slabs of
// loads are in flight and the compute reads only LDS.  Per slab and stage:
//  - A: BM rows x 64 fp16 activations (operand order), 128 bytes a row, the
//    16-byte chunk c of row r at position c ^ a_swz(r).  Rows past the tile's
//    end load a valid row whose results are never stored.
//  - B: packed codes (tile-major, see moe_w4_pack): per 32-column block one
//    contiguous 1 KiB piece [32 columns][2 reduction halves] x 16 bytes.
//    Each lane dequantises its 16 bytes in registers (11 VALU instructions
//    per 8 codes) against the column's packed fp16 scale and bias.
//  - S: per column and reduction half the packed (scale, bias) word of the
//    slab's group, 128 contiguous bytes per 32 columns.
// One wait (s_waitcnt on this wave's own outstanding loads, a count known
// at compile time) and one barrier per slab; the slab loop has no branches.  MFMA v_mfma_f32_32x32x16_f16,
// fp32 accumulation.
// Work items (tile, column block) are spread over the 8 XCDs in contiguous
// ranges, so the column blocks of one tile, and the tiles of one expert, run
// on the same XCD at about the same time and share its L2.
#include <algorithm>

#include "internal.h"

namespace moe {
namespace {

constexpr int kSlabK = 64;

// A tiles in LDS: the 16-byte chunk c of tile row r sits at position
// c ^ a_swz(r) of the row's 128 bytes.  A fragment read takes one logical
// chunk of 16 consecutive rows in each 16-lane group; the LDS serves 16 lanes
// of a 16-byte read per cycle over 64 four-byte banks, so the even rows of the
// 16 must use 8 distinct positions (they share banks 0..31 of a 256-byte
// line) and so must the odd rows (banks 32..63): rows 2m and 2m + 1 take
// pattern m.  (r % 8 gave rows r and r + 8 the same position: a two-way
// conflict on every fragment read.)
__device__ __forceinline__ int a_swz(int r) { return (r >> 1) & 7; }

template <int V>
struct IntTag {
  static constexpr int value = V;
};

struct MfmaParams {
  const half_t* a;
  moe_w4_packed b0, b1;
  const int32_t* sorted_pairs;
  const float* topk_weights;
  const int32_t* blocks;
  const int32_t* num_blocks;
  void* out;
  BankTail t0, t1;  // per-expert 2^-c and dequantisation form of b0 / b1
  int8_t* hexp;     // h's exponents [P][I / 16]: written by S6, read by S7
  int32_t* tflags;  // per tile: a row of it has a nonzero exponent
  int8_t* yexp;     // S7 with PACK: y16e exponents [P][N / 16]
  int N, K, log2_G, top_k, E, P, max_blocks;
};

// WAVES waves per workgroup: the tile covers 64 * WAVES weight columns.
// With 4 waves several workgroups fit a CU (two of 128 rows, three of 64
// rows with a 3-stage ring), so one workgroup's prologue and epilogue
// overlap another's main loop.
// G32: group size 32, the two reduction halves of a slab have their own
// (scale, bias) words; for G >= 64 one word serves both and is copied once.
// STAGES: depth of the LDS ring (STAGES - 1 slabs in flight); WGS_PER_CU:
// workgroups meant to share a CU, passed to the compiler as the waves per
// SIMD that budget implies (WGS_PER_CU * WAVES / 4).
// PACK (S7 only): out is y16e block floating point (int16 mantissas, exponents
// at yexp) instead of fp32.
// DENSE (the unfused ablation): the banks hold weights already expanded to
// fp16 in operand order (moe_w4_expand: per 32-column block and slab, four
// 1 KiB pieces, piece i the dequantised word i of every (column, half)), and
// the kernel copies and multiplies them with no dequantisation.
// y16_exp (internal.h) for m >= 0 (not NaN) from the float's bits: for m (1 + 2^-15)
// normal its frexp exponent is the biased exponent - 126; zero and subnormal
// products land below -128 and clamp there, as y16_exp's m > 0 test and
// clamp give.
__device__ __forceinline__ int y16_exp_bits(float m) {
  const uint32_t u = __float_as_uint(m * (1.0f + 0x1p-15f));
  const int e = max(-128, min(127, (int)(u >> 23) - 141));
  return __float_as_uint(m) >= 0x7F000000u ? 127 : e;
}
// h_block_exp (internal.h) of m >= 0 given as its bits (no branches): 0 when m is 0,
// in [2^-10, 2^15) or NaN; 127 above 3e38; else the frexp exponent (biased
// exponent - 126; subnormals land below -128) less 15, clamped.
__device__ __forceinline__ int h_block_exp_bits(uint32_t u) {
  const bool keep = u == 0u || u - 0x3A800000u < 0x47000000u - 0x3A800000u || u > 0x7F800000u;
  const int e = max(-128, min(127, (int)(u >> 23) - 141));
  return keep ? 0 : u > 0x7F61B1E6u ? 127 : e;
}

template <int MODE, int MB, int WAVES, bool G32, int STAGES, int WGS_PER_CU, bool PACK = false,
          bool DENSE = false>
__global__ __launch_bounds__(64 * WAVES, WGS_PER_CU * WAVES / 4) void w4_mfma_kernel(const MfmaParams p) {
  constexpr bool GATE_UP = MODE == MOE_GEMM_GATE_UP_SWIGLU;
  constexpr int BM = MB * 32;
  constexpr int kBCols = 64 * WAVES;                     // weight columns per workgroup
  constexpr int kBStage = kBCols * (DENSE ? 128 : 32);   // bytes of codes (or fp16 weights) per stage
  constexpr int kSStage = DENSE ? 0 : kBCols * 4 * (G32 ? 2 : 1);  // bytes of scale / bias words per stage
  constexpr int A_BYTES = BM * 128;                      // per stage
  constexpr int STAGE = A_BYTES + kBStage + kSStage;
  constexpr int A_INSTR = BM / 8;                        // 1 KiB A loads per stage
  constexpr int A_PER_WAVE = A_INSTR >= WAVES ? A_INSTR / WAVES : 1;
  constexpr int B_PER_WAVE = DENSE ? 8 : 2;              // 1 KiB code blocks (or fp16 pieces) per wave
  constexpr int S_PER_WAVE = DENSE ? 0 : G32 ? 2 : 1;    // 256 B scale-word loads per wave
  constexpr int OUT_COLS = GATE_UP ? kBCols / 2 : kBCols; // output columns per workgroup
  __shared__ __attribute__((aligned(16))) char lds[STAGES * STAGE];
  __shared__ float row_w[BM];  // S7: routing weight of each row
  __shared__ int erow[GATE_UP ? 1 : BM];  // S7, tiles with scaled h rows: each row's largest exponent
  static_assert(!GATE_UP || BM * OUT_COLS * 4 <= STAGES * STAGE, "fp32 h tile must fit the ring");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS and block addresses stay scalar
  const int col = lane & 31, khalf = lane >> 5;

  // the pointers of the first dependent reads are fetched with the kernel
  // arguments, not one by one between those reads
  asm volatile("" ::"s"(p.num_blocks), "s"(p.blocks), "s"(p.tflags), "s"(p.sorted_pairs), "s"(p.topk_weights),
               "s"(p.t0.unscale), "s"(p.t0.general), "s"(p.t1.unscale), "s"(p.t1.general));

  // ---- work item: XCD-contiguous ranges over (tile, column block)
  const int nblk = min(*p.num_blocks, p.max_blocks);
  const int N = p.N, K = p.K;
  const int nbn = (N + OUT_COLS - 1) / OUT_COLS;
  const int total = nblk * nbn;
  const int span = (total + kNumXcd - 1) / kNumXcd;
  const int local = blockIdx.x / kNumXcd;
  if (local >= span) return;
  const int item = (blockIdx.x % kNumXcd) * span + local;
  if (item >= total) return;
  const int tile = item / nbn, nb = item % nbn;
  const int e = p.blocks[3 * tile], row0 = p.blocks[3 * tile + 1], rows = p.blocks[3 * tile + 2];
  // S7: a tile some of whose h rows carry nonzero exponents takes the scaled
  // path below (uniform)
  const int tflag = GATE_UP ? 0 : p.tflags[tile];
  // the entry's words and the flag are read in one round trip (else the
  // compiler reads rows only after the checks on e)
  asm volatile("" ::"s"(e), "s"(row0), "s"(rows), "s"(tflag));
  const bool scaled = tflag != 0;
  // a malformed block map is skipped, never dereferenced out of bounds
  if (e < 0 || e >= p.E || rows <= 0 || rows > BM || row0 < 0 || row0 > p.P - rows) return;
  // the expert's factors 2^-c (its weights were scaled by 2^c at pack time),
  // used by the epilogue, and dequantisation form, used from the first
  // multiply on: the loads are issued here and waited for only there, after
  // the first copies of the ring are in flight (uniform: scalar loads)
  const float us0 = p.t0.unscale[e], us1 = GATE_UP ? p.t1.unscale[e] : 1.0f;
  const bool gen = !DENSE && (p.t0.general[e] | (GATE_UP ? p.t1.general[e] : 0u)) != 0;

  // ---- A loads: instruction j covers rows 8j..8j+7; lane l fills physical
  // chunk l % 8 of row r = 8j + l / 8, i.e. logical chunk (l % 8) ^ a_swz(r).
  // The half-height loop (rows < BM / 2) with fewer first-half copies than
  // waves: wave w issues copy w mod (A_INSTR / 2), the same bytes to the
  // same LDS place as another wave (a harmless duplicate), so every wave
  // issues the same number of copies per slab.
  constexpr bool HALF_DUP = MB > 1 && A_PER_WAVE * (MB / 2) < MB;
  constexpr int NA = A_PER_WAVE + (HALF_DUP ? 1 : 0);
  int arow[NA], a_lds[NA], achunk[NA];
#pragma unroll
  for (int a = 0; a < NA; a++) {
    const int j = a == A_PER_WAVE ? wave % (A_INSTR / 2) : A_INSTR >= WAVES ? wave + WAVES * a : wave % A_INSTR;
    arow[a] = row0 + min(8 * j + (lane >> 3), rows - 1);
    a_lds[a] = 1024 * j;
    achunk[a] = (lane & 7) ^ a_swz(8 * j + (lane >> 3));
  }
  if constexpr (GATE_UP) {
    // token rows of the slots' pairs: every pair is read before any is used
    // (one round trip); an invalid pair reads a valid row (never stored)
    int pr[NA];
#pragma unroll
    for (int a = 0; a < NA; a++) pr[a] = p.sorted_pairs[arow[a]];
#pragma unroll
    for (int a = 0; a < NA; a++) arow[a] = min(max(pr[a], 0), p.P - 1) / p.top_k;
  }
  // A copies a wave issues for a tile of `rows` rows: instruction j is
  // needed only while 8 j < rows (with j = wave + WAVES a, the copies of 8-row
  // groups past the tile are skipped; those LDS rows then hold stale values
  // whose products land only in rows that are never stored).  Uniform per
  // wave, so the slab waits below count this wave's own copies.  Only for
  // tiles of up to 64 rows: at T = 512 a tile's rows are spread around 32
  // (gate/up -4%, down -3%), while 128-row tiles, nearly all full at the T
  // that selects them, measured 1-2% slower with the runtime count.
  auto a_copies = [&](int apw) -> int {
    if constexpr (HALF_DUP || A_INSTR < WAVES || MB > 2) return apw;
    const int ng = (rows + 7) >> 3;
    return min(apw, max(0, (ng - wave + WAVES - 1) / WAVES));
  };
  const half_t* asrc[NA];
#pragma unroll
  for (int a = 0; a < NA; a++) asrc[a] = p.a + (size_t)arow[a] * K + 8 * achunk[a];
  const half_t* const asrc_h = HALF_DUP ? asrc[NA - 1] : nullptr;
  const int a_lds_h = HALF_DUP ? a_lds[NA - 1] : 0;

  // ---- S7 routing weights of the tile's rows (0 past the tile)
  if (!GATE_UP && tid < BM) {
    const int pair = tid < rows ? p.sorted_pairs[row0 + tid] : -1;
    row_w[tid] = (pair >= 0 && pair < p.P) ? p.topk_weights[pair] : 0.0f;
  }

  // packed 32-column block (index into the bank's N/32) of weight-column
  // block jb (0..15) of this tile, and its bank: in S6 block jb holds gate
  // (jb even) or up (jb odd) columns 32 (jb / 2).., in S7 down columns 32 jb..
  // Blocks past N reload the last block (results never stored).
  const int nbl = N / 32;
  auto block_of = [&](int jb, const moe_w4_packed*& bank) -> int {
    int n0;
    if (GATE_UP) {
      bank = (jb & 1) ? &p.b1 : &p.b0;
      n0 = nb * OUT_COLS + (jb >> 1) * 32;
    } else {
      bank = &p.b0;
      n0 = nb * OUT_COLS + jb * 32;
    }
    return (size_t)e * nbl + (min(n0, N - 32) >> 5);
  };

  // ---- B loads: instruction j is weight-column block j, one 1 KiB packed
  // block per slab ([32 columns][2 halves] x 16 bytes) inside its chunk's
  // 4 KiB run.
  const int slabs = K / kSlabK;
  const uint32_t* bsrc[B_PER_WAVE];
#pragma unroll
  for (int b = 0; b < B_PER_WAVE; b++) {
    const int j = DENSE ? 2 * wave + (b >> 2) : B_PER_WAVE * wave + b;
    const moe_w4_packed* bank;
    const int blk = block_of(j, bank);
    if (DENSE)  // piece b & 3 of the block's 4 KiB per slab
      bsrc[b] = bank->words + ((size_t)(blk >> 2) * slabs * 4 + (blk & 3)) * 1024 + 256 * (b & 3) + 4 * lane;
    else
      bsrc[b] = bank->words + ((size_t)(blk >> 2) * slabs * 4 + (blk & 3)) * 256 + 4 * lane;
  }

  // ---- scale / bias words: stage layout [reduction half t][kBCols columns];
  // instruction t of wave w covers columns 64w..64w+63 (blocks 2w, 2w+1),
  // 128 contiguous bytes per block, group g = (64 s + 32 t) / G.
  const int log2G = p.log2_G;
  const int gpr = K >> log2G;  // groups per row
  const uint32_t* ssrc;
  {
    const moe_w4_packed* bank;
    const int blk = block_of(2 * wave + (lane >> 5), bank);
    ssrc = bank->sb + (size_t)(blk >> 2) * gpr * 128 + (blk & 3) * 32 + (lane & 31);
  }
  bool active = true;
  {
    const int first = nb * OUT_COLS + (GATE_UP ? wave * 32 : wave * 64);
    active = first < N;  // uniform per wave
  }

  floatx16_t acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++) acc[mb][cb] = floatx16_t{};

  // The main loop for MBA active 32-row blocks (MBA = MB, or MB / 2 when the
  // tile's rows fit in the first half: the copies of the other half's
  // activations and its MFMAs are skipped; its accumulators stay zero and
  // its rows are never stored).
  // GEN: the general dequantisation (see dequant_word_gen).  SCALED (S7):
  // h rows with nonzero exponents; each slab's activations are brought to
  // their row's largest exponent in LDS before the multiplies (one stage, no
  // copies in flight across slabs: such tiles are rare).  PRO: this call
  // issues the ring's first copies itself (else the caller did, through
  // prologue() with the same MBA, before choosing GEN).
  auto pipeline = [&](auto mba, auto gen_tag, auto scaled_tag, auto pro_tag) {
    constexpr int MBA = decltype(mba)::value;
    constexpr bool GEN = decltype(gen_tag)::value != 0;
    constexpr bool SCALED = decltype(scaled_tag)::value != 0;
    constexpr bool PRO = decltype(pro_tag)::value != 0;
    constexpr bool DUP = HALF_DUP && MBA < MB;
    constexpr int APW = DUP ? 1 : A_PER_WAVE * MBA / MB;  // activation copies used (rows < 32 MBA)
    // this wave's copies per slab: DA = na + B_PER_WAVE + S_PER_WAVE
    const int na = a_copies(APW);
    auto issue = [&](int s, int stage) {
      char* base = lds + stage * STAGE;
#pragma unroll
      for (int a = 0; a < APW; a++)
        if (a < na) lds_load16((DUP ? asrc_h : asrc[a]) + s * kSlabK, base + (DUP ? a_lds_h : a_lds[a]));
#pragma unroll
      for (int b = 0; b < B_PER_WAVE; b++)
        lds_load16(bsrc[b] + s * (DENSE ? 4096 : 1024), base + A_BYTES + 1024 * (B_PER_WAVE * wave + b));
#pragma unroll
      for (int t = 0; t < S_PER_WAVE; t++)
        lds_load4(ssrc + ((s * kSlabK + 32 * t) >> log2G) * 128,
                  base + A_BYTES + kBStage + 4 * kBCols * t + 256 * wave);
    };

    auto compute = [&](int stage) {
      const char* base = lds + stage * STAGE;
      if constexpr (DENSE || GATE_UP || WAVES == 8) {
        // reads placed by the compiler: the expanded weights of the unfused
        // ablation; 8-wave tiles, whose register budget holds no fragments
        // ahead; and the gate/up GEMM, where reading ahead measured 3-8%
        // slower (its 32-slab loop keeps the copy addresses in registers
        // only without the extra fragments)
        u32x4 q[2];
        half2_t s2[2], b2[2], n2[2];
        if constexpr (!DENSE) {
#pragma unroll
          for (int cb = 0; cb < 2; cb++)
            q[cb] = *reinterpret_cast<const u32x4*>(base + A_BYTES + (wave * 64 + cb * 32 + col) * 32 +
                                                    16 * khalf);
#pragma unroll
          for (int cb = 0; cb < 2; cb++) {
            const uint32_t sb = reinterpret_cast<const uint32_t*>(
                base + A_BYTES + kBStage)[(G32 ? khalf : 0) * kBCols + wave * 64 + cb * 32 + col];
            sb_pairs(sb, s2[cb], b2[cb]);
            if constexpr (GEN) n2[cb] = s2[cb] * half2_t{(half_t)-32.0f, (half_t)-32.0f};
          }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
          half8_t bf[2];
#pragma unroll
          for (int cb = 0; cb < 2; cb++) {
            if constexpr (DENSE)
              bf[cb] = *reinterpret_cast<const half8_t*>(base + A_BYTES + (2 * wave + cb) * 4096 +
                                                         1024 * i + 16 * (2 * col + khalf));
            else if constexpr (GEN)
              bf[cb] = __builtin_bit_cast(half8_t, dequant_word_gen(q[cb][i], s2[cb], n2[cb], b2[cb]));
            else
              bf[cb] = __builtin_bit_cast(half8_t, dequant_word(q[cb][i], s2[cb], b2[cb]));
          }
#pragma unroll
          for (int mb = 0; mb < MBA; mb++) {
            const int r = mb * 32 + col;
            const half8_t af = *reinterpret_cast<const half8_t*>(
                base + r * 128 + (((4 * khalf + i) ^ a_swz(col)) << 4));
#pragma unroll
            for (int cb = 0; cb < 2; cb++)
              acc[mb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[cb], acc[mb][cb], 0, 0, 0);
          }
        }
      } else {
        // the slab's LDS reads are issued ahead, in use order: the two code
        // blocks, the two (scale, bias) words, then the activation fragments
        // of the first PD = 2 steps, and at each later step those of step +
        // 1; step i then waits only until its own fragments have landed (LDS
        // reads complete in order), instead of a full round trip before
        // every pair of MFMAs (S7: 255-260 -> 241 us at T = 8192; reading
        // all four steps ahead gained less, 251)
        constexpr int PD = 2;
        u32x4 q[2], af[4][MBA];
        uint32_t sbw[2];
#pragma unroll
        for (int cb = 0; cb < 2; cb++)
          q[cb] = lds_read16(base + A_BYTES + (wave * 64 + cb * 32 + col) * 32 + 16 * khalf);
#pragma unroll
        for (int cb = 0; cb < 2; cb++)
          sbw[cb] = lds_read4(base + A_BYTES + kBStage + 4 * ((G32 ? khalf : 0) * kBCols + wave * 64 + cb * 32 + col));
        auto read_a = [&](int i) {
#pragma unroll
          for (int mb = 0; mb < MBA; mb++)
            af[i][mb] = lds_read16(base + (mb * 32 + col) * 128 + (((4 * khalf + i) ^ a_swz(col)) << 4));
        };
#pragma unroll
        for (int i = 0; i < PD; i++) read_a(i);
        half2_t s2[2], b2[2], n2[2];
        auto step = [&](auto itag) {
          constexpr int I = decltype(itag)::value;
          constexpr int LAST = I + PD - 1 < 3 ? I + PD - 1 : 3;  // last step whose fragments are issued
          if constexpr (I >= 1 && I + PD - 1 <= 3) read_a(I + PD - 1);
          lds_wait_n<MBA * (LAST - I)>(af[I][0]);
#pragma unroll
          for (int mb = 1; mb < MBA; mb++) lds_tie(af[I][mb]);
          if constexpr (I == 0) {
#pragma unroll
            for (int cb = 0; cb < 2; cb++) {
              lds_tie(q[cb]);
              lds_tie(sbw[cb]);
              sb_pairs(sbw[cb], s2[cb], b2[cb]);
              if constexpr (GEN) n2[cb] = s2[cb] * half2_t{(half_t)-32.0f, (half_t)-32.0f};
            }
          }
          half8_t bf[2];
#pragma unroll
          for (int cb = 0; cb < 2; cb++) {
            if constexpr (GEN)
              bf[cb] = __builtin_bit_cast(half8_t, dequant_word_gen(q[cb][I], s2[cb], n2[cb], b2[cb]));
            else
              bf[cb] = __builtin_bit_cast(half8_t, dequant_word(q[cb][I], s2[cb], b2[cb]));
          }
#pragma unroll
          for (int mb = 0; mb < MBA; mb++)
#pragma unroll
            for (int cb = 0; cb < 2; cb++)
              acc[mb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, af[I][mb]), bf[cb],
                                                                   acc[mb][cb], 0, 0, 0);
        };
        step(IntTag<0>{});
        step(IntTag<1>{});
        step(IntTag<2>{});
        step(IntTag<3>{});
      }
    };

    // slab s lives in stage s % STAGES.  Every slab step of a wave issues the
    // same copies (slabs past the end reload the last slab into a stage that
    // is never read again), so when slab s is about to be computed exactly the
    // copies of STAGES - 2 later slabs ((STAGES - 2) * DA instructions of this
    // wave) were issued after its own: waiting until at most that many are
    // outstanding means slab s has landed.  Right after the barrier, stage
    // (s + STAGES - 1) % STAGES (computed last at slab s - 1, by every wave)
    // is refilled with slab s + STAGES - 1.
    const int S = slabs;
    if constexpr (SCALED) {
      const int nbk = K / 16;  // exponent bytes per h row
      for (int s = 0; s < S; s++) {
        issue(s, 0);
        wait_vm_barrier<0>();
        // activation chunk (row r, physical chunk pc) holds reduction indices
        // 64 s + 8 (pc ^ a_swz(r)) .. + 7, inside 16-column block 4 s + lc / 2
        for (int c = tid; c < 32 * MBA * 8; c += 64 * WAVES) {
          const int r = c >> 3, pc = c & 7, lc = pc ^ a_swz(r);
          const int d = p.hexp[(size_t)(row0 + min(r, rows - 1)) * nbk + 4 * s + (lc >> 1)] - erow[r];
          if (d != 0) {
            uint4* at = reinterpret_cast<uint4*>(lds + r * 128 + pc * 16);
            *at = scale_half8(*at, d);
          }
        }
        // the exponent loads and the rescaled LDS writes complete, then all waves meet
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        compute(0);
        asm volatile("s_barrier" ::: "memory");  // stage 0 is refilled next
      }
    } else {
      if constexpr (PRO) {
#pragma unroll
        for (int j = 0; j < STAGES - 1; j++) issue(min(j, S - 1), j);
      }
      for (int s = 0; s < S; s++) {
        wait_vm_barrier_n<(STAGES - 2) * (B_PER_WAVE + S_PER_WAVE), STAGES - 2, APW>(na);
        issue(min(s + STAGES - 1, S - 1), (s + STAGES - 1) % STAGES);
        compute(s % STAGES);
      }
    }
  };
  if (!GATE_UP && scaled) {
    // each row's largest exponent (rows past the tile repeat its last row);
    // the epilogue scales the row's output by 2^that (with the routing weight)
    const int nbk = K / 16;
    for (int r = tid; r < BM; r += 64 * WAVES) {
      const uint32_t* er = reinterpret_cast<const uint32_t*>(p.hexp + (size_t)(row0 + min(r, rows - 1)) * nbk);
      int m = -128;
      for (int b = 0; b < nbk / 4; b++) m = max(m, max_i8x4(er[b]));
      erow[r] = m;
    }
    __syncthreads();
  }
  // uniform per workgroup: every wave takes the same branch.  The ring's
  // first copies are issued (for the chosen tile height) before the branch on
  // the dequantisation form, whose scalar loads then overlap them.
  auto prologue = [&](auto mba) {
    constexpr int MBA = decltype(mba)::value;
    constexpr bool DUP = HALF_DUP && MBA < MB;
    constexpr int APW = DUP ? 1 : A_PER_WAVE * MBA / MB;
    const int na = a_copies(APW);
#pragma unroll
    for (int j = 0; j < STAGES - 1; j++) {
      const int s = min(j, slabs - 1);
      char* base = lds + j * STAGE;
#pragma unroll
      for (int a = 0; a < APW; a++)
        if (a < na) lds_load16((DUP ? asrc_h : asrc[a]) + s * kSlabK, base + (DUP ? a_lds_h : a_lds[a]));
#pragma unroll
      for (int b = 0; b < B_PER_WAVE; b++)
        lds_load16(bsrc[b] + s * (DENSE ? 4096 : 1024), base + A_BYTES + 1024 * (B_PER_WAVE * wave + b));
#pragma unroll
      for (int t = 0; t < S_PER_WAVE; t++)
        lds_load4(ssrc + ((s * kSlabK + 32 * t) >> log2G) * 128,
                  base + A_BYTES + kBStage + 4 * kBCols * t + 256 * wave);
    }
  };
  constexpr int MBH = MB > 1 ? MB / 2 : 1;
  if (!GATE_UP && scaled) {
    if (gen) pipeline(IntTag<MB>{}, IntTag<DENSE ? 0 : 1>{}, IntTag<1>{}, IntTag<1>{});
    else pipeline(IntTag<MB>{}, IntTag<0>{}, IntTag<1>{}, IntTag<1>{});
  } else if (MB > 1 && rows <= BM / 2) {
    prologue(IntTag<MBH>{});
    if (gen) pipeline(IntTag<MBH>{}, IntTag<DENSE ? 0 : 1>{}, IntTag<0>{}, IntTag<0>{});
    else pipeline(IntTag<MBH>{}, IntTag<0>{}, IntTag<0>{}, IntTag<0>{});
  } else {
    prologue(IntTag<MB>{});
    if (gen) pipeline(IntTag<MB>{}, IntTag<DENSE ? 0 : 1>{}, IntTag<0>{}, IntTag<0>{});
    else pipeline(IntTag<MB>{}, IntTag<0>{}, IntTag<0>{}, IntTag<0>{});
  }

  // ---- epilogue.  Accumulator register r of lane l holds row
  // 8*(r/4) + 4*(l/32) + r%4 and column l%32 of each 32x32 block.
  if (GATE_UP) {
    // h = silu(gate) * up in fp32 into an LDS tile [BM][OUT_COLS] (operand
    // order: column 8g + j at 8g + interleaved_pos(j)), then stored as fp16
    // with one exponent per row and 16-column block (h_block_exp), 16-byte
    // row stores.  The ring is free once every copy has landed (the last
    // steps reloaded the last slab) and every wave has finished its MFMAs.
    wait_vm<0>();
    __syncthreads();
    float* tile_f = reinterpret_cast<float*>(lds);
    if (active) {
      const int lc = wave * 32 + (col & ~7) + interleaved_pos(col & 7);
#pragma unroll
      for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int row = mb * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
          tile_f[row * OUT_COLS + lc] = silu_mul(acc[mb][0][r] * us0, acc[mb][1][r] * us1);
        }
    }
    __syncthreads();
    const int n0 = nb * OUT_COLS;
    const int chunks = min(OUT_COLS, N - n0) / 8;  // 16-byte pieces per row (an even count)
    bool any = false;
    // every lane runs every round, so that lane pairs (2i, 2i + 1) -- the two
    // 8-column pieces of one 16-column block -- exchange their maxima (both
    // store the block's exponent byte)
    auto rounds = [&](auto full_tag) {
      constexpr bool FULLC = decltype(full_tag)::value != 0;  // chunks == OUT_COLS / 8 (a power of two)
      constexpr int LOGC = __builtin_ctz(OUT_COLS / 8);
      const int total8 = rows * chunks;
      for (int base = 0; base < total8; base += 64 * WAVES) {
        const int idx = base + tid;
        const bool ok = idx < total8;
        const int row = !ok ? 0 : FULLC ? idx >> LOGC : idx / chunks;
        const int ch = !ok ? 0 : FULLC ? idx & (OUT_COLS / 8 - 1) : idx % chunks;
        const float4 v0 = *reinterpret_cast<const float4*>(tile_f + row * OUT_COLS + 8 * ch);
        const float4 v1 = *reinterpret_cast<const float4*>(tile_f + row * OUT_COLS + 8 * ch + 4);
        float m8;
        asm("v_max3_f32 %0, |%1|, |%2|, |%3|\n\tv_max3_f32 %0, %0, |%4|, |%5|\n\tv_max3_f32 %0, %0, |%6|, |%7|\n\t"
            "v_max_f32 %0, %0, |%8|"
            : "=&v"(m8) : "v"(v0.x), "v"(v0.y), "v"(v0.z), "v"(v0.w), "v"(v1.x), "v"(v1.y), "v"(v1.z), "v"(v1.w));
        uint32_t mu = __float_as_uint(m8);
        mu = max(mu, (uint32_t)__builtin_amdgcn_mov_dpp((int)mu, 0xB1, 0xF, 0xF, true));
        const int ex = h_block_exp_bits(mu);
        if (ok) {
          const half2_t o0 = {(half_t)ldexpf(v0.x, -ex), (half_t)ldexpf(v0.y, -ex)};
          const half2_t o1 = {(half_t)ldexpf(v0.z, -ex), (half_t)ldexpf(v0.w, -ex)};
          const half2_t o2 = {(half_t)ldexpf(v1.x, -ex), (half_t)ldexpf(v1.y, -ex)};
          const half2_t o3 = {(half_t)ldexpf(v1.z, -ex), (half_t)ldexpf(v1.w, -ex)};
          *reinterpret_cast<uint4*>(reinterpret_cast<half_t*>(p.out) + (size_t)(row0 + row) * N + n0 + 8 * ch) =
              make_uint4(__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1),
                         __builtin_bit_cast(uint32_t, o2), __builtin_bit_cast(uint32_t, o3));
          p.hexp[(size_t)(row0 + row) * (N / 16) + (n0 + 8 * ch) / 16] = (int8_t)ex;
          any |= ex != 0;
        }
      }
    };
    if (chunks == OUT_COLS / 8) rounds(IntTag<1>{});
    else rounds(IntTag<0>{});
    if (any) p.tflags[tile] = 1;
  } else if constexpr (PACK) {
    // The accumulators go through a wave-private fp32 LDS tile of 32 rows x
    // 64 columns (one 32-row block at a time) and come back as 8 consecutive
    // columns of one row per lane: lane l takes row 8k + l / 8 of the block
    // (k = 0..3) at columns 8 (l % 8) .. + 7 of the wave's 64.  Row pitch 64
    // words; a row's columns are XORed with 32 when its bit 2 is set and with
    // 4 when its bit 0 is, so the two half-waves of a column write (rows r
    // and r + 4) fall on disjoint banks, and so do the two rows each 16-lane
    // group of a 16-byte read covers.  The two lanes of one row's 16-column
    // block exchange their maxima (one DPP step), hence its exponent; each
    // lane stores its 8 int16 mantissas (8 lanes: 128 contiguous bytes of a
    // row) and the block's exponent byte (both lanes store the same byte).
    // The ring is free once every copy has landed and every wave has
    // finished its MFMAs.
    static_assert(WAVES * 32 * 64 * 4 <= STAGES * STAGE, "epilogue tile must fit the ring");
    wait_vm<0>();
    __syncthreads();
    if (!active) return;
    float* const tile = reinterpret_cast<float*>(lds) + wave * 32 * 64;
    auto swz = [](int row) { return (row & 4 ? 32 : 0) ^ (row & 1 ? 4 : 0); };
    const int q = lane & 7, rq = lane >> 3;  // column octet, row within 8
    const size_t mstride = (size_t)N * 2, estride = (size_t)N / 16;
    const int c0 = nb * OUT_COLS + wave * 64;
    // this lane's row rq of the tile: the later rows are uniform offsets from it
    char* const lane_out = reinterpret_cast<char*>(p.out) + (size_t)(row0 + rq) * mstride + (size_t)(c0 + 8 * q) * 2;
    int8_t* const lane_exp = p.yexp + (size_t)(row0 + rq) * estride + c0 / 16 + (q >> 1);
    auto block = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value != 0;
#pragma unroll
      for (int mb = 0; mb < MB; mb++) {
        if (!FULL && mb * 32 >= rows) break;  // (uniform) no row of this block is stored
        // register r of lane l: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
        for (int cb = 0; cb < 2; cb++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int row = 8 * (r >> 2) + 4 * khalf + (r & 3);
            tile[row * 64 + ((cb * 32 + col) ^ swz(row))] = acc[mb][cb][r];
          }
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const int rr = 8 * k + rq;
          const float4 v0 = *reinterpret_cast<const float4*>(tile + rr * 64 + ((8 * q) ^ swz(rr)));
          const float4 v1 = *reinterpret_cast<const float4*>(tile + rr * 64 + ((8 * q + 4) ^ swz(rr)));
          const int row = mb * 32 + rr;
          const float w = (scaled ? ldexpf(row_w[row], erow[row]) : row_w[row]) * us0;
          // the block's largest |a|: the bits of non-negative floats order as
          // unsigned integers, so the pair exchange takes an integer maximum
          float m8;
          asm("v_max3_f32 %0, |%1|, |%2|, |%3|\n\tv_max3_f32 %0, %0, |%4|, |%5|\n\tv_max3_f32 %0, %0, |%6|, |%7|\n\t"
              "v_max_f32 %0, %0, |%8|"
              : "=&v"(m8) : "v"(v0.x), "v"(v0.y), "v"(v0.z), "v"(v0.w), "v"(v1.x), "v"(v1.y), "v"(v1.z), "v"(v1.w));
          uint32_t m = __float_as_uint(m8);
          m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
          const int ex = y16_exp_bits(__uint_as_float(m) * fabsf(w));
          const float ws = ex == -128 ? 0.0f : ldexpf(w, -ex);
          const uint2 lo = y16_pack4(v0.x, v0.y, v0.z, v0.w, ws), hi = y16_pack4(v1.x, v1.y, v1.z, v1.w, ws);
          if (FULL || row < rows) {
            *reinterpret_cast<uint4*>(lane_out + (size_t)(mb * 32 + 8 * k) * mstride) = make_uint4(lo.x, lo.y, hi.x, hi.y);
            lane_exp[(size_t)(mb * 32 + 8 * k) * estride] = (int8_t)ex;
          }
        }
      }
    };
    if (rows == BM) block(IntTag<1>{});
    else block(IntTag<0>{});
  } else {
    if (!active) return;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = mb * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row >= rows) continue;
        const float w = (scaled ? ldexpf(row_w[row], erow[row]) : row_w[row]) * us0;
        float* orow = reinterpret_cast<float*>(p.out) + (size_t)(row0 + row) * N;
#pragma unroll
        for (int cb = 0; cb < 2; cb++)
          orow[nb * OUT_COLS + wave * 64 + cb * 32 + col] = w * acc[mb][cb][r];
      }
    }
  }
}


// x bf16 -> fp16, each 8-element chunk interleaved (0,4,1,5,2,6,3,7); the
// per-tile flags of the gate/up kernel cleared.
__global__ __launch_bounds__(256) void stage_x_kernel(const uint4* __restrict__ in,
                                                      uint4* __restrict__ out, int64_t n8,
                                                      int32_t* __restrict__ tflags, int64_t nflags) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nflags) tflags[i] = 0;
  if (i >= n8) return;
  out[i] = bf16x8_to_half_interleaved(in[i]);
}

template <int MODE, bool PACK>
hipError_t launch_mode(const GemmArgs& a, hipStream_t s) {
  const int64_t P = (int64_t)a.T * a.top_k;
  const int64_t max_blocks = a.grid_tiles >= 0 ? a.grid_tiles : P / a.block_m + (P < a.E ? P : a.E);
  if (max_blocks == 0) return hipSuccess;
  const int log2_G = a.G == 32 ? 5 : a.G == 64 ? 6 : 7;  // G in {32, 64, 128}
  MfmaParams p{a.a, a.b0, a.b1, a.sorted_pairs, a.topk_weights, a.blocks, a.num_blocks, a.out,
               a.t0, a.t1, a.hexp, a.tflags, a.yexp, a.N, a.K, log2_G, a.top_k, a.E, (int)P,
               (int)max_blocks};
  // 4 waves (256 weight columns) per workgroup and two or three workgroups
  // per CU, so one workgroup's prologue and epilogue overlap another's main
  // loop; 64- and 128-row tiles use a 3-stage ring to fit three and two
  // workgroups' LDS (and 64-row tiles a register budget for three)
  const int bcols = 256;
  const int out_cols = MODE == MOE_GEMM_GATE_UP_SWIGLU ? bcols / 2 : bcols;
  const int64_t items = max_blocks * ((a.N + out_cols - 1) / out_cols);
  const int64_t grid = ((items + kNumXcd - 1) / kNumXcd) * kNumXcd;
  const bool g32 = a.G == 32;
  if (a.dense) {  // expanded fp16 weights: larger B stages, one workgroup per CU
    switch (a.block_m) {
      case 32: w4_mfma_kernel<MODE, 1, 4, false, 4, 1, PACK, true><<<grid, 256, 0, s>>>(p); break;
      case 64: w4_mfma_kernel<MODE, 2, 4, false, 3, 1, PACK, true><<<grid, 256, 0, s>>>(p); break;
      case 128: w4_mfma_kernel<MODE, 4, 4, false, 3, 1, PACK, true><<<grid, 256, 0, s>>>(p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (MODE == MOE_GEMM_DOWN && a.block_m == 64 && !g32) {
    // S7 on 64-row tiles (K = I: few slabs per item, so an item is mostly its
    // prologue, first copies and epilogue): four 4-wave workgroups per CU on
    // a 2-stage ring, so at T = 512 every item is resident in one round
    // (36 -> 32 us against 8-wave workgroups with 512 columns, two per CU)
    w4_mfma_kernel<MODE, 2, 4, false, 2, 4, PACK><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
  }
  switch (a.block_m * 2 + (g32 ? 1 : 0)) {
    case 64: w4_mfma_kernel<MODE, 1, 4, false, 4, 2, PACK><<<grid, 256, 0, s>>>(p); break;
    case 65: w4_mfma_kernel<MODE, 1, 4, true, 4, 2, PACK><<<grid, 256, 0, s>>>(p); break;
    case 128: w4_mfma_kernel<MODE, 2, 4, false, 3, 3, PACK><<<grid, 256, 0, s>>>(p); break;
    // group size 32 stages two (scale, bias) copies per slab: three 64-row
    // workgroups would need 166 KB of LDS, so two share a CU, with a deeper ring
    case 129: w4_mfma_kernel<MODE, 2, 4, true, 4, 2, PACK><<<grid, 256, 0, s>>>(p); break;
    case 256: w4_mfma_kernel<MODE, 4, 4, false, 3, 2, PACK><<<grid, 256, 0, s>>>(p); break;
    case 257: w4_mfma_kernel<MODE, 4, 4, true, 3, 2, PACK><<<grid, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// y[t][:] = sum_j y_sorted[pair_slot[t*k + j]][:], j ascending, fp32: the
// k weighted expert outputs of a token added in a fixed order, so the layer
// output is deterministic.  All k slot indices and then all k rows are
// loaded before the sum (KMAX >= k, guards for j >= k), so a thread has k
// row loads in flight instead of k round trips.  Out-of-range slots are
// skipped.
// fp32 y_sorted: one thread per 4 columns of y (16 bytes in per slot, 16
// out).  With out: also out = bf16(residual + y), four values per thread.
template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float4* __restrict__ y_sorted,
                                                      const int32_t* __restrict__ pair_slot,
                                                      float4* __restrict__ y, int T, int H4,
                                                      int k, const uint2* __restrict__ residual,
                                                      uint2* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * H4) return;
  const int t = (int)(i / H4), c = (int)(i % H4);
  const int P = T * k;
  int slot[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++) {
    slot[j] = j < k ? pair_slot[(size_t)t * k + j] : -1;
    if (slot[j] >= P) slot[j] = -1;
  }
  float4 v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++)
    v[j] = slot[j] < 0 ? make_float4(0.f, 0.f, 0.f, 0.f) : y_sorted[(size_t)slot[j] * H4 + c];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < KMAX; j++) {
    if (slot[j] < 0) continue;
    acc.x += v[j].x;
    acc.y += v[j].y;
    acc.z += v[j].z;
    acc.w += v[j].w;
  }
  y[i] = acc;
  if (out) out[i] = residual_add_bf16x4(residual[i], acc);
}

// The same over y16e block floating point: one thread per 8 columns of y
// (per slot 16 bytes of mantissas and the block's exponent byte in, 32
// bytes out); the decoded values are exact in fp32, so the sum is the fp32
// sum of the decoded rows in choice order.
template <int KMAX>
__global__ __launch_bounds__(256) void combine16_kernel(const uint4* __restrict__ ym,
                                                        const int8_t* __restrict__ ye,
                                                        const int32_t* __restrict__ pair_slot,
                                                        float4* __restrict__ y, int T, int H8,
                                                        int k, const uint2* __restrict__ residual,
                                                        uint2* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * H8) return;
  const int t = (int)(i / H8), c = (int)(i % H8);
  const int P = T * k;
  int slot[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++) {
    slot[j] = j < k ? pair_slot[(size_t)t * k + j] : -1;
    if (slot[j] >= P) slot[j] = -1;
  }
  uint4 m[KMAX];
  int ex[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; j++) {
    const size_t row = (size_t)(slot[j] < 0 ? 0 : slot[j]);
    m[j] = ym[row * H8 + c];
    ex[j] = ye[row * (H8 / 2) + (c >> 1)];
  }
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; q++) acc[q] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; j++) {
    if (slot[j] < 0) continue;
    float v[8];
    y16_unpack8(m[j], ex[j], v);
#pragma unroll
    for (int q = 0; q < 8; q++) acc[q] += v[q];
  }
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const float4 a4 = make_float4(acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]);
    y[2 * i + h] = a4;
    if (out) out[2 * i + h] = residual_add_bf16x4(residual[2 * i + h], a4);
  }
}

}  // namespace

hipError_t launch_w4_mfma(const GemmArgs& a, hipStream_t s) {
  if (a.mode == MOE_GEMM_GATE_UP_SWIGLU) return launch_mode<MOE_GEMM_GATE_UP_SWIGLU, false>(a, s);
  return a.y16e ? launch_mode<MOE_GEMM_DOWN, true>(a, s) : launch_mode<MOE_GEMM_DOWN, false>(a, s);
}

hipError_t launch_stage_x(const uint16_t* x, half_t* xh, int64_t n_elems, int32_t* tflags,
                          int64_t nflags, hipStream_t s) {
  const int64_t n8 = n_elems / 8;
  const int64_t n = std::max(n8, tflags ? nflags : 0);
  stage_x_kernel<<<(n + 255) / 256, 256, 0, s>>>(reinterpret_cast<const uint4*>(x),
                                                 reinterpret_cast<uint4*>(xh), n8, tflags,
                                                 tflags ? nflags : 0);
  return hipGetLastError();
}

template <int KMAX>
void launch_combine_k(const void* ys, const int8_t* yexp, const int32_t* pair_slot, float4* yo, int T,
                      int H, int k, const uint2* res, uint2* out, hipStream_t s) {
  if (yexp) {
    const int64_t n = (int64_t)T * (H / 8);
    combine16_kernel<KMAX><<<(n + 255) / 256, 256, 0, s>>>(reinterpret_cast<const uint4*>(ys), yexp,
                                                           pair_slot, yo, T, H / 8, k, res, out);
  } else {
    const int64_t n = (int64_t)T * (H / 4);
    combine_kernel<KMAX><<<(n + 255) / 256, 256, 0, s>>>(reinterpret_cast<const float4*>(ys), pair_slot,
                                                         yo, T, H / 4, k, res, out);
  }
}

hipError_t launch_combine(const void* y_sorted, const int8_t* yexp, const int32_t* pair_slot, float* y,
                          int T, int H, int k, hipStream_t s, const uint16_t* residual,
                          uint16_t* out) {
  float4* yo = reinterpret_cast<float4*>(y);
  const uint2* res = reinterpret_cast<const uint2*>(residual);
  uint2* o = reinterpret_cast<uint2*>(out);
  if (k <= 2) launch_combine_k<2>(y_sorted, yexp, pair_slot, yo, T, H, k, res, o, s);
  else if (k <= 4) launch_combine_k<4>(y_sorted, yexp, pair_slot, yo, T, H, k, res, o, s);
  else if (k <= 8) launch_combine_k<8>(y_sorted, yexp, pair_slot, yo, T, H, k, res, o, s);
  else launch_combine_k<16>(y_sorted, yexp, pair_slot, yo, T, H, k, res, o, s);  // k <= 16
  return hipGetLastError();
}

}  // namespace moe
