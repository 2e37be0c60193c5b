// gemm.hip -- S6/S7 grouped W4 GEMM on fp16 MFMA with the 4-bit
// dequantisation fused into the kernel (page "Perplexity's Lily engine beats
// MLX by 35% on M5 Max", architecture paragraph: dequantising inside the
// grouped GEMM keeps expanded 16-bit weights out of memory), the activation
// staging pass, and the S8 combine.
//
// Tile of one workgroup (256 threads = 4 waves): BM rows (slots of one
// expert, from the block map) x 128 output columns of the gate AND up banks
// (S6) or x 256 columns of the down bank (S7), over the whole reduction
// dimension in slabs of 64.  Every wave owns all BM rows and two 32-column
// blocks, so the codes it dequantises feed BM/32 MFMAs each.
//  - A (activations) is staged per slab in LDS, rows padded to 144 bytes so
//    that the 16-byte fragment reads of 8 consecutive rows hit distinct banks.
//  - B (weights) is read straight from HBM: each lane loads one 16-byte piece
//    (32 codes of one row) per column block per slab, and dequantises it in
//    registers against the row's fp16-converted scale and bias.
//  - MFMA v_mfma_f32_32x32x16_f16, fp32 accumulation.
//  - The next slab's A and B loads are issued before the current slab's
//    MFMAs; A is double-buffered in LDS, one barrier per slab.
// Work items (tile, column block) are spread over the 8 XCDs in contiguous
// ranges, so the column blocks of one tile, and the tiles of one expert, run
// on the same XCD at about the same time and share its L2.
#include "internal.h"

namespace moe {
namespace {

constexpr int kSlabK = 64;
constexpr int kLdsRow = kSlabK + 8;  // halfs per LDS row (144 bytes)

struct MfmaParams {
  const half_t* a;
  moe_w4_bank b0, b1;
  const int32_t* sorted_pairs;
  const float* topk_weights;
  const int32_t* blocks;
  const int32_t* num_blocks;
  void* out;
  int N, K, G, top_k, E, P, max_blocks;
};

template <int MODE, int MB>
__global__ __launch_bounds__(256, 2) void w4_mfma_kernel(const MfmaParams p) {
  constexpr int BM = MB * 32;
  constexpr int WG_N = MODE == MOE_GEMM_GATE_UP_SWIGLU ? 128 : 256;
  constexpr int CH = BM * (kSlabK / 8) / 256;  // 16-byte A chunks per thread per slab
  __shared__ half_t lds_a[2][BM * kLdsRow];
  __shared__ float row_w[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, khalf = lane >> 5;

  // ---- work item: XCD-contiguous ranges over (tile, column block)
  const int nblk = min(*p.num_blocks, p.max_blocks);
  const int nbn = p.N / WG_N;
  const int total = nblk * nbn;
  const int span = (total + kNumXcd - 1) / kNumXcd;
  const int local = blockIdx.x / kNumXcd;
  if (local >= span) return;
  const int item = (blockIdx.x % kNumXcd) * span + local;
  if (item >= total) return;
  const int tile = item / nbn, nb = item % nbn;
  const int e = p.blocks[3 * tile], row0 = p.blocks[3 * tile + 1], rows = p.blocks[3 * tile + 2];
  // a malformed block map is skipped, never dereferenced out of bounds
  if (e < 0 || e >= p.E || rows <= 0 || rows > BM || row0 < 0 || row0 > p.P - rows) return;
  const int K = p.K, N = p.N;

  // ---- A staging addresses (fixed rows for the whole K loop)
  const half_t* asrc[CH];
  int aoff[CH];
#pragma unroll
  for (int c = 0; c < CH; c++) {
    const int idx = tid + 256 * c, r = idx >> 3, ch = idx & 7;
    aoff[c] = r * kLdsRow + ch * 8;
    asrc[c] = nullptr;
    if (r < rows) {
      int srow = row0 + r;
      if (MODE == MOE_GEMM_GATE_UP_SWIGLU) {
        const int pair = p.sorted_pairs[row0 + r];
        srow = (pair >= 0 && pair < p.P) ? pair / p.top_k : -1;
      }
      if (srow >= 0) asrc[c] = p.a + (size_t)srow * K + ch * 8;
    }
  }
  if (MODE == MOE_GEMM_DOWN && tid < BM) {
    const int pair = tid < rows ? p.sorted_pairs[row0 + tid] : -1;
    row_w[tid] = (pair >= 0 && pair < p.P) ? p.topk_weights[pair] : 0.0f;
  }

  // ---- B addresses: column block cb of this wave
  const uint32_t* qp[2];
  const uint16_t* sp[2];
  const uint16_t* bp[2];
#pragma unroll
  for (int cb = 0; cb < 2; cb++) {
    const moe_w4_bank& bank = (MODE == MOE_GEMM_GATE_UP_SWIGLU && cb == 1) ? p.b1 : p.b0;
    const int n = MODE == MOE_GEMM_GATE_UP_SWIGLU ? nb * 128 + wave * 32 + col
                                                  : nb * 256 + wave * 64 + cb * 32 + col;
    const size_t rowi = (size_t)e * N + n;
    qp[cb] = bank.qweight + rowi * (K / 8) + 4 * khalf;
    sp[cb] = bank.scales + rowi * (K / p.G);
    bp[cb] = bank.biases + rowi * (K / p.G);
  }

  auto load_a = [&](int s, uint4* v) {
#pragma unroll
    for (int c = 0; c < CH; c++)
      v[c] = asrc[c] ? *reinterpret_cast<const uint4*>(asrc[c] + s * kSlabK) : make_uint4(0, 0, 0, 0);
  };
  auto store_a = [&](int buf, const uint4* v) {
#pragma unroll
    for (int c = 0; c < CH; c++) {
      uint4 d = MODE == MOE_GEMM_DOWN ? interleave_halves(v[c]) : v[c];
      *reinterpret_cast<uint4*>(&lds_a[buf][aoff[c]]) = d;
    }
  };
  auto load_b = [&](int s, uint4* q, uint16_t* sc, uint16_t* bi) {
    const int g = (s * kSlabK + 32 * khalf) / p.G;
#pragma unroll
    for (int cb = 0; cb < 2; cb++) {
      q[cb] = *reinterpret_cast<const uint4*>(qp[cb] + s * (kSlabK / 8));
      sc[cb] = sp[cb][g];
      bi[cb] = bp[cb][g];
    }
  };

  floatx16_t acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; mb++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++) acc[mb][cb] = floatx16_t{};

  uint4 av[CH];
  uint4 qc[2];
  uint16_t scl[2], bia[2];
  load_a(0, av);
  load_b(0, qc, scl, bia);
  store_a(0, av);
  __syncthreads();

  const int S = K / kSlabK;
  for (int s = 0; s < S; s++) {
    const bool more = s + 1 < S;
    uint4 qn[2];
    uint16_t scn[2], bin[2];
    if (more) {
      load_a(s + 1, av);
      load_b(s + 1, qn, scn, bin);
    }
    const half_t* abuf = lds_a[s & 1];
    half2_t s2[2], b2[2];
#pragma unroll
    for (int cb = 0; cb < 2; cb++) {
      s2[cb] = bf16_pair_to_half2(scl[cb]);
      b2[cb] = bf16_pair_to_half2(bia[cb]);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      half8_t bf[2];
#pragma unroll
      for (int cb = 0; cb < 2; cb++) {
        const uint32_t w = i == 0 ? qc[cb].x : i == 1 ? qc[cb].y : i == 2 ? qc[cb].z : qc[cb].w;
        bf[cb] = __builtin_bit_cast(half8_t, dequant_word(w, s2[cb], b2[cb]));
      }
#pragma unroll
      for (int mb = 0; mb < MB; mb++) {
        const half8_t af = *reinterpret_cast<const half8_t*>(
            &abuf[(mb * 32 + col) * kLdsRow + 32 * khalf + 8 * i]);
#pragma unroll
        for (int cb = 0; cb < 2; cb++)
          acc[mb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[cb], acc[mb][cb], 0, 0, 0);
      }
    }
    if (more) store_a((s + 1) & 1, av);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int cb = 0; cb < 2; cb++) {
        qc[cb] = qn[cb];
        scl[cb] = scn[cb];
        bia[cb] = bin[cb];
      }
    }
  }

  // ---- epilogue.  Accumulator register r of lane l holds row
  // 8*(r/4) + 4*(l/32) + r%4 and column l%32 of each 32x32 block.
#pragma unroll
  for (int mb = 0; mb < MB; mb++) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int row = mb * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
      if (row >= rows) continue;
      const size_t orow = (size_t)(row0 + row) * N;
      if (MODE == MOE_GEMM_GATE_UP_SWIGLU) {
        const int n = nb * 128 + wave * 32 + col;
        reinterpret_cast<half_t*>(p.out)[orow + n] = (half_t)silu_mul(acc[mb][0][r], acc[mb][1][r]);
      } else {
        const float w = row_w[row];
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
          const int n = nb * 256 + wave * 64 + cb * 32 + col;
          reinterpret_cast<float*>(p.out)[orow + n] = w * acc[mb][cb][r];
        }
      }
    }
  }
}

// x bf16 -> fp16, each 8-element chunk interleaved (0,4,1,5,2,6,3,7).
// bf16 values inside the fp16 range convert exactly.
__global__ __launch_bounds__(256) void stage_x_kernel(const uint4* __restrict__ in,
                                                      uint4* __restrict__ out, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 v = in[i];
  auto lo = [](uint32_t d) { return (half_t)__uint_as_float(d << 16); };
  auto hi = [](uint32_t d) { return (half_t)__uint_as_float(d & 0xFFFF0000u); };
  const half2_t o0 = {lo(v.x), lo(v.z)}, o1 = {hi(v.x), hi(v.z)};
  const half2_t o2 = {lo(v.y), lo(v.w)}, o3 = {hi(v.y), hi(v.w)};
  out[i] = make_uint4(__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1),
                      __builtin_bit_cast(uint32_t, o2), __builtin_bit_cast(uint32_t, o3));
}

// y[t][:] = sum_j y_sorted[pair_slot[t*k + j]][:], j ascending, fp32.
__global__ __launch_bounds__(256) void combine_kernel(const float4* __restrict__ y_sorted,
                                                      const int32_t* __restrict__ pair_slot,
                                                      float4* __restrict__ y, int T, int H4,
                                                      int k) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * H4) return;
  const int t = (int)(i / H4), c = (int)(i % H4);
  const int P = T * k;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; j++) {
    const int slot = pair_slot[(size_t)t * k + j];
    if (slot < 0 || slot >= P) continue;
    const float4 v = y_sorted[(size_t)slot * H4 + c];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  y[i] = acc;
}

template <int MODE>
hipError_t launch_mode(const GemmArgs& a, hipStream_t s) {
  const int64_t P = (int64_t)a.T * a.top_k;
  const int64_t max_blocks = P / a.block_m + (P < a.E ? P : a.E);
  MfmaParams p{a.a, a.b0, a.b1, a.sorted_pairs, a.topk_weights, a.blocks, a.num_blocks, a.out,
               a.N, a.K, a.G, a.top_k, a.E, (int)P, (int)max_blocks};
  const int wg_n = MODE == MOE_GEMM_GATE_UP_SWIGLU ? 128 : 256;
  const int64_t items = max_blocks * (a.N / wg_n);
  const int64_t grid = ((items + kNumXcd - 1) / kNumXcd) * kNumXcd;
  switch (a.block_m) {
    case 32: w4_mfma_kernel<MODE, 1><<<grid, 256, 0, s>>>(p); break;
    case 64: w4_mfma_kernel<MODE, 2><<<grid, 256, 0, s>>>(p); break;
    case 128: w4_mfma_kernel<MODE, 4><<<grid, 256, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4_mfma(const GemmArgs& a, hipStream_t s) {
  return a.mode == MOE_GEMM_GATE_UP_SWIGLU ? launch_mode<MOE_GEMM_GATE_UP_SWIGLU>(a, s)
                                           : launch_mode<MOE_GEMM_DOWN>(a, s);
}

hipError_t launch_stage_x(const uint16_t* x, half_t* xh, int64_t n_elems, hipStream_t s) {
  const int64_t n8 = n_elems / 8;
  stage_x_kernel<<<(n8 + 255) / 256, 256, 0, s>>>(reinterpret_cast<const uint4*>(x),
                                                  reinterpret_cast<uint4*>(xh), n8);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y_sorted, const int32_t* pair_slot, float* y, int T,
                          int H, int k, hipStream_t s) {
  const int64_t n = (int64_t)T * (H / 4);
  combine_kernel<<<(n + 255) / 256, 256, 0, s>>>(reinterpret_cast<const float4*>(y_sorted),
                                                 pair_slot, reinterpret_cast<float4*>(y), T, H / 4,
                                                 k);
  return hipGetLastError();
}

}  // namespace moe
