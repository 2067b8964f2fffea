// k_grouped_mm.hip -- grouped GEMM over packed fp4 expert weights with
// dequantization on the fly, for gfx950 (bf16 MFMA).
//
// Method: "nemo_automodel.components.quantization.mxfp4", MXFP4GroupedMM
// forward / backward, and "nemo_automodel.components.quantization.nvfp4",
// NVFP4GroupedMM forward / backward.  Activations are grouped by expert:
// expert e owns rows [offs[e-1], offs[e]) of x (offs[-1] = 0).  Its weights
// W_e [N, K] are stored packed along K; they are dequantized into the
// activation dtype exactly as dequantize_mxfp4 / dequantize_nvfp4 do, then
//   forward  (TRANS = 0): y[t, n] = sum_k x[t, k] * W_e[n, k]   (x [T, K], y [T, N])
//   backward (TRANS = 1): y[t, k] = sum_n x[t, n] * W_e[n, k]   (x [T, N], y [T, K])
// with float32 accumulation and one rounding of each output to bfloat16.
//
// Work: a workgroup (4 waves, 2 x 2) computes a BM x 128 output tile of one
// expert (BM = 128 token rows) with v_mfma_f32_32x32x16_bf16 (each wave
// BM/2 x 64 = BM/64 x 2 MFMA tiles), stepping the reduction by 64.
// Both operands are staged in LDS.  The activation tile is copied as is,
// [row][reduction] bf16 with 16-byte row padding.  The weight tile is
// dequantized in registers with the gfx950 fp4 converters on its way to LDS:
// for the forward product as [output column][reduction], for the backward as
// the weights' own [reduction][output column] rows, read transposed into the
// MFMA operand with ds_read_b64_tr_b16.
// The global loads of the next reduction step are issued before the MFMAs of
// the current one.  They are ordinary (temporal) loads: every activation
// tile is read by all output-column tiles of its token tile and every weight
// tile by all token tiles of its expert, and those reads meet in L2.  Workgroups map to (expert, token tile, output tile) in an
// XCD-aware order (see xcd_logical); the per-expert tile counts come from offs
// through a workgroup prefix sum, so
// the host never reads offs.
#include "mxq_kernel_common.h"
#include "mxq_launch_gemm.h"

namespace mxq {

namespace gmm {

constexpr int BN = 128;         // output columns per tile (token rows per tile: BM, 128 or 256)
constexpr int BK = 64;          // reduction step
constexpr int LDS_STRIDE = BK + 8;   // bf16 elements per LDS row (16-byte pad)
// Backward weight tile: BK reduction rows of BN output columns, row-major,
// with a 16-element pad (consecutive rows 8 banks apart).
constexpr int WT_STRIDE = BN + 16;
static_assert(BK * WT_STRIDE <= BN * LDS_STRIDE, "both weight-tile layouts share one LDS array");
constexpr int THREADS = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct Args {
  const uint16_t* x;          // [T, R] bf16 activations
  const uint8_t* packed;      // [E, N, K/2]
  const uint8_t* scales;      // [E, N, K/32] e8m0 or [E, N, K/16] e4m3
  const float* row_scale;     // [E, N] (NVFP4)
  const int32_t* offs;        // [E] cumulative token counts
  uint16_t* y;                // [T, C] bf16
  int64_t T, E, N, K;
};

// Dequantized bf16 of 8 consecutive weights (one packed dword) in the
// arithmetic of dequantize_mxfp4 / dequantize_nvfp4 with a bf16 output, up
// to the sign of zero: code 8 stays -0 here (the dequantizers give +0).  The
// accumulators start at +0 and +0 + -0 = +0, so no output changes (checked
// bit for bit against a build that canonicalises), and NVFP4 saves 4 of its
// 24 VALU operations per 8 weights.
template <int FMT>
__device__ __forceinline__ u32x4 deq8(uint32_t w, uint32_t sb, float g) {
  if constexpr (FMT == FMT_MXFP4) {
    u32x4 o = e2m1_unpack8_bf16_hw(w, e8m0_as_scale(sb));   // exact
    if (sb == 255u) o = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    return o;
  } else {
    const float sigma = e4m3_decode_any(sb);
    float f[8];
    e2m1_unpack8_f32_hw(w, 1.0f, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (f[i] * sigma) * g;   // exact, then RN
    return u32x4{bf16x2_rne(f[0], f[1]), bf16x2_rne(f[2], f[3]),
                 bf16x2_rne(f[4], f[5]), bf16x2_rne(f[6], f[7])};
  }
}

// Scale byte of weight (row n of expert e, column k).
template <int FMT>
__device__ __forceinline__ uint32_t scale_at(const Args& a, int64_t row, int64_t k) {
  constexpr int B = (FMT == FMT_MXFP4) ? 32 : 16;
  return a.scales[row * (a.K / B) + k / B];
}

// Registers holding one reduction step of both operands in flight.
template <int BM>
struct Stage {
  u32x4 av[BM / 32];          // BM / 32 x 8 activations
  u32x4 wv;                   // 32 packed codes of one weight row
  uint32_t sb[2];             // scale bytes of the two 16-column halves
  float g[1];                 // NVFP4 row scale
};

template <int FMT, int TRANS, int BM>
__device__ __forceinline__ void load_stage(const Args& a, Stage<BM>& st, int tid, int64_t e,
                                           int64_t m0, int64_t m1, int64_t c0, int64_t r0,
                                           int64_t R) {
  // activations: BM rows x 64 columns = 8 * BM chunks of 8, BM / 32 per thread
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    const int c = tid + THREADS * i;
    const int64_t row = m0 + (c >> 3);
    st.av[i] = row < m1 ? *reinterpret_cast<const u32x4*>(a.x + row * R + r0 + (c & 7) * 8)
                        : u32x4{0u, 0u, 0u, 0u};
  }
  if constexpr (TRANS == 0) {
    // W_e rows c0 .. c0+127, columns r0 .. r0+63: thread -> (row tid/2, half tid%2)
    const int64_t row = e * a.N + c0 + (tid >> 1);
    const int64_t k = r0 + (tid & 1) * 32;
    st.wv = *reinterpret_cast<const u32x4*>(a.packed + row * (a.K / 2) + k / 2);
    st.sb[0] = scale_at<FMT>(a, row, k);
    st.sb[1] = (FMT == FMT_MXFP4) ? st.sb[0] : scale_at<FMT>(a, row, k + 16);
    st.g[0] = (FMT == FMT_NVFP4) ? a.row_scale[row] : 1.0f;
  } else {
    // W_e rows r0 .. r0+63 (reduction), columns c0 .. c0+127: thread -> (row
    // tid/4, quarter tid%4 of 32 columns); 4 lanes read each row's 64 bytes
    const int64_t row = e * a.N + r0 + (tid >> 2);
    const int64_t k = c0 + (tid & 3) * 32;
    st.wv = *reinterpret_cast<const u32x4*>(a.packed + row * (a.K / 2) + k / 2);
    st.sb[0] = scale_at<FMT>(a, row, k);
    st.sb[1] = (FMT == FMT_MXFP4) ? st.sb[0] : scale_at<FMT>(a, row, k + 16);
    st.g[0] = (FMT == FMT_NVFP4) ? a.row_scale[row] : 1.0f;
  }
}

template <int FMT, int TRANS, int BM>
__device__ __forceinline__ void store_stage(const Stage<BM>& st, uint16_t* As, uint16_t* Bs, int tid) {
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    const int c = tid + THREADS * i;
    *reinterpret_cast<u32x4*>(As + (c >> 3) * LDS_STRIDE + (c & 7) * 8) = st.av[i];
  }
  const uint32_t w[4] = {st.wv.x, st.wv.y, st.wv.z, st.wv.w};
  if constexpr (TRANS == 0) {
    uint16_t* dst = Bs + (tid >> 1) * LDS_STRIDE + (tid & 1) * 32;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(dst + 8 * j) = deq8<FMT>(w[j], st.sb[j >> 1], st.g[0]);
  } else {
    // backward: weight row n (reduction), output columns kq .. kq+31 stay a
    // row of the tile; the MFMA operand is transposed on the way out of LDS
    const int n = tid >> 2, kq = (tid & 3) * 32;
    uint16_t* dst = Bs + n * WT_STRIDE + kq;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(dst + 8 * j) = deq8<FMT>(w[j], st.sb[j >> 1], st.g[0]);
  }
}

// Backward B operand of v_mfma_f32_32x32x16_bf16 from the row-major weight
// tile: lane l needs reduction rows kk + 8 (l / 32) + 0..7 of output column
// col0 + l % 32.  ds_read_b64_tr_b16 works on groups of 16 lanes: lane i of a
// group receives, for t = 0..3, the 16-bit element at offset i % 4 of the 8
// bytes that lane 4 t + i / 4 of the group addressed (checked on the chip).
// So lane j of a group addresses row nb + j / 4, columns kc + 4 (j % 4) ..,
// and lane i gets rows nb .. nb + 3 of column kc + i; two reads (nb, nb + 4)
// give the 8 rows.
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 read_b_trans(const uint16_t* Bs, int kk, int col0, int lane) {
  const int g = lane >> 4, jl = lane & 15;
  const int nb = kk + 8 * (g >> 1) + (jl >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (jl & 3);
  typedef __attribute__((address_space(3))) s16x4* LdsS16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS16x4)(Bs + nb * WT_STRIDE + col));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsS16x4)(Bs + (nb + 4) * WT_STRIDE + col));
  const s16x4 v[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v);
}

// Which expert and token tile this workgroup owns: tile counts per expert,
// an inclusive prefix sum over the workgroup, and a search.  Returns false
// when the slot is beyond the last tile.
template <int BM>
__device__ __forceinline__ bool find_tile(const Args& a, int64_t slot, int64_t& e_out,
                                          int64_t& m0, int64_t& m1) {
  __shared__ int64_t s_found[3];
  __shared__ int64_t s_wave[THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_found[0] = -1;
  __syncthreads();
  int64_t base = 0;
  for (int64_t e0 = 0; e0 < a.E; e0 += THREADS) {
    const int64_t e = e0 + tid;
    int64_t lo = 0, hi = 0, cnt = 0;
    if (e < a.E) {
      lo = e > 0 ? (int64_t)a.offs[e - 1] : 0;
      hi = (int64_t)a.offs[e];
      lo = lo < 0 ? 0 : (lo > a.T ? a.T : lo);
      hi = hi < lo ? lo : (hi > a.T ? a.T : hi);
      cnt = (hi - lo + BM - 1) / BM;
    }
    int64_t incl = cnt;            // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int64_t before = base;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    int64_t total = 0;
    for (int w = 0; w < THREADS / 64; ++w) total += s_wave[w];
    const int64_t first = before + incl - cnt;
    if (cnt > 0 && slot >= first && slot < first + cnt) {
      s_found[0] = e;
      s_found[1] = lo + (slot - first) * BM;
      s_found[2] = hi;
    }
    base += total;
    __syncthreads();
  }
  e_out = s_found[0];
  m0 = s_found[1];
  m1 = s_found[2];
  return e_out >= 0;
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  Logical tile L = xcd-major renumbering of the workgroup id, so that one
// XCD runs a contiguous range of logical tiles (a bijection for any count).
__device__ __forceinline__ int64_t xcd_logical(int64_t b, int64_t G) {
  constexpr int64_t X = 8;
  const int64_t xcd = b % X, pos = b / X, q = G / X, r = G % X;
  return xcd < r ? xcd * (q + 1) + pos : r * (q + 1) + (xcd - r) * q + pos;
}

// Waves per SIMD the register allocation must allow.  Left to itself the
// compiler takes 156 registers (3 waves); at 4 it fits 128 with a few spills
// outside the reduction loop, and the extra workgroup per CU keeps more
// global loads in flight (NVFP4 6-10% faster, MXFP4 forward 2-4%).
#ifndef MXQ_GMM_WAVES_PER_EU
#define MXQ_GMM_WAVES_PER_EU 4
#endif
#define MXQ_GMM_OCCUPANCY __attribute__((amdgpu_waves_per_eu(MXQ_GMM_WAVES_PER_EU, MXQ_GMM_WAVES_PER_EU)))

template <int FMT, int TRANS, int BM>
__global__ __launch_bounds__(THREADS) MXQ_GMM_OCCUPANCY void k_grouped_mm(Args a, int64_t ntiles_c) {
  constexpr int MT = BM / 64;               // 32 x 32 MFMA tiles per wave along the tokens
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t R = TRANS ? a.N : a.K;      // reduction length
  const int64_t C = TRANS ? a.K : a.N;      // output columns
  int64_t e, m0, m1;
  // logical tile -> (token slot, output tile), output tiles fastest: the
  // tiles that share an activation tile, and then those that share an
  // expert's weights, run next to each other on one XCD
  const int64_t L = xcd_logical(blockIdx.x, gridDim.x);
  const int64_t slot = L / ntiles_c;
  if (!find_tile<BM>(a, slot, e, m0, m1)) return;   // uniform over the workgroup
  const int64_t c0 = (L - slot * ntiles_c) * BN;
  const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * 64;   // wave tile origin

  f32x16 acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  Stage<BM> st;
  load_stage<FMT, TRANS, BM>(a, st, tid, e, m0, m1, c0, 0, R);
  for (int64_t r0 = 0; r0 < R; r0 += BK) {
    store_stage<FMT, TRANS, BM>(st, As, Bs, tid);
    __syncthreads();
    if (r0 + BK < R) load_stage<FMT, TRANS, BM>(a, st, tid, e, m0, m1, c0, r0 + BK, R);
    // backward: LLVM's MFMA-interleaving schedule (iglp strategy 1) measured
    // 2-4% faster for MXFP4; for the forward product it is 27% slower
    if constexpr (TRANS == 1) __builtin_amdgcn_iglp_opt(1);
    // MXFP4: waves in their MFMA phase take issue priority over those loading,
    // dequantizing and storing the next tile (2.5-4% faster both ways); NVFP4's
    // heavier dequantization needs the issue slots (3% slower backward)
    if constexpr (FMT == FMT_MXFP4) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[MT], bfr[2];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                    As + (wm + 32 * i + (lane & 31)) * LDS_STRIDE + kk + 8 * (lane >> 5)));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (TRANS == 0)
          bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                      Bs + (wn + 32 * j + (lane & 31)) * LDS_STRIDE + kk + 8 * (lane >> 5)));
        else
          bfr[j] = read_b_trans(Bs, kk, wn + 32 * j, lane);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if constexpr (FMT == FMT_MXFP4) __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  }

  // epilogue: accumulator register q of lane l is row 8*(q/4) + 4*(l/32) +
  // q%4, column l%32 of its 32 x 32 tile; one rounding to bf16 by the
  // hardware conversion: round to nearest even like the integer rounding of
  // f32_to_bf16_rne, in one instruction instead of five (NVFP4 up to 4%
  // faster, outputs bit-identical); a NaN stays a NaN, with the hardware's
  // payload
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm + 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        const int64_t col = c0 + wn + 32 * j + (lane & 31);
        if (row < m1) a.y[row * C + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][q]);
      }
}

}  // namespace gmm

hipError_t launch_grouped_mm(const void* x, int64_t T, const uint8_t* packed,
                             const uint8_t* scales, const float* row_scale,
                             int64_t E, int64_t N, int64_t K, const int32_t* offs,
                             int fmt, int trans, void* y, hipStream_t s) {
  gmm::Args a;
  a.x = static_cast<const uint16_t*>(x);
  a.packed = packed;
  a.scales = scales;
  a.row_scale = row_scale;
  a.offs = offs;
  a.y = static_cast<uint16_t*>(y);
  a.T = T; a.E = E; a.N = N; a.K = K;
  const int64_t C = trans ? K : N;
  // token-tile slots: at most ceil(T / bm) + E over all experts (slots past
  // the last tile exit at once), times the output tiles
  // 128-row token tiles (256-row tiles need 280 registers per lane, one wave
  // per SIMD, and measured slower)
  constexpr int bm = 128;
  const int64_t slots = (T + bm - 1) / bm + E;
  const int64_t ntc = C / gmm::BN;
  const dim3 grid((unsigned)(slots * ntc)), block(gmm::THREADS);
#define MXQ_GMM_LAUNCH(F, TR) hipLaunchKernelGGL((gmm::k_grouped_mm<F, TR, bm>), grid, block, 0, s, a, ntc)
  if (fmt == FMT_MXFP4) {
    if (trans) MXQ_GMM_LAUNCH(FMT_MXFP4, 1); else MXQ_GMM_LAUNCH(FMT_MXFP4, 0);
  } else {
    if (trans) MXQ_GMM_LAUNCH(FMT_NVFP4, 1); else MXQ_GMM_LAUNCH(FMT_NVFP4, 0);
  }
#undef MXQ_GMM_LAUNCH
  return hipGetLastError();
}

}  // namespace mxq
