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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
    const float sigma = e4m3_decode_hw(sb);
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

// Registers holding one reduction step of a thread's share of the weight tile.
struct WStage {
  u32x4 wv;                   // 32 packed codes of one weight row
  uint32_t sb;                // MXFP4: the scale byte; NVFP4: the scale bytes
                              // of the two 16-column halves, low byte first
  float g;                    // NVFP4 row scale
};

template <int FMT, int TRANS>
__device__ __forceinline__ void load_w(const Args& a, WStage& w, int tid, int64_t e, int64_t c0,
                                       int64_t r0) {
  int64_t row, k;
  if constexpr (TRANS == 0) {
    // W_e rows c0 .. c0+127, columns r0 .. r0+63: thread -> (row tid/2, half tid%2)
    row = e * a.N + c0 + (tid >> 1);
    k = r0 + (tid & 1) * 32;
  } else {
    // W_e rows r0 .. r0+63 (reduction), columns c0 .. c0+127: thread -> (row
    // tid/4, quarter tid%4 of 32 columns); 4 lanes read each row's 64 bytes
    row = e * a.N + r0 + (tid >> 2);
    k = c0 + (tid & 3) * 32;
  }
  w.wv = *reinterpret_cast<const u32x4*>(a.packed + row * (a.K / 2) + k / 2);
  if constexpr (FMT == FMT_MXFP4) {
    w.sb = scale_at<FMT>(a, row, k);
  } else {
    // the two scale bytes are adjacent (k is a multiple of 32): one 16-bit
    // load, so that no arithmetic joins two loads right after they issue
    uint16_t pair;
    __builtin_memcpy(&pair, a.scales + row * (a.K / 16) + k / 16, 2);
    w.sb = pair;
  }
  w.g = (FMT == FMT_NVFP4) ? a.row_scale[row] : 1.0f;
}

template <int FMT, int TRANS>
__device__ __forceinline__ void store_w(const WStage& w, uint16_t* Bs, int tid) {
  const uint32_t v[4] = {w.wv.x, w.wv.y, w.wv.z, w.wv.w};
  // forward: [output column][reduction] rows of the tile; backward: weight
  // row n (reduction), output columns kq .. kq+31 stay a row of the tile and
  // the MFMA operand is transposed on the way out of LDS
  uint16_t* dst = TRANS == 0 ? Bs + (tid >> 1) * LDS_STRIDE + (tid & 1) * 32
                             : Bs + (tid >> 2) * WT_STRIDE + (tid & 3) * 32;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<u32x4*>(dst + 8 * j) =
        deq8<FMT>(v[j], FMT == FMT_MXFP4 ? w.sb : (w.sb >> (8 * (j >> 1))) & 0xFFu, w.g);
}

// Registers holding one reduction step of both operands in flight.
template <int BM>
struct Stage {
  u32x4 av[BM / 32];          // BM / 32 x 8 activations
  WStage w;
};

// Activations from row m0 on through a buffer resource (BUF): one 32-bit
// offset per thread instead of a 64-bit pointer per load, for tiles whose
// byte offsets fit in 31 bits (BM * R * 2 < 2^31, checked by the launcher).
// Rows past the end of the tensor read zeros (the hardware's range check);
// rows of later groups are read as they are.  Either kind feeds only
// accumulator rows that are never stored.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t act_rsrc(const Args& a, int64_t m0, int64_t R) {
  const int64_t left = (a.T - m0) * R * 2;             // bytes from row m0 to the end
  const int nrec = left > 0x7FFFFFFF ? 0x7FFFFFFF : (int)left;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x + m0 * R), 0, nrec,
                                           0x00020000);
}

template <int FMT, int TRANS, int BM, bool BUF>
__device__ __forceinline__ void load_stage(const Args& a, Stage<BM>& st, int tid, int64_t e,
                                           int64_t m0, int64_t m1, int64_t c0, int64_t r0,
                                           int64_t R) {
  // activations: BM rows x 64 columns = 8 * BM chunks of 8, BM / 32 per thread.
  if constexpr (BUF) {
    const __amdgpu_buffer_rsrc_t rs = act_rsrc(a, m0, R);
    const int vbase = (int)(((tid >> 3) * R + (tid & 7) * 8) * 2);
#pragma unroll
    for (int i = 0; i < BM / 32; ++i)
      st.av[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rs, vbase + (int)((32 * i * R + r0) * 2), 0, 0));
  } else {
    // Rows past the end of the group read the group's last row instead (in
    // bounds, and no branch around each load): they feed only accumulator
    // rows that are never stored.
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      const int c = tid + THREADS * i;
      int64_t row = m0 + (c >> 3);
      row = row < m1 ? row : m1 - 1;
      st.av[i] = *reinterpret_cast<const u32x4*>(a.x + row * R + r0 + (c & 7) * 8);
    }
  }
  load_w<FMT, TRANS>(a, st.w, tid, e, c0, r0);
}

template <int FMT, int TRANS, int BM>
__device__ __forceinline__ void store_stage(const Stage<BM>& st, uint16_t* As, uint16_t* Bs, int tid) {
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    const int c = tid + THREADS * i;
    *reinterpret_cast<u32x4*>(As + (c >> 3) * LDS_STRIDE + (c & 7) * 8) = st.av[i];
  }
  store_w<FMT, TRANS>(st.w, Bs, tid);
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

// Token tiles of all experts together (uniform over the workgroup): the sum
// of ceil(group / BM) over the groups offs describes, clamped as find_tile
// clamps them.
template <int BM>
__device__ __forceinline__ int64_t total_tiles(const Args& a) {
  __shared__ int64_t s_part[THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t sum = 0;
  for (int64_t e = tid; e < a.E; e += THREADS) {
    int64_t lo = e > 0 ? (int64_t)a.offs[e - 1] : 0;
    int64_t hi = (int64_t)a.offs[e];
    lo = lo < 0 ? 0 : (lo > a.T ? a.T : lo);
    hi = hi < lo ? lo : (hi > a.T ? a.T : hi);
    sum += (hi - lo + BM - 1) / BM;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d);
  if (lane == 0) s_part[wave] = sum;
  __syncthreads();
  int64_t tot = 0;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) tot += s_part[w];
  return tot;
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  The grid is sized for the most token tiles the groups could need (the
// host never reads offs), ceil(T / BM) + E per output tile; the G tiles that
// exist are split evenly over the XCDs, each XCD taking a contiguous range of
// logical tiles, and the surplus workgroups of every XCD exit.  (Numbering
// all grid slots instead put every surplus slot on the last XCDs: a third of
// the chip idle for 256 tokens per expert.)  Returns -1 for a surplus
// workgroup.
__device__ __forceinline__ int64_t xcd_logical(int64_t b, int64_t G) {
  constexpr int64_t X = 8;
  const int64_t xcd = b % X, pos = b / X, q = G / X, r = G % X;
  const int64_t cnt = q + (xcd < r ? 1 : 0);
  if (pos >= cnt) return -1;
  return xcd * q + (xcd < r ? xcd : r) + pos;
}

// Waves per SIMD the register allocation must allow.  128-row tiles: left to
// itself the compiler takes 156 registers (3 waves); at 4 it fits 128 with a
// few spills outside the reduction loop, and the extra workgroup per CU keeps
// more global loads in flight (NVFP4 6-10% faster, MXFP4 forward 2-4%).
// 256-row tiles: 236-248 registers without spills at 2 waves (at 3 or 4 the
// accumulators move to AGPRs and the kernel runs one wave per SIMD).
#ifndef MXQ_GMM_WAVES_PER_EU
#define MXQ_GMM_WAVES_PER_EU 4
#endif
#ifndef MXQ_GMM_WAVES_PER_EU_256
#define MXQ_GMM_WAVES_PER_EU_256 2
#endif

template <int BM>
constexpr int gmm_waves_per_eu() { return BM == 256 ? MXQ_GMM_WAVES_PER_EU_256 : MXQ_GMM_WAVES_PER_EU; }

template <int FMT, int TRANS, int BM, bool BUF>
__global__ __launch_bounds__(THREADS)
__attribute__((amdgpu_waves_per_eu(gmm_waves_per_eu<BM>(), gmm_waves_per_eu<BM>())))
void k_grouped_mm(Args a, int64_t ntiles_c) {
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
  const int64_t L = xcd_logical(blockIdx.x, total_tiles<BM>(a) * ntiles_c);
  if (L < 0) return;                        // uniform over the workgroup
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
  load_stage<FMT, TRANS, BM, BUF>(a, st, tid, e, m0, m1, c0, 0, R);
  for (int64_t r0 = 0; r0 < R; r0 += BK) {
    store_stage<FMT, TRANS, BM>(st, As, Bs, tid);
    __syncthreads();
    if (r0 + BK < R) load_stage<FMT, TRANS, BM, BUF>(a, st, tid, e, m0, m1, c0, r0 + BK, R);
    // backward, 128-row tiles: LLVM's MFMA-interleaving schedule (iglp
    // strategy 1) measured 2-4% faster for MXFP4; for the forward product it
    // is 27% slower.  With 256-row tiles the backward runs 1-3% faster without
    // it (MXFP4 291 against 300 us on the expert shapes).
#ifndef MXQ_GMM_IGLP_256
#define MXQ_GMM_IGLP_256 0
#endif
#ifndef MXQ_GMM_PRIO_256
#define MXQ_GMM_PRIO_256 1
#endif
    if constexpr (TRANS == 1 && (BM == 128 || MXQ_GMM_IGLP_256)) __builtin_amdgcn_iglp_opt(1);
    // 256-row tiles: the small-GEMM interleaving of LDS reads with MFMAs (iglp
    // strategy 0) measured 2-2.5% faster for NVFP4 both ways (forward 536 ->
    // 526 us, backward 551 -> 538 us on the expert shapes) and for the MXFP4
    // forward (296 -> 289 us); the MXFP4 backward moved within run-to-run
    // noise (+-2%), so it keeps the compiler's own schedule.  With the
    // branch-free NVFP4 decode, no hint or strategy 1 was 4-7% slower.
    else if constexpr (BM == 256 && !MXQ_GMM_IGLP_256 && (FMT != FMT_MXFP4 || TRANS == 0))
      __builtin_amdgcn_iglp_opt(0);
    // MXFP4: waves in their MFMA phase take issue priority over those loading,
    // dequantizing and storing the next tile (2.5-4% faster both ways); NVFP4's
    // heavier dequantization needs the issue slots (3% slower both ways)
    if constexpr (FMT == FMT_MXFP4 && (BM == 128 || MXQ_GMM_PRIO_256)) __builtin_amdgcn_s_setprio(1);
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
          // weights as the A operand, activations as B: the accumulators
          // hold the tile transposed (see the epilogue)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if constexpr (FMT == FMT_MXFP4 && (BM == 128 || MXQ_GMM_PRIO_256)) __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  }

  // epilogue.  With the weights as the MFMA's A operand, accumulator register
  // q of lane l holds token row l % 32 of its 32 x 32 tile and output column
  // 8 (q / 4) + 4 (l / 32) + q % 4: registers 4g .. 4g+3 are four consecutive
  // columns of one row.  (The products are the same as with the operands the
  // other way round, and so were the outputs, bit for bit, on the MoE expert
  // shapes in both directions.)  One rounding to bf16 by the hardware pair
  // conversion, round to nearest even like the integer rounding of
  // f32_to_bf16_rne; a NaN stays a NaN, with the hardware's payload.  Each
  // 32-row band of the wave's tile goes through the wave's own LDS region
  // (the operand tiles are free after the last barrier; LDS accesses of one
  // wave run in order, so no barrier is needed between the bands), written
  // as 8-byte pieces and read back as 16-byte row chunks: 16-byte global
  // stores, 2-3% faster than one 2-byte store per output (bit-identical).
  {
    constexpr int EP = 64 + 8;                 // bf16 per LDS row of a band
    static_assert(4 * 32 * EP <= BM * LDS_STRIDE, "four waves' bands fit in As");
    uint16_t* band = As + wave * (32 * EP);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int col = 32 * j + 8 * gq + 4 * (lane >> 5);
          const u32x2 v = {bf16x2_rne(acc[i][j][4 * gq], acc[i][j][4 * gq + 1]),
                           bf16x2_rne(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3])};
          *reinterpret_cast<u32x2*>(band + (lane & 31) * EP + col) = v;
        }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ch = lane + 64 * t;          // 32 rows x 8 chunks of 8 columns
        const int r = ch >> 3, cc = (ch & 7) * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(band + r * EP + cc);
        const int64_t row = m0 + wm + 32 * i + r;
        if (row < m1) *reinterpret_cast<u32x4*>(a.y + row * C + c0 + wn + cc) = v;
      }
    }
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
  // Token-tile height: 256 rows when the experts average 256 tokens or more
  // (each weight tile is dequantized once per 256 rows and every activation
  // tile is read by half as many workgroups: on the MoE expert shapes with
  // 256 and 512 tokens per expert 6-8% faster than 128-row tiles, except the
  // NVFP4 backward, within 2%), else 128 rows (a 256-row tile of a small group
  // would spend its MFMAs on rows that are not there).  The grid holds the
  // most token tiles the groups could need, ceil(T / bm) + E per output tile
  // (slots past the last tile exit at once).
#ifndef MXQ_GMM_BM
#define MXQ_GMM_BM 0
#endif
  const bool tall = MXQ_GMM_BM == 256 || (MXQ_GMM_BM == 0 && T >= 256 * E);
  const int64_t bm = tall ? 256 : 128;
  const int64_t slots = (T + bm - 1) / bm + E;
  const int64_t ntc = C / gmm::BN;
  const dim3 grid((unsigned)(slots * ntc)), block(gmm::THREADS);
#define MXQ_GMM_LAUNCH(F, TR, BUF)                                                               \
  do {                                                                                          \
    if (tall) hipLaunchKernelGGL((gmm::k_grouped_mm<F, TR, 256, BUF>), grid, block, 0, s, a, ntc); \
    else hipLaunchKernelGGL((gmm::k_grouped_mm<F, TR, 128, BUF>), grid, block, 0, s, a, ntc);      \
  } while (0)
  // Activation loads through a buffer resource: MXFP4 forward 281 -> 270 us
  // and backward 274 -> 258 us on the expert shapes (outputs bit-identical,
  // ragged groups included); NVFP4 forward 3% slower, backward unchanged, so
  // NVFP4 keeps 64-bit pointers, and so does a reduction too long for 31-bit
  // byte offsets within a 256-row tile.
  const int64_t R = trans ? N : K;
  const bool buf = R * 2 * 256 < (int64_t(1) << 31);
  if (fmt == FMT_MXFP4) {
    if (buf) {
      if (trans) MXQ_GMM_LAUNCH(FMT_MXFP4, 1, true); else MXQ_GMM_LAUNCH(FMT_MXFP4, 0, true);
    } else {
      if (trans) MXQ_GMM_LAUNCH(FMT_MXFP4, 1, false); else MXQ_GMM_LAUNCH(FMT_MXFP4, 0, false);
    }
  } else {
    if (trans) MXQ_GMM_LAUNCH(FMT_NVFP4, 1, false); else MXQ_GMM_LAUNCH(FMT_NVFP4, 0, false);
  }
#undef MXQ_GMM_LAUNCH
  return hipGetLastError();
}

}  // namespace mxq
