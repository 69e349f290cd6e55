// Dual-path MXFP4 GEMM of the SharQ path, for gfx950.
//
// "SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
// Inference" (arXiv:2606.26587), abstract, sentence 4 (a sparse FP4 GEMM on
// the backbone and a dense FP4 GEMM on the residual) and sentence 5 (both
// read one FP4 weight payload through path-specific scale views):
//
//   Y = deq(backbone) W^T + deq(residual) W^T,   fp32 accumulate, fp32 out.
//
// Both paths run on the CDNA4 block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 (E2M1) A and B operands and one
// E8M0 scale per 32 k per row and per column.  gfx950 has no structured-sparse
// MFMA for FP4 operands, so the 2:4 backbone is expanded to dense FP4 (zeros
// at the dropped positions) while it is staged into LDS (or, in the
// dense-expanded variant, read in the dense layout the preparation wrote).
// Each K step stages the W tile once and feeds it to the MFMAs of both paths,
// which accumulate into the same registers.
//
// Kernels: dual_gemm_dense_kernel (prefill, backbone in the dense layout the
// preparation wrote; its GROUPED form runs a mixture-of-experts layer's
// expert GEMMs over gathered activation rows), dual_gemm_decomp_kernel
// (prefill, the 2:4 backbone expanded in LDS), dual_gemm_decode_kernel and
// dual_gemm_skinny_kernel (m <= 32, bound by streaming W).  The prefill kernels stage 128-k steps of every
// operand in LDS with direct global -> LDS loads; LDS rows are 64 bytes (four
// 16-byte chunks) and chunk c of row r sits at c ^ ((r >> 2) & 3), so sixteen
// lanes reading one chunk of sixteen consecutive rows hit sixteen different
// bank groups.
//
// Operand layout of the 32x32x64 FP4 MFMA (lane l, h = l / 32): A row l % 32
// and B column l % 32, 32 consecutive k (16 bytes) per lane; the lane's scale
// register holds the E8M0 byte of those k.  Within a 128-k step lane half h
// takes the k blocks 2h (first MFMA) and 2h + 1 (second MFMA); A and B use the
// same assignment, so the dot products are unchanged.  The row's scale word
// is shifted right by 16h once and op_sel picks byte 0 or 1.
// Accumulator: lane l holds column l % 32, rows 8 (r / 4) + 4 h + r % 4.
#include <stddef.h>

#include <type_traits>

#include "fp4_device.h"
#include "gemm_common.h"
#include "kernels.h"
#include "prep_block.h"

namespace sharq {
namespace {

using namespace gemm;

// ---------------------------------------------------------------------------
// Dense-operand pipeline: the backbone is read in its dense layout, so all
// three operand tiles and the four scale arrays go global -> LDS with
// buffer_load ... lds (lane l's bytes land at M0 + l * size; loads past the
// end of an operand read 0), STAGES - 1 K steps ahead of the MFMAs, into a
// ring of STAGES LDS stages.  A workgroup of NW wavefronts owns a TBM x TBN
// tile; small tiles let two workgroups share a CU, so that one workgroup's
// MFMAs run while the other waits at its barrier.  Before a step each
// wavefront waits until at most the later stages' loads are in flight, then
// a barrier makes all wavefronts' loads visible and frees the stage read on
// the previous step.

template <int TBM, int TBN>
struct DStage {
  u32x4 as[TBM * 4];
  u32x4 ar[TBM * 4];
  u32x4 w[TBN * 4];
  uint32_t sas[TBM], sar[TBM], sws[TBN], swd[TBN];
};

// Load plan of one stage: 16-byte chunk loads of 16 rows each (A backbone,
// A residual, W), then 4-byte scale loads of 64 rows each (backbone, residual,
// W sparse view, W dense view); wavefront w takes loads w, w + NW, ...
template <int TBM, int TBN, int NW>
struct DPlan {
  static constexpr int kA = TBM / 16, kW = TBN / 16;
  static constexpr int kS = 2 * (TBM / 64) + 2 * (TBN / 64);
  static constexpr int kChunkPer = (2 * kA + kW + NW - 1) / NW;
  static constexpr int kScalePer = (kS + NW - 1) / NW;
  static constexpr int kMinPerWave = (2 * kA + kW) / NW + kS / NW;   // waitcnt allowance per stage
};

struct DRsrc {
  OpStream as, ar, w, sas, sar, sws, swd;
};

template <int TBM, int TBN, int NW>
struct DOffs {
  uint32_t chunk[DPlan<TBM, TBN, NW>::kChunkPer];
  uint32_t scale[DPlan<TBM, TBN, NW>::kScalePer];
};

// Tile rows of the A operands: plain tiles stream rows m0 .. of A (offsets
// relative to row m0; rows past the last one lie past the descriptor's range
// and read 0); a grouped tile gathers activation row row_index[i] for its
// grouped rows i = m0 .. (offsets relative to row 0).  Its rows past the
// group's end (their outputs are not stored) are kPast when zero_past, which
// the load plan turns into an offset past the operand, so that they read 0:
// zero operands cost the MFMAs less energy than a repeated row, and the
// grouped GEMMs run at the board's power limit (gate+up 1.2-2.5% faster).
// Otherwise they repeat the group's last row: the SiLU epilogue would send a
// zero gate down its binary64 path, so the gate+up kernel with that epilogue
// keeps real rows there.
struct ARows {
  static constexpr uint32_t kPast = 0xFFFFFFFFu;
  const int32_t *idx;   // grouped: the gather (null: grouped row i is activation row i)
  int64_t m0, m_end;
  bool grouped, zero_past;
  __device__ __forceinline__ uint32_t operator()(int r) const {
    if (!grouped) return (uint32_t)r;
    int64_t i = m0 + r;
    if (i >= m_end) {
      if (zero_past) return kPast;
      i = m_end - 1;
    }
    return (uint32_t)(idx ? (int64_t)idx[i] : i);
  }
};

// Byte offset of row `row` (+ `add`) in stream `s`; kPast rows go to the
// first offset past the descriptor's range (raw buffer loads there return 0).
__device__ __forceinline__ uint32_t row_offset(const OpStream &s, uint32_t row, uint32_t add) {
  return row == ARows::kPast ? s.size + add : row * s.row_stride + add;
}

// Tile rows of W: plain tiles stream rows n0 .. of W (offsets relative to
// row n0); a gate+up tile (SPLIT) reads the gate rows j0 .. j0 + hb - 1 as its
// first hb rows and the up rows half + j0 .. as its last hb (offsets relative
// to row 0), so that one tile holds the gate and up columns of the same j.
template <bool SPLIT>
struct WRows {
  int64_t j0, half;
  int hb;
  __device__ __forceinline__ uint32_t operator()(int r) const {
    if (!SPLIT) return (uint32_t)r;
    return (uint32_t)(r < hb ? j0 + r : half + j0 + (r - hb));
  }
};

template <int TBM, int TBN, int NW, bool SPLIT = false>
__device__ __forceinline__ void plan_loads(const GemmArgs &a, int64_t m0, int64_t n0, int wave,
                                           int lane, DRsrc &R, DOffs<TBM, TBN, NW> &O,
                                           const ARows &arow, int64_t w_row0, int64_t w_rows,
                                           const WRows<SPLIT> &wrow = WRows<SPLIT>{0, 0, 0}) {
  using P = DPlan<TBM, TBN, NW>;
  const int lrow = lane >> 2, lchunk = (lane & 3) ^ ((lane >> 4) & 3);
  const int64_t steps = a.k / BK;
  const int64_t a_rows = arow.grouped ? a.tokens : a.m, a_r0 = arow.grouped ? 0 : m0;
  R.as = op_stream(a.s_dense, a.ld_sd, a.s_ksm, a_rows, a_r0, steps, 64);
  R.ar = op_stream(a.r_codes, a.ld_rc, a.r_ksm, a_rows, a_r0, steps, 64);
  R.w = op_stream(a.w_codes, a.ld_wc, a.w_ksm, w_rows, w_row0 + n0, steps, 64);
  R.sas = op_stream(a.s_scales, a.ld_ss, a.s_ksm, a_rows, a_r0, steps, 4);
  R.sar = op_stream(a.r_scales, a.ld_rs, a.r_ksm, a_rows, a_r0, steps, 4);
  R.sws = op_stream(a.ws_scales, a.ld_wss, a.w_ksm, w_rows, w_row0 + n0, steps, 4);
  R.swd = op_stream(a.wd_scales, a.ld_wds, a.w_ksm, w_rows, w_row0 + n0, steps, 4);
#pragma unroll
  for (int j = 0; j < P::kChunkPer; ++j) {
    int q = wave + NW * j;
    if (q < 2 * P::kA) {
      const bool res = q >= P::kA;
      if (res) q -= P::kA;
      O.chunk[j] = row_offset(res ? R.ar : R.as, arow(16 * q + lrow), lchunk * 16);
    } else {
      q -= 2 * P::kA;
      O.chunk[j] = wrow(16 * q + lrow) * R.w.row_stride + lchunk * 16;
    }
  }
#pragma unroll
  for (int j = 0; j < P::kScalePer; ++j) {
    int t = wave + NW * j;
    if (t < 2 * (TBM / 64)) {
      const bool res = t >= TBM / 64;
      if (res) t -= TBM / 64;
      O.scale[j] = row_offset(res ? R.sar : R.sas, arow(64 * t + lane), 0);
    } else {
      t -= 2 * (TBM / 64);
      uint32_t rs = R.sws.row_stride;
      if (t >= TBN / 64) { t -= TBN / 64; rs = R.swd.row_stride; }
      O.scale[j] = wrow(64 * t + lane) * rs;
    }
  }
}

template <int TBM, int TBN, int NW>
__device__ __forceinline__ void issue_stage(const DRsrc &R, const DOffs<TBM, TBN, NW> &O, int wave,
                                            int kt, const DStage<TBM, TBN> &S) {
  using P = DPlan<TBM, TBN, NW>;
  using St = DStage<TBM, TBN>;
  const uint32_t base = lds_addr(&S);
  const uint32_t t = (uint32_t)kt;
  constexpr uint32_t oar = offsetof(St, ar), ow = offsetof(St, w);
  constexpr uint32_t osas = offsetof(St, sas), osar = offsetof(St, sar);
  constexpr uint32_t osws = offsetof(St, sws), oswd = offsetof(St, swd);
#pragma unroll
  for (int j = 0; j < P::kChunkPer; ++j) {
    const int q = wave + NW * j;
    // loads NW j .. NW j + NW - 1 go to one operand when the operand
    // boundaries are multiples of NW: resolved at compile time
    const int q0 = NW * j;
    if (q0 + NW <= P::kA) b2l16(R.as.rsrc, O.chunk[j], t * R.as.step, base + q * 1024);
    else if (q0 >= P::kA && q0 + NW <= 2 * P::kA)
      b2l16(R.ar.rsrc, O.chunk[j], t * R.ar.step, base + oar + (q - P::kA) * 1024);
    else if (q0 >= 2 * P::kA && q0 + NW <= 2 * P::kA + P::kW)
      b2l16(R.w.rsrc, O.chunk[j], t * R.w.step, base + ow + (q - 2 * P::kA) * 1024);
    else if (q < P::kA) b2l16(R.as.rsrc, O.chunk[j], t * R.as.step, base + q * 1024);
    else if (q < 2 * P::kA) b2l16(R.ar.rsrc, O.chunk[j], t * R.ar.step, base + oar + (q - P::kA) * 1024);
    else if (q < 2 * P::kA + P::kW)
      b2l16(R.w.rsrc, O.chunk[j], t * R.w.step, base + ow + (q - 2 * P::kA) * 1024);
  }
#pragma unroll
  for (int j = 0; j < P::kScalePer; ++j) {
    int q = wave + NW * j;
    if (q >= P::kS) continue;
    if (q < TBM / 64) b2l4(R.sas.rsrc, O.scale[j], t * R.sas.step, base + osas + 256 * q);
    else if ((q -= TBM / 64) < TBM / 64) b2l4(R.sar.rsrc, O.scale[j], t * R.sar.step, base + osar + 256 * q);
    else if ((q -= TBM / 64) < TBN / 64) b2l4(R.sws.rsrc, O.scale[j], t * R.sws.step, base + osws + 256 * q);
    else b2l4(R.swd.rsrc, O.scale[j], t * R.swd.step, base + oswd + 256 * (q - TBN / 64));
  }
}

// One 128-k step of wavefront (wm, wn): 64 rows x TBN/2 columns.
// Side work of a step that runs under its MFMAs: pre() issues its LDS reads
// with the step's, post() its arithmetic and LDS writes, interleaved with the
// MFMAs.
struct NoSide {
  static constexpr int kValuPerMfma = 0;
  __device__ __forceinline__ void pre() {}
  __device__ __forceinline__ void post() {}
};

template <int TBM, int TBN, int NIT = 2, class Stage, class Side = NoSide>
__device__ __forceinline__ void compute_stage(const Stage &S, v16f (&acc)[2][TBN / 64],
                                              int wm, int wn, int h, int li, Side side = Side()) {
  // NIT: the wavefront's 32-row tiles that take part (1: rows 64 wm + 32 ..
  // lie past a grouped tile's group; the other tile keeps its zeros)
  constexpr int TN = TBN / 64;
  static_assert(NIT == 1 || NIT == 2, "one or both 32-row tiles");
  // the step's LDS reads are issued at raised wavefront priority, so that they
  // go out ahead of the MFMAs another wavefront of the SIMD is issuing
  __builtin_amdgcn_s_setprio(1);
  int sas[2], sar[2], sws[TN], swd[TN];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = wm * 64 + it * 32 + li;
    sas[it] = (int)(S.sas[r] >> (16 * h));
    sar[it] = (int)(S.sar[r] >> (16 * h));
  }
#pragma unroll
  for (int jt = 0; jt < TN; ++jt) {
    const int r = wn * (TBN / 2) + jt * 32 + li;
    sws[jt] = (int)(S.sws[r] >> (16 * h));
    swd[jt] = (int)(S.swd[r] >> (16 * h));
  }
  u32x4 ras[2][2], rar[2][2], rb[2][TN];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int c = 2 * h + s;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = wm * 64 + it * 32 + li;
      ras[s][it] = S.as[lds_slot(r, c)];
      rar[s][it] = S.ar[lds_slot(r, c)];
    }
#pragma unroll
    for (int jt = 0; jt < TN; ++jt) {
      const int r = wn * (TBN / 2) + jt * 32 + li;
      rb[s][jt] = S.w[lds_slot(r, c)];
    }
  }
  side.pre();
  // every LDS read of the step is issued before the first MFMA (left to
  // itself the compiler reuses one register set and waits on each A
  // fragment just before its MFMAs)
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    v8i fas[2], far[2], fb[TN];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      fas[it] = as_operand(ras[s][it]);
      far[it] = as_operand(rar[s][it]);
    }
#pragma unroll
    for (int jt = 0; jt < TN; ++jt) fb[jt] = as_operand(rb[s][jt]);
    // backbone MFMAs for every tile first, then the residual ones: 2 TN
    // independent accumulators between two updates of the same tile
#pragma unroll
    for (int path = 0; path < 2; ++path)
#pragma unroll
      for (int it = 0; it < NIT; ++it)
#pragma unroll
        for (int jt = 0; jt < TN; ++jt) {
          const v8i fa = path == 0 ? fas[it] : far[it];
          const int sa = path == 0 ? sas[it] : sar[it];
          const int sw = path == 0 ? sws[jt] : swd[jt];
          if (s == 0)
            acc[it][jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb[jt], acc[it][jt], 4, 4, 0, sa, 0, sw);
          else
            acc[it][jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb[jt], acc[it][jt], 4, 4, 1, sa, 1, sw);
        }
  }
  if (Side::kValuPerMfma > 0) {
    static_assert(Side::kValuPerMfma == 0 || NIT == 2, "the side work's schedule assumes both tiles");
    side.post();
    // one MFMA, then kValuPerMfma VALU instructions of the side work, ...
#pragma unroll
    for (int i = 0; i < 4 * TN * 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, Side::kValuPerMfma, 0);
    }
  }
}

// Grouped tiles: the grid holds ceil(m / TBM) + groups tile rows times the
// tile columns, an upper bound of the tiles the groups need, so that the group
// sizes can stay on the device.  The workgroup counts each group's tile rows
// (group offsets clamped to [0, m], so that no tile writes outside Y whatever
// the offsets hold), scans them in LDS, and numbers the real tiles group by
// group (tile row, then tile column).  Workgroups go to the 8 XCDs round
// robin (XCD = id % 8); XCD x takes the x-th eighth of the real tiles, so that
// every XCD gets the same share of the work and a group's tiles, which share
// its weight and its gathered rows, stay in one L2.  Workgroups past their
// XCD's share have no work.
template <int TBM>
__device__ __forceinline__ bool grouped_tile(const GemmArgs &a, uint32_t id, uint32_t gn, int64_t &m0,
                                             int64_t &m_end, int64_t &group, uint32_t &tn) {
  __shared__ int32_t cnt[256];
  __shared__ int64_t found[3];
  const int t = threadIdx.x;
  int64_t lo = 0, hi = 0;
  if (t < a.groups) {
    lo = min(max(a.group_off[t], (int64_t)0), a.m);
    hi = min(max(a.group_off[t + 1], lo), a.m);
  }
  const int32_t c = (int32_t)((hi - lo + TBM - 1) / TBM);
  cnt[t] = c;
  if (t == 0) found[0] = -1;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {   // inclusive scan
    const int32_t v = cnt[t] + (t >= d ? cnt[t - d] : 0);
    __syncthreads();
    cnt[t] = v;
    __syncthreads();
  }
  const uint32_t real = (uint32_t)cnt[255] * gn, per = (real + 7) / 8;
  const uint32_t local = id / 8, tile = (id % 8) * per + local;
  const int32_t end = cnt[t], begin = end - c;
  const int32_t tm = (int32_t)(tile / gn);
  if (local < per && tile < real && c > 0 && tm >= begin && tm < end) {
    found[0] = t;
    found[1] = lo + (int64_t)(tm - begin) * TBM;
    found[2] = hi;
  }
  __syncthreads();
  group = found[0];
  m0 = found[1];
  m_end = found[2];
  tn = tile % gn;
  return group >= 0;
}

// The steps of the epilogue that depend on the wavefront's half, with the
// half fixed at compile time (a run-time index into the accumulators would
// put them in scratch memory).  KEEP: the 32-row half (it) this wavefront
// finishes; 0 for the gate wavefront, 1 for the up wavefront.
template <int KEEP, int TN>
__device__ __forceinline__ void silu_hand_over(const v16f (&acc)[2][TN], float *mine, int lane) {
#pragma unroll
  for (int jt = 0; jt < TN; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mine[(jt * 16 + r) * 64 + lane] = acc[1 - KEEP][jt][r];
}

// 16 values at a time: their LDS reads go out together, the fp32 evaluation
// runs without branches, and only the lanes and values that need it repeat
// in binary64 (evaluated one by one with a branch each, every value waited
// for its own LDS read and took three branches: 43 us of the gate+up GEMM).
template <int KEEP, int TN>
__device__ __forceinline__ void silu_finish(v16f (&acc)[2][TN], const float *theirs, int lane, bool active) {
#pragma unroll
  for (int jt = 0; jt < TN; ++jt) {
    float other[16];
    uint32_t x[16], slow = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) other[r] = theirs[(jt * 16 + r) * 64 + lane];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float g = KEEP == 0 ? acc[KEEP][jt][r] : other[r];
      const float u = KEEP == 0 ? other[r] : acc[KEEP][jt][r];
      slow |= silu_mul_fast(g, u, x[r]) ? 0u : 1u << r;
    }
    // rows of a wavefront that skipped its MFMAs (all past the group's end:
    // zero gates, outputs not stored) leave their fast values unrepaired
    if (slow && active) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (slow & (1u << r)) {
          const float g = KEEP == 0 ? acc[KEEP][jt][r] : other[r];
          const float u = KEEP == 0 ? other[r] : acc[KEEP][jt][r];
          x[r] = silu_mul_slow(g, u);
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[KEEP][jt][r] = __uint_as_float(x[r]);
  }
}

template <int KEEP, int TN, int kHs>
__device__ __forceinline__ void silu_put_x(const v16f (&acc)[2][TN], uint16_t *xs, int wm, int h, int li) {
#pragma unroll
  for (int jt = 0; jt < TN; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + KEEP * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      xs[row * kHs + jt * 32 + li] = (uint16_t)__float_as_uint(acc[KEEP][jt][r]);
    }
}

// The exchange and x = bf16(silu(g) u) for this wavefront's half, then the x
// tile into LDS.  One function per half with its barriers inside: the half
// is wave-uniform (from the readfirstlane'd wavefront index, a scalar
// branch) and both halves pass the same four barriers.  With the halves'
// steps merged after run-time branches instead, the accumulators of both
// halves ended up in scratch memory.
template <int KEEP, int TN, int kHs, int kVals>
__device__ __forceinline__ void silu_x_tile(v16f (&acc)[2][TN], float *xch, uint16_t *xs, int wave,
                                            int wm, int h, int li, int lane, bool active) {
  __syncthreads();                      // every wavefront is done with the stages
  silu_hand_over<KEEP>(acc, xch + wave * kVals, lane);
  __syncthreads();
  silu_finish<KEEP>(acc, xch + (wave ^ 1) * kVals, lane, active);
  __syncthreads();                      // the exchange is read before the x tile overwrites it
  silu_put_x<KEEP, TN, kHs>(acc, xs, wm, h, li);
  __syncthreads();
}

// SiLU(gate) * up and the preparation of the result (the down projection's
// input), from the accumulators of a gate+up tile: its first TBN / 2 columns
// are the gate columns j0 .. j0 + TBN / 2 - 1 and its last TBN / 2 the up
// columns of the same j, so wavefront (wm, 0) holds the gate and wavefront
// (wm, 1) the up accumulators of rows 64 wm .. 64 wm + 63, lane for lane.
// Each of the two hands the other the half (32 rows) it does not finish
// itself through LDS (fp32, lane-major: no bank conflicts); each forms x =
// bf16(silu(g) u) for its own half, exactly as the preparation kernel does
// from the stored fp32 product; the tile of x (bf16, rows padded by 16 bytes)
// then goes to LDS, and every lane prepares 32-column blocks of it exactly as
// the preparation kernel prepares a block.  The stages' LDS is free by then.
template <int TBM, int TBN, int STAGES>
__device__ __forceinline__ void silu_prep_epilogue(DStage<TBM, TBN> (&st)[STAGES], v16f (&acc)[2][TBN / 64],
                                                   const PrepArgs &p, int64_t m0, int64_t m_end, int64_t j0,
                                                   int wave, int lane, int nit) {
  constexpr int TN = TBN / 64, HB = TBN / 2, NB = HB / 32;
  constexpr int kVals = TN * 16 * 64;   // floats one wavefront hands over
  constexpr int kHs = HB + 8;           // LDS row stride of the x tile, in bf16
  static_assert(TBM == 128 && HB % 32 == 0, "four wavefronts: two row halves x (gate, up)");
  static_assert(4 * kVals * sizeof(float) <= sizeof(st), "the exchange fits in the stages");
  static_assert(TBM * kHs * sizeof(uint16_t) <= sizeof(st), "the x tile fits in the stages");
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, li = lane & 31;
  float *xch = reinterpret_cast<float *>(&st[0]);
  uint16_t *xs = reinterpret_cast<uint16_t *>(&st[0]);
  // the wavefront finishing 32-row tile KEEP = wn of its rows
  if (wn == 0) silu_x_tile<0, TN, kHs, kVals>(acc, xch, xs, wave, wm, h, li, lane, nit > 0);
  else silu_x_tile<1, TN, kHs, kVals>(acc, xch, xs, wave, wm, h, li, lane, nit > 1);
  // blocks of a row sit in adjacent lanes: k-step-major outputs leave as
  // contiguous runs (the tile's columns are one 128-k step when HB = 128)
#pragma unroll
  for (int i = 0; i < TBM * NB / 256; ++i) {
    const int q = (int)threadIdx.x + 256 * i, r = q / NB, b = q % NB;
    const int64_t row = m0 + r;
    if (row >= m_end) continue;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(xs + r * kHs + 32 * b);
    uint32_t xw[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 t = src[c];
      xw[4 * c + 0] = t.x;
      xw[4 * c + 1] = t.y;
      xw[4 * c + 2] = t.z;
      xw[4 * c + 3] = t.w;
    }
    float xf[32];
    unpack32(xw, xf);
    BlockOut o;
    quantize_block_mx(xw, xf, o);
    store_block<0, false>(p, row, j0 / 32 + b, o);
  }
}

// One tile of the dense-operand GEMM.  SILU: a gate+up tile whose epilogue is
// silu_prep_epilogue (W's rows: n / 2 gate rows, then n / 2 up rows) instead
// of the fp32 Y stores.
template <int TBM, int TBN, int NW, int STAGES, bool GROUPED, bool SILU, bool BF16 = false>
__device__ __forceinline__ void dense_tile(const GemmArgs &a, uint32_t band, const PrepArgs *prep) {
  static_assert(TBM == 32 * NW, "two 32-row tiles per wavefront, two wavefronts per column");
  static_assert(!GROUPED || 64 * NW == 256, "the group scan takes one thread a group: 256 threads, 256 groups");
  constexpr int TN = TBN / 64;
  using P = DPlan<TBM, TBN, NW>;
  __shared__ DStage<TBM, TBN> st[STAGES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, li = lane & 31;
  uint32_t tm = 0, tn = 0;
  const uint32_t gn = (uint32_t)((a.n + TBN - 1) / TBN);
  if (!GROUPED) xcd_tile(blockIdx.x, (uint32_t)((a.m + TBM - 1) / TBM), gn, band, tm, tn);
  int64_t m0 = (int64_t)tm * TBM, m_end = a.m, group = 0;
  if (GROUPED && !grouped_tile<TBM>(a, blockIdx.x, gn, m0, m_end, group, tn)) return;   // uniform: no work
  const int64_t n0 = (int64_t)tn * TBN;
  const ARows arow{a.row_index, m0, m_end, GROUPED, !SILU};
  // a grouped tile's wavefronts skip the LDS reads and MFMAs of their 32-row
  // tiles that lie wholly past the group's end (nit of their two take part;
  // they still issue their share of the stage loads and meet every
  // barrier); those outputs are not stored, and the SiLU epilogue does not
  // repair their (zero-gate) values in binary64.
  const int64_t wr0 = m0 + wm * 64;
  const int nit = !GROUPED ? 2 : (wr0 >= m_end ? 0 : (wr0 + 32 >= m_end ? 1 : 2));
  const int64_t w_row0 = GROUPED ? group * a.n : 0, w_rows = GROUPED ? (group + 1) * a.n : a.n;

  v16f acc[2][TN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int ksteps = (int)(a.k / BK);
  DRsrc R;
  DOffs<TBM, TBN, NW> O;
  if constexpr (SILU)
    plan_loads<TBM, TBN, NW, true>(a, m0, 0, wave, lane, R, O, arow, w_row0, w_rows,
                                   WRows<true>{n0 / 2, a.n / 2, TBN / 2});
  else
    plan_loads<TBM, TBN, NW>(a, m0, n0, wave, lane, R, O, arow, w_row0, w_rows);
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < ksteps) issue_stage<TBM, TBN, NW>(R, O, wave, p, st[p]);

  // one step: wait for its stage, the barrier, the next stage's loads, and
  // (COMPUTE) the step's LDS reads and MFMAs
  int cur = 0;
  auto step = [&](int kt, auto compute) {
    // stages kt + 1 .. kt + STAGES - 2 may stay in flight
    const int ahead = min(ksteps - 1 - kt, STAGES - 2);
    if (STAGES == 3 && ahead >= 1) wait_vmcnt<P::kMinPerWave>();
    else wait_vmcnt<0>();
    stage_barrier();
    if (kt + STAGES - 1 < ksteps) {
      const int nxt = cur == 0 ? STAGES - 1 : cur - 1;
      issue_stage<TBM, TBN, NW>(R, O, wave, kt + STAGES - 1, st[nxt]);
    }
    if constexpr (decltype(compute)::value > 0)
      compute_stage<TBM, TBN, decltype(compute)::value>(st[cur], acc, wm, wn, h, li);
    cur = cur == STAGES - 1 ? 0 : cur + 1;
  };
  // the branch stays outside the loops, so that the accumulators keep their
  // registers through the loop
  if (nit == 2) {
    for (int kt = 0; kt < ksteps; ++kt) step(kt, std::integral_constant<int, 2>{});
  } else if (GROUPED && nit == 1) {
    for (int kt = 0; kt < ksteps; ++kt) step(kt, std::integral_constant<int, 1>{});
  } else if (GROUPED) {
    for (int kt = 0; kt < ksteps; ++kt) step(kt, std::integral_constant<int, 0>{});
  }

  if constexpr (SILU) {
    silu_prep_epilogue<TBM, TBN, STAGES>(st, acc, *prep, m0, m_end, n0 / 2, wave, lane, nit);
    return;
  }
  // Y leaves with non-temporal stores: nothing here reads it back, and fp32
  // tiles left dirty in the L2s (qkv shape: 50 MB against 32 MB of L2) slowed
  // the kernel's end and the next kernel's start (qkv GEMM 55.5 -> 52.9 us).
  // BF16 (sharq_dual_gemm_bf16): the same values rounded to bf16, in
  // instances of their own (the conversion's registers would otherwise count
  // against every fp32 instance: 128 x 256 grouped tiles went from two
  // wavefronts per SIMD to one)
  if constexpr (BF16)
    store_tile_bf16<TBM, TBN>(a.y16, a.ld_y, m0, n0, m_end, a.n, wm, wn, h, li, acc, 1.0f);
  else
    store_tile<TBM, TBN>(a.y, a.ld_y, m0, n0, m_end, a.n, wm, wn, h, li, acc, 1.0f);
}

template <int TBM, int TBN, int NW, int STAGES, bool GROUPED = false, bool BF16 = false>
__global__ __launch_bounds__(64 * NW) void dual_gemm_dense_kernel(GemmArgs a, uint32_t band) {
  dense_tile<TBM, TBN, NW, STAGES, GROUPED, false, BF16>(a, band, nullptr);
}

// The gate+up projection with SiLU(gate) * up and the down projection's
// preparation in its epilogue (no fp32 Y); GROUPED: every expert's, over the
// gathered rows of each group (the output rows are the grouped rows).  Two wavefronts per SIMD (two
// workgroups per CU, as the plain kernel): left alone the epilogue's
// registers took the kernel to 276 VGPRs, one wavefront per SIMD.
template <int TBM, int TBN, int NW, int STAGES, bool GROUPED = false>
__global__ __launch_bounds__(64 * NW, 2) void dual_gemm_silu_prep_kernel(GemmArgs a, uint32_t band, PrepArgs p) {
  dense_tile<TBM, TBN, NW, STAGES, GROUPED, true>(a, band, &p);
}

template <int TBM, int TBN, int NW, int STAGES>
void launch_grouped(const GemmArgs &a, hipStream_t s) {
  // an upper bound of the real tiles, rounded up to whole rounds of the 8 XCDs
  const int64_t gm = (a.m + TBM - 1) / TBM + a.groups, gn = (a.n + TBN - 1) / TBN;
  const int64_t tiles = (gm * gn + 7) / 8 * 8;
  dual_gemm_dense_kernel<TBM, TBN, NW, STAGES, true><<<dim3((unsigned)tiles), dim3(64 * NW), 0, s>>>(a, 0);
}

template <int TBM, int TBN, int NW, int STAGES>
void launch_dense(const GemmArgs &a, hipStream_t s) {
  const int64_t gm = (a.m + TBM - 1) / TBM, gn = (a.n + TBN - 1) / TBN;
  const uint32_t band = xcd_band_rows(gm, gn, TBM, TBN, TBN <= 128 ? 3 : 2);
  if (a.y16)
    dual_gemm_dense_kernel<TBM, TBN, NW, STAGES, false, true><<<dim3((unsigned)(gm * gn)), dim3(64 * NW), 0, s>>>(a, band);
  else
    dual_gemm_dense_kernel<TBM, TBN, NW, STAGES><<<dim3((unsigned)(gm * gn)), dim3(64 * NW), 0, s>>>(a, band);
}

// ---------------------------------------------------------------------------
// Prefill with the 2:4 backbone as the preparation wrote it (DECOMPRESS): the
// tiled kernel above, with the backbone streamed compressed (codes 32 and meta
// 16 bytes per row and 128-k step instead of 64 dense bytes) and expanded once
// per workgroup in LDS.  At step kt the workgroup computes step kt from stage
// kt % 2, and meanwhile (a) streams step kt + 1's residual, W and scales into
// stage (kt + 1) % 2, (b) streams step kt + 2's compressed backbone into the
// compressed area of stage kt % 2 (step kt's was expanded a step earlier),
// and (c) expands step kt + 1's compressed backbone, which landed during step
// kt - 1, into the dense area of stage (kt + 1) % 2.  One barrier a step.
// Every wavefront issues the same loads each step (padding loads read
// nothing: an empty buffer resource), so the loop has no branch; the steps
// past the end are fetched the same way and never used.
template <int TBM, int TBN>
struct XStage {
  u32x4 as[TBM * 4];           // dense backbone, expanded in LDS
  u32x4 ar[TBM * 4];
  u32x4 w[TBN * 4];
  uint32_t sas[TBM], sar[TBM], sws[TBN], swd[TBN];
  uint8_t codes[TBM * 32];     // compressed backbone: 32 code bytes a row
  uint8_t meta[TBM * 16];      // 16 meta bytes a row
  u32x4 spare[64];             // destination of padding loads
};

template <int TBM, int TBN, int NW>
struct XPlan {
  static constexpr int kChunks = TBM / 32 + TBM / 64 + TBM / 16 + TBN / 16;   // 16-byte loads
  static constexpr int kScales = 2 * (TBM / 64) + 2 * (TBN / 64);             // 4-byte loads
  static constexpr int kChunkPer = (kChunks + NW - 1) / NW, kScalePer = (kScales + NW - 1) / NW;
  static constexpr int kPerWave = kChunkPer + kScalePer;
};

// One load of this wavefront: resource, bytes per step, the lane's offset at
// step 0, its LDS offset within a stage, and which step it fetches at step
// kt (kt + 1 + ahead).
struct XLoad {
  i32x4 rsrc;
  uint32_t step, voff, lds, ahead;
};

template <int TBM, int TBN, int NW>
__device__ __forceinline__ void decomp_plan(const GemmArgs &a, int64_t m0, int64_t n0, int wave, int lane,
                                            XLoad (&L)[XPlan<TBM, TBN, NW>::kPerWave]) {
  using P = XPlan<TBM, TBN, NW>;
  using St = XStage<TBM, TBN>;
  const int64_t steps = a.k / BK;
  const OpStream sc = op_stream(a.s_codes, a.ld_sc, a.s_ksm, a.m, m0, steps, 32);
  const OpStream sm = op_stream(a.meta, a.ld_meta, a.s_ksm, a.m, m0, steps, 16);
  const OpStream ar = op_stream(a.r_codes, a.ld_rc, a.r_ksm, a.m, m0, steps, 64);
  const OpStream w = op_stream(a.w_codes, a.ld_wc, a.w_ksm, a.n, n0, steps, 64);
  const OpStream sas = op_stream(a.s_scales, a.ld_ss, a.s_ksm, a.m, m0, steps, 4);
  const OpStream sar = op_stream(a.r_scales, a.ld_rs, a.r_ksm, a.m, m0, steps, 4);
  const OpStream sws = op_stream(a.ws_scales, a.ld_wss, a.w_ksm, a.n, n0, steps, 4);
  const OpStream swd = op_stream(a.wd_scales, a.ld_wds, a.w_ksm, a.n, n0, steps, 4);
  const i32x4 none = make_rsrc(a.w_codes, 0u);
  constexpr int NC = TBM / 32, NM = TBM / 64, NA = TBM / 16, NB = TBN / 16;
  // 16-byte loads: compressed codes (32 rows of 32 bytes each), meta (64 rows
  // of 16 bytes), residual and W (16 rows of 64 bytes, chunk-swizzled)
#pragma unroll
  for (int j = 0; j < P::kChunkPer; ++j) {
    const int q = wave + NW * j;
    const int op = q < NC ? 0 : q < NC + NM ? 1 : q < NC + NM + NA ? 2 : q < NC + NM + NA + NB ? 3 : 4;
    const int i = op == 0 ? q : op == 1 ? q - NC : op == 2 ? q - NC - NM : q - NC - NM - NA;
    const OpStream o = op == 0 ? sc : op == 1 ? sm : op == 2 ? ar : w;
    uint32_t voff, lds;
    if (op == 0) {
      voff = (uint32_t)(32 * i + (lane >> 1)) * o.row_stride + (lane & 1) * 16;
      lds = (uint32_t)offsetof(St, codes) + (uint32_t)i * 1024;
    } else if (op == 1) {
      voff = (uint32_t)(64 * i + lane) * o.row_stride;
      lds = (uint32_t)offsetof(St, meta) + (uint32_t)i * 1024;
    } else {
      const int lrow = lane >> 2, lchunk = (lane & 3) ^ ((lane >> 4) & 3);
      voff = (uint32_t)(16 * i + lrow) * o.row_stride + lchunk * 16;
      lds = (op == 2 ? (uint32_t)offsetof(St, ar) : (uint32_t)offsetof(St, w)) + (uint32_t)i * 1024;
    }
    const bool real = op < 4;
    L[j].rsrc = real ? o.rsrc : none;
    L[j].step = real ? o.step : 0u;
    L[j].voff = real ? voff : 0u;
    L[j].lds = real ? lds : (uint32_t)offsetof(St, spare);
    L[j].ahead = op < 2 ? 1u : 0u;
  }
#pragma unroll
  for (int j = 0; j < P::kScalePer; ++j) {
    const int q = wave + NW * j;
    constexpr int TA = TBM / 64, T = TBN / 64;
    const int op = q < TA ? 0 : q < 2 * TA ? 1 : q < 2 * TA + T ? 2 : q < 2 * TA + 2 * T ? 3 : 4;
    const int i = op == 0 ? q : op == 1 ? q - TA : op == 2 ? q - 2 * TA : q - 2 * TA - T;
    const OpStream o = op == 0 ? sas : op == 1 ? sar : op == 2 ? sws : swd;
    const uint32_t lds = op == 0 ? (uint32_t)offsetof(St, sas) : op == 1 ? (uint32_t)offsetof(St, sar)
                       : op == 2 ? (uint32_t)offsetof(St, sws) : (uint32_t)offsetof(St, swd);
    const bool real = op < 4;
    XLoad &d = L[P::kChunkPer + j];
    d.rsrc = real ? o.rsrc : none;
    d.step = real ? o.step : 0u;
    d.voff = real ? (uint32_t)(64 * i + lane) * o.row_stride : 0u;
    d.lds = real ? lds + (uint32_t)i * 256 : (uint32_t)offsetof(St, spare);
    d.ahead = 0u;
  }
}

// The loads of step kt: each fetches step kt + 1 + ahead into stage
// (kt + 1 + ahead) % 2.  kRawOnly: only the compressed backbone's, for step
// kt + 2 (the prologue's step 0).
template <int TBM, int TBN, int NW, bool kRawOnly = false>
__device__ __forceinline__ void decomp_issue(const XLoad (&L)[XPlan<TBM, TBN, NW>::kPerWave], int kt,
                                             uint32_t base0, uint32_t base1) {
  using P = XPlan<TBM, TBN, NW>;
#pragma unroll
  for (int j = 0; j < P::kPerWave; ++j) {
    if (kRawOnly && !L[j].ahead) continue;
    // (uniform values; readfirstlane keeps them in scalar registers)
    const uint32_t t = (uint32_t)kt + 1u + L[j].ahead;
    const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane((int)(t * L[j].step));
    const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)(((t & 1u) ? base1 : base0) + L[j].lds));
    if (j < P::kChunkPer) b2l16(L[j].rsrc, L[j].voff, soff, lds);
    else b2l4(L[j].rsrc, L[j].voff, soff, lds);
  }
}

// The workgroup expands a stage's compressed backbone into its dense area:
// unit u = 16 dense bytes (chunk u % 4 of row u / 4) from 8 code bytes and 4
// meta bytes.
template <int TBM, int TBN, int NW>
__device__ __forceinline__ void decomp_expand(XStage<TBM, TBN> &S, int tid) {
#pragma unroll
  for (int i = 0; i < TBM * 4 / (64 * NW); ++i) {
    const int u = tid + 64 * NW * i, r = u >> 2, c = u & 3;
    const u32x2 cb = *reinterpret_cast<const u32x2 *>(S.codes + r * 32 + 8 * c);
    const uint32_t mb = *reinterpret_cast<const uint32_t *>(S.meta + r * 16 + 4 * c);
    uint32_t d[4];
    expand8(cb.x, cb.y, mb, d);
    S.as[lds_slot(r, c)] = u32x4{d[0], d[1], d[2], d[3]};
  }
}

// Expansion of one stage's compressed backbone as side work of the MFMAs.
template <int TBM, int TBN, int NW>
struct ExpandSide {
  static constexpr int kUnits = TBM * 4 / (64 * NW);
  static constexpr int kValuPerMfma = 6;
  XStage<TBM, TBN> *S;
  int tid;
  u32x2 cb[kUnits];
  uint32_t mb[kUnits];
  __device__ __forceinline__ void pre() {
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      const int u = tid + 64 * NW * i, r = u >> 2, c = u & 3;
      cb[i] = *reinterpret_cast<const u32x2 *>(S->codes + r * 32 + 8 * c);
      mb[i] = *reinterpret_cast<const uint32_t *>(S->meta + r * 16 + 4 * c);
    }
  }
  __device__ __forceinline__ void post() {
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      const int u = tid + 64 * NW * i, r = u >> 2, c = u & 3;
      uint32_t d[4];
      expand8(cb[i].x, cb[i].y, mb[i], d);
      S->as[lds_slot(r, c)] = u32x4{d[0], d[1], d[2], d[3]};
    }
  }
};

template <int TBM, int TBN, int NW, bool BF16 = false>
__global__ __launch_bounds__(64 * NW) void dual_gemm_decomp_kernel(GemmArgs a, uint32_t band) {
  static_assert(TBM == 32 * NW, "two 32-row tiles per wavefront, two wavefronts per column");
  constexpr int TN = TBN / 64;
  using P = XPlan<TBM, TBN, NW>;
  __shared__ XStage<TBM, TBN> st[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, li = lane & 31;
  uint32_t tm, tn;
  xcd_tile(blockIdx.x, (uint32_t)((a.m + TBM - 1) / TBM), (uint32_t)((a.n + TBN - 1) / TBN), band, tm, tn);
  const int64_t m0 = (int64_t)tm * TBM, n0 = (int64_t)tn * TBN;

  v16f acc[2][TN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int ksteps = (int)(a.k / BK);
  XLoad L[P::kPerWave];
  decomp_plan<TBM, TBN, NW>(a, m0, n0, wave, lane, L);
  const uint32_t base0 = lds_addr(&st[0]), base1 = lds_addr(&st[1]);
  // prologue: step 0's compressed backbone, then step 0's other operands and
  // step 1's compressed backbone
  decomp_issue<TBM, TBN, NW, true>(L, -2, base0, base1);
  decomp_issue<TBM, TBN, NW>(L, -1, base0, base1);
  wait_vmcnt<0>();
  stage_barrier();
  decomp_expand<TBM, TBN, NW>(st[0], tid);

  for (int kt = 0; kt < ksteps; ++kt) {
    const int cur = kt & 1;
    // every load issued at step kt - 1 has landed (step kt's operands, step
    // kt + 1's compressed backbone); the barrier also publishes step kt's
    // expansion and frees stage (kt + 1) % 2 and step kt's compressed area
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    stage_barrier();
    decomp_issue<TBM, TBN, NW>(L, kt, base0, base1);
    compute_stage<TBM, TBN>(st[cur], acc, wm, wn, h, li, ExpandSide<TBM, TBN, NW>{&st[cur ^ 1], tid});
  }
  // no loads may land in LDS after the workgroup ends
  wait_vmcnt<0>();

#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < TN; ++jt) {
      const int64_t col = n0 + wn * (TBN / 2) + jt * 32 + li;
      if (col >= a.n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + it * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < a.m) put_y<true>(a.y, BF16 ? a.y16 : nullptr, row * a.ld_y + col, acc[it][jt][r]);
      }
    }
}

template <int TBM, int TBN, int NW>
void launch_decomp(const GemmArgs &a, hipStream_t s) {
  const int64_t gm = (a.m + TBM - 1) / TBM, gn = (a.n + TBN - 1) / TBN;
  const uint32_t band = xcd_band_rows(gm, gn, TBM, TBN, TBN >= 256 ? 1 : 2);
  if (a.y16)
    dual_gemm_decomp_kernel<TBM, TBN, NW, true><<<dim3((unsigned)(gm * gn)), dim3(64 * NW), 0, s>>>(a, band);
  else
    dual_gemm_decomp_kernel<TBM, TBN, NW><<<dim3((unsigned)(gm * gn)), dim3(64 * NW), 0, s>>>(a, band);
}


// ---------------------------------------------------------------------------
// Skinny kernel for m <= 32 (decode): the GEMM streams W once and is bound by
// HBM bandwidth, not by the MFMAs.  A workgroup of NW wavefronts owns all
// rows (padded to 32 with zeros) x 32 columns; its wavefronts split K (128-k
// steps w, w + NW, ...), each loading its fragments straight from global
// memory (W streams once; A is small and stays in L2), and the NW partial
// tiles are summed through LDS as a fixed pairwise tree.  Many short
// wavefronts keep more loads in flight than a few long ones.  Lane (h, li):
// row / column li, k blocks 2h (first MFMA) and 2h + 1 (second), as in the
// tiled kernels.
// The 32-bit word of E8M0 scales of row r for 128-k step kt.
__device__ __forceinline__ uint32_t scale_word(const uint8_t *p, int64_t ld, int ksm, int64_t r,
                                               int kt) {
  return *reinterpret_cast<const uint32_t *>(p + arr_off(r, kt, ld, ksm, 4));
}

struct SkFrag {
  u32x4 fs[2], fr[2], fw[2];
  int sas, sar, sws, swd;
};

template <bool kDense>
__device__ __forceinline__ void sk_load(const GemmArgs &a, int kt, int h, bool row_ok, bool col_ok,
                                        int64_t r, int64_t c, SkFrag &F) {
  const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int chunk = 2 * h + s;
    F.fr[s] = row_ok ? *reinterpret_cast<const u32x4 *>(a.r_codes + arr_off(r, kt, a.ld_rc, a.r_ksm, 64) + chunk * 16) : z;
    F.fw[s] = col_ok ? *reinterpret_cast<const u32x4 *>(a.w_codes + arr_off(c, kt, a.ld_wc, a.w_ksm, 64) + chunk * 16) : z;
    if (kDense) {
      F.fs[s] = row_ok ? *reinterpret_cast<const u32x4 *>(a.s_dense + arr_off(r, kt, a.ld_sd, a.s_ksm, 64) + chunk * 16) : z;
    } else if (row_ok) {
      const u32x2 cb = *reinterpret_cast<const u32x2 *>(a.s_codes + arr_off(r, kt, a.ld_sc, a.s_ksm, 32) + chunk * 8);
      const uint32_t mb = *reinterpret_cast<const uint32_t *>(a.meta + arr_off(r, kt, a.ld_meta, a.s_ksm, 16) + chunk * 4);
      uint32_t d[4];
      expand8(cb.x, cb.y, mb, d);
      F.fs[s] = u32x4{d[0], d[1], d[2], d[3]};
    } else {
      F.fs[s] = z;
    }
  }
  F.sas = row_ok ? (int)(scale_word(a.s_scales, a.ld_ss, a.s_ksm, r, kt) >> (16 * h)) : 0;
  F.sar = row_ok ? (int)(scale_word(a.r_scales, a.ld_rs, a.r_ksm, r, kt) >> (16 * h)) : 0;
  F.sws = col_ok ? (int)(scale_word(a.ws_scales, a.ld_wss, a.w_ksm, c, kt) >> (16 * h)) : 0;
  F.swd = col_ok ? (int)(scale_word(a.wd_scales, a.ld_wds, a.w_ksm, c, kt) >> (16 * h)) : 0;
}

__device__ __forceinline__ void sk_mfma(const SkFrag &F, v16f &acc) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand(F.fs[0]), as_operand(F.fw[0]), acc, 4, 4, 0, F.sas, 0, F.sws);
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand(F.fr[0]), as_operand(F.fw[0]), acc, 4, 4, 0, F.sar, 0, F.swd);
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand(F.fs[1]), as_operand(F.fw[1]), acc, 4, 4, 1, F.sas, 1, F.sws);
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as_operand(F.fr[1]), as_operand(F.fw[1]), acc, 4, 4, 1, F.sar, 1, F.swd);
}

template <bool kDense, int U, int NW>
__global__ __launch_bounds__(64 * NW) void dual_gemm_skinny_kernel(GemmArgs a) {
  __shared__ float part[NW][64][17];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  const bool row_ok = li < a.m;
  const int64_t col = n0 + li;
  const bool col_ok = col < a.n;
  const int64_t r = row_ok ? li : 0, c = col_ok ? col : 0;
  const int ksteps = (int)(a.k / BK);

  v16f acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

  // wavefront w takes 128-k steps w, w + NW, ...; U steps' loads in flight
  // before their MFMAs
  int kt = wave;
  for (; kt + NW * (U - 1) < ksteps; kt += NW * U) {
    SkFrag F[U];
#pragma unroll
    for (int u = 0; u < U; ++u) sk_load<kDense>(a, kt + NW * u, h, row_ok, col_ok, r, c, F[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) sk_mfma(F[u], acc);
  }
  for (; kt < ksteps; kt += NW) {
    SkFrag F;
    sk_load<kDense>(a, kt, h, row_ok, col_ok, r, c, F);
    sk_mfma(F, acc);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) part[wave][lane][i] = acc[i];
  __syncthreads();
  // thread t sums (lane t % 64, accumulator slots (t / 64) * 16 / NW ..) over
  // the wavefronts as a fixed pairwise tree
  constexpr int SLOTS = 16 / NW;
  static_assert(SLOTS >= 1 && 16 % NW == 0, "NW divides 16");
  const int l = tid & 63, q = tid >> 6;
  const int64_t ocol = n0 + (l & 31);
  if (ocol < a.n) {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int i = SLOTS * q + j;
      const int row = 8 * (i >> 2) + 4 * (l >> 5) + (i & 3);
      float v[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) v[w] = part[w][l][i];
#pragma unroll
      for (int width = NW / 2; width >= 1; width >>= 1)
#pragma unroll
        for (int w = 0; w < width; ++w) v[w] = v[2 * w] + v[2 * w + 1];
      if (row < a.m) put_y<false>(a.y, a.y16, row * a.ld_y + ocol, v[0]);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode kernel for m <= 32: the GEMM streams W once and is bound by HBM
// bandwidth.  A workgroup of four wavefronts owns all rows (padded to 32 with
// zeros) x 128 columns, one 32 x 32 MFMA tile per wavefront, over the whole
// K.  W, both A operands and the four scale arrays go global -> LDS with
// buffer_load ... lds through a ring of STAGES 128-k steps (STAGES - 1 in
// flight), which keeps far more bytes in flight than loads into registers.
// Lane (h, li): row / column li, k blocks 2h (first MFMA) and 2h + 1.
template <int STAGES>
struct KStage {
  u32x4 w[128 * 4];            // 128 W rows x 64 bytes (chunk-swizzled)
  u32x4 as[32 * 4], ar[32 * 4];
  uint32_t sws[128], swd[128], sas[64], sar[64];   // A scale rows 32..63 stay unused
};

template <int STAGES>
__global__ __launch_bounds__(256) void dual_gemm_decode_kernel(GemmArgs a) {
  __shared__ KStage<STAGES> st[STAGES];
  using St = KStage<STAGES>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * 128;
  const int64_t steps = a.k / BK;
  const int ksteps = (int)steps;

  // streams and this wavefront's loads: W chunk groups 2w, 2w + 1 (16 rows
  // each); wave 0 the backbone rows and scales, wave 1 the residual's, waves
  // 2 and 3 the two W scale views
  const OpStream sw = op_stream(a.w_codes, a.ld_wc, a.w_ksm, a.n, n0, steps, 64);
  const int lrow = lane >> 2, lchunk = (lane & 3) ^ ((lane >> 4) & 3);
  const uint32_t vw0 = (uint32_t)(16 * (2 * wave) + lrow) * sw.row_stride + lchunk * 16;
  const uint32_t vw1 = (uint32_t)(16 * (2 * wave + 1) + lrow) * sw.row_stride + lchunk * 16;
  OpStream sa, ss;
  uint32_t osa = 0, oss = 0;
  if (wave == 0) {
    sa = op_stream(a.s_dense, a.ld_sd, a.s_ksm, a.m, 0, steps, 64);
    ss = op_stream(a.s_scales, a.ld_ss, a.s_ksm, a.m, 0, steps, 4);
    osa = offsetof(St, as); oss = offsetof(St, sas);
  } else if (wave == 1) {
    sa = op_stream(a.r_codes, a.ld_rc, a.r_ksm, a.m, 0, steps, 64);
    ss = op_stream(a.r_scales, a.ld_rs, a.r_ksm, a.m, 0, steps, 4);
    osa = offsetof(St, ar); oss = offsetof(St, sar);
  } else {
    ss = wave == 2 ? op_stream(a.ws_scales, a.ld_wss, a.w_ksm, a.n, n0, steps, 4)
                   : op_stream(a.wd_scales, a.ld_wds, a.w_ksm, a.n, n0, steps, 4);
    oss = wave == 2 ? offsetof(St, sws) : offsetof(St, swd);
  }
  const uint32_t va0 = (uint32_t)lrow * sa.row_stride + lchunk * 16;
  const uint32_t va1 = (uint32_t)(16 + lrow) * sa.row_stride + lchunk * 16;
  const uint32_t vs0 = (uint32_t)lane * ss.row_stride;
  const uint32_t vs1 = (uint32_t)(64 + lane) * ss.row_stride;

  // A rows 16..31 exist only for m > 16: with m <= 16 their load would read
  // nothing (past the end) and only cost issue slots; the rows' LDS then holds
  // stale codes whose scales are 0 (rows past m load as zeros), and those
  // output rows are never stored
  const bool two_a = a.m > 16;
  auto issue = [&](int kt, const St &S) {
    const uint32_t base = lds_addr(&S), t = (uint32_t)kt;
    b2l16(sw.rsrc, vw0, t * sw.step, base + offsetof(St, w) + (2 * wave) * 1024);
    b2l16(sw.rsrc, vw1, t * sw.step, base + offsetof(St, w) + (2 * wave + 1) * 1024);
    if (wave < 2) {
      b2l16(sa.rsrc, va0, t * sa.step, base + osa);
      if (two_a) b2l16(sa.rsrc, va1, t * sa.step, base + osa + 1024);
      b2l4(ss.rsrc, vs0, t * ss.step, base + oss);
    } else {
      b2l4(ss.rsrc, vs0, t * ss.step, base + oss);
      b2l4(ss.rsrc, vs1, t * ss.step, base + oss + 256);
    }
  };

  v16f acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < ksteps) issue(p, st[p]);

  const int wc = 32 * wave + li;     // the lane's W row within the tile
  int cur = 0;
  for (int kt = 0; kt < ksteps; ++kt) {
    // stages kt + 1 .. kt + STAGES - 2 may stay in flight (4 or 5 loads each)
    if (kt + STAGES - 2 < ksteps) wait_vmcnt<4 * (STAGES - 2)>();
    else wait_vmcnt<0>();
    stage_barrier();
    if (kt + STAGES - 1 < ksteps) issue(kt + STAGES - 1, st[cur == 0 ? STAGES - 1 : cur - 1]);
    const St &S = st[cur];
    const int sas = (int)(S.sas[li] >> (16 * h)), sar = (int)(S.sar[li] >> (16 * h));
    const int sws = (int)(S.sws[wc] >> (16 * h)), swd = (int)(S.swd[wc] >> (16 * h));
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 2 * h + s;
      const v8i fs = as_operand(S.as[lds_slot(li, c)]);
      const v8i fr = as_operand(S.ar[lds_slot(li, c)]);
      const v8i fw = as_operand(S.w[lds_slot(wc, c)]);
      if (s == 0) {
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fs, fw, acc, 4, 4, 0, sas, 0, sws);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr, fw, acc, 4, 4, 0, sar, 0, swd);
      } else {
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fs, fw, acc, 4, 4, 1, sas, 1, sws);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr, fw, acc, 4, 4, 1, sar, 1, swd);
      }
    }
    cur = cur == STAGES - 1 ? 0 : cur + 1;
  }
  const int64_t col = n0 + wc;
  if (col < a.n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < a.m) put_y<false>(a.y, a.y16, row * a.ld_y + col, acc[r]);
    }
  }
}

}  // namespace

// Grouped (mixture-of-experts) dual GEMM over the dense backbone view: the
// prefill kernel's tiles, 128 x 256 when there are enough of them (a group's
// short K makes each tile's prologue and epilogue weigh more, and wider tiles
// have fewer: Qwen3-30B-A3B's gate+up 189 -> 176 us against 128 x 192), else
// 128 x 192 or 128 x 128.
hipError_t launch_dual_gemm_silu_prep_mx(const GemmArgs &a, const PrepArgs &p, hipStream_t s) {
  // 128 x 256 tiles: 128 columns of x (one 128-k step of the down
  // projection's operands) from 128 gate and 128 up columns
  constexpr int TBM = 128, TBN = 256;
  const int64_t gm = (a.m + TBM - 1) / TBM, gn = a.n / TBN;
  dual_gemm_silu_prep_kernel<TBM, TBN, 4, 2>
      <<<dim3((unsigned)(gm * gn)), dim3(256), 0, s>>>(a, xcd_band_rows(gm, gn, TBM, TBN, 2), p);
  return hipGetLastError();
}

hipError_t launch_grouped_dual_gemm_silu_prep_mx(const GemmArgs &a, const PrepArgs &p, hipStream_t s) {
  // the grouped kernel's upper bound of the tiles, whole rounds of the 8 XCDs
  constexpr int TBM = 128, TBN = 256;
  const int64_t gm = (a.m + TBM - 1) / TBM + a.groups, gn = a.n / TBN;
  const int64_t tiles = (gm * gn + 7) / 8 * 8;
  dual_gemm_silu_prep_kernel<TBM, TBN, 4, 2, true><<<dim3((unsigned)tiles), dim3(256), 0, s>>>(a, 0, p);
  return hipGetLastError();
}

hipError_t launch_grouped_dual_gemm_mx(const GemmArgs &a, hipStream_t s) {
  const int64_t mt = (a.m + 127) / 128 + a.groups;
  if (mt * ((a.n + 255) / 256) >= 512 && a.k <= 8192)
    launch_grouped<128, 256, 4, 2>(a, s);
  else if (mt * ((a.n + 191) / 192) >= 512 && a.k <= 8192)
    launch_grouped<128, 192, 4, 2>(a, s);
  else
    launch_grouped<128, 128, 4, 2>(a, s);
  return hipGetLastError();
}

hipError_t launch_dual_gemm_mx(const GemmArgs &a, bool dense_expanded, hipStream_t s) {
  // decode with fewer 128-column tiles than half the CUs (Llama-3.1-8B's QKV,
  // O and down projections at 16 tokens): one workgroup a 32-column tile, K
  // split over sixteen wavefronts, so that four times as many CUs stream W
  // (measured at 16 tokens: QKV 11.1 -> 5.9 us, O 11.1 -> 5.1, down 32.7 ->
  // 12.9; gate+up, 224 tiles, stays on the decode kernel: 12.4 against 19.1)
  const bool few_tiles = (a.n + 127) / 128 < 128;
  const dim3 g32((unsigned)((a.n + 31) / 32));
  if (a.m <= 32 && few_tiles) {
    if (dense_expanded) dual_gemm_skinny_kernel<true, 1, 16><<<g32, dim3(1024), 0, s>>>(a);
    else dual_gemm_skinny_kernel<false, 1, 16><<<g32, dim3(1024), 0, s>>>(a);
  } else if (a.m <= 32 && dense_expanded) {
    // decode: W streams through LDS, four 128-k steps in flight
    dual_gemm_decode_kernel<4><<<dim3((unsigned)((a.n + 127) / 128)), dim3(256), 0, s>>>(a);
  } else if (a.m <= 32) {
    // decode with the 2:4 backbone expanded in registers: split-K over four
    // wavefronts, fragments loaded straight from global memory
    dual_gemm_skinny_kernel<false, 1, 4><<<g32, dim3(256), 0, s>>>(a);
  } else if (dense_expanded) {
    // 128-row tiles, two LDS stages: 128 x 192 (two workgroups a CU) when
    // that still gives every CU two tiles and K is short; else 128 x 128
    // (three a CU), whose smaller K step keeps more loads in flight per CU
    const int64_t mt = (a.m + 127) / 128;
    if (mt * ((a.n + 191) / 192) >= 512 && a.k <= 8192)
      launch_dense<128, 192, 4, 2>(a, s);
    else
      launch_dense<128, 128, 4, 2>(a, s);
  } else {
    // the same tiles; 128 x 256 when that still gives every CU a tile: the
    // expansion's cost per step does not grow with TBN, the MFMAs' does
    const int64_t mt = (a.m + 127) / 128;
    if (mt * ((a.n + 191) / 192) >= 512 && a.k <= 8192)
      launch_decomp<128, 192, 4>(a, s);
    else if (mt * ((a.n + 255) / 256) >= 256)
      launch_decomp<128, 256, 4>(a, s);
    else
      launch_decomp<128, 128, 4>(a, s);
  }
  return hipGetLastError();
}

}  // namespace sharq
