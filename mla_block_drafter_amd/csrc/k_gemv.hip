// Work planning and format dispatch of the skinny GEMM (kernels in gemv_impl.h,
// instantiated per weight format in k_gemv_<fmt>.hip).
#include <algorithm>
#include <cmath>

#include "kernels.h"

namespace dspark {

// Split-K fills one round of resident waves: at most kMaxWaves (eight per CU
// at the GEMM kernels' occupancy), so no nearly empty second round doubles
// the time.  In the pass this beat a lower target that cold-cache
// microbenchmarks of single launches preferred.
constexpr int kMaxWaves = 2048;

GemvPlan plan_gemv(const PackedMat& w, int M, bool allow_split, bool gather, bool i8_in) {
  GemvPlan p{};
  const bool f32 = w.fmt == DT_F32;
  p.hilo = (!f32 && !gather && M <= 8) ? 1 : 0;
  p.MT = p.hilo ? 1 : (M + 15) / 16;
  const int T = w.ngroups * w.TG;
  // Several tiles per wave share one activation fragment per k step (and,
  // with LDS staging, one staged slice per workgroup); split-K then restores
  // the wave count.
  // Two tiles per wave streamed best for most M = 7 shapes (the unsplit
  // 163,840-row lm_head included).  Four won where split-K still leaves
  // enough waves: the Markov gather GEMM (k range only 256) and split
  // matrices of at least 1792 tiles (the fused 28,672-row gate/up).  One
  // when the matrix has too few tiles.
  p.TPW = 1;
  if (p.MT == 1 && w.fmt == DT_MXFP4) {
    // four tiles share each quad's four activation fragments (a 16-row
    // tile's quad of E2M1 codes is only 1 KiB); with a short k range
    // (q_b's 1536) two tiles per wave measured faster
    if (w.TG % 4 == 0 && w.KB >= 128 && T / 4 >= (allow_split ? 64 : 256)) p.TPW = 4;
    else if (w.TG % 2 == 0 && T / 2 >= (allow_split ? 64 : 256)) p.TPW = 2;
  } else if (p.MT > 1) {
    // several m-tiles: four tiles per wave share every activation fragment
    // load (with one, the fragments of all m-tiles were re-read from L2 for
    // every 16 weight rows).  Not for eight m-tiles (their accumulators alone
    // take 128 registers) nor for the per-head W_UK / W_UV groups (measured
    // slower there).  FP8 and BF16 weights read the fragments from LDS (A_LDS_BF),
    // where two tiles per wave measured faster: half the registers, so two
    // waves per SIMD hide each other's waits.
    if (!gather && p.MT <= 7 && w.ngroups == 1 && w.TG % 4 == 0 && T / 4 >= 64)
      p.TPW = (w.fmt == DT_FP8 || w.fmt == DT_BF16) ? 2 : 4;
  } else if (p.MT == 1) {
    if (w.TG % 4 == 0 && ((gather && T / 4 >= 256) || (allow_split && T / 4 >= 448))) p.TPW = 4;
    else if (w.TG % 2 == 0 && T / 2 >= (allow_split ? 128 : 256)) p.TPW = 2;
  }
  const int waves = T / p.TPW;
  const int ksteps = f32 ? (w.Kp >> 4) : w.KB;
  // activation fragments of several m-tiles shared through LDS (A_LDS_BF),
  // whose k loop steps over pairs of k blocks; lds_bf_waves() waves per
  // workgroup share each staged chunk
  // (grouped matrices too when every workgroup's tiles lie in one group and
  // the k range is one staged chunk: the per-head W_UK, K = 128, went from 23
  // to 15 us per launch at M = 112; W_UV, K = 512 in four chunks over only
  // 128 workgroups, measured slower staged and reads its fragments directly)
  const bool lds_bf = (w.fmt == DT_FP8 || w.fmt == DT_BF16) && p.MT > 1 && !gather &&
                      (w.ngroups == 1 || (w.TG % (p.TPW * lds_bf_waves(w.fmt)) == 0 && w.KB <= LDS_BF_CK));
  const int wpg = lds_bf ? lds_bf_waves(w.fmt) : 4;
  p.grid_x = (waves + wpg - 1) / wpg;
  const int unit = w.fmt == DT_MXFP4 ? 4 : (w.fmt == DT_Q8_0 || w.fmt == DT_FP8 || lds_bf) ? 2 : 1;
  int S = 1;
  if (allow_split)
    S = std::max(1, std::min(kMaxWaves / std::max(waves, 1), ksteps / 8));
  int per = (ksteps + S - 1) / S;
  per = (per + unit - 1) / unit * unit;
  // activation staging in LDS (every tile of a workgroup in one group):
  // bf16 fragments 1 KiB per k step and 16-row tile, int8 codes 512 B per
  // k step; at most 64 KiB per workgroup (two workgroups per CU)
  const bool one_group = w.ngroups == 1 || w.TG % (4 * p.TPW) == 0;
  const bool i8 = w.fmt == DT_Q8_0 && p.hilo;
  const int cap = i8 ? 126 : 64;
  // Producers write the consumer's fragments directly (no staging in the
  // GEMM): bf16 hi/lo fragments for BF16 / FP8 weights, int8 hi/lo codes for
  // Q8_0 when the producer supports them; otherwise Q8_0 stages fp32 rows.
  p.amode = 0;
  if (lds_bf) {
    p.amode = 5;  // A_LDS_BF: the workgroup's activation chunks shared through LDS
  } else if (i8 && i8_in && !gather) {
    p.amode = 3;
  } else if (w.fmt == DT_Q8_0 && !gather && one_group) {
    if (allow_split) {
      while ((long long)p.MT * per > cap) per = ((per / 2) + unit - 1) / unit * unit;
    }
    if ((long long)p.MT * per <= cap) p.amode = i8 ? 2 : 1;
  }
  p.ksteps_per_split = per;
  p.S = (ksteps + per - 1) / per;
  return p;
}

// Share of the reduction taken by waves 0..3 of an eight-wave column-owning
// workgroup.
constexpr double OWN_SPLIT_HI = 0.5625;

// Column-owning plan: a workgroup per OWN_COLS output columns, its waves
// splitting the reduction.  About 2000 waves in all (eight per workgroup for
// the 224-workgroup hidden-size outputs, four for the 448 of the fused
// gate/up), each with at least one k unit.
GemvPlan plan_own(const PackedMat& w, int M, bool swiglu, bool i8_in) {
  GemvPlan p{};
  if (M < 1 || M > 8 || w.ngroups != 1 || w.fmt == DT_F32) return p;
  if (w.fmt == DT_Q8_0 && !i8_in) return p;
  if (swiglu && (w.G % 2 || w.TG * 16 != w.G)) return p;
  const int outG = swiglu ? w.G / 2 : w.G;
  if (outG % OWN_COLS) return p;
  const int nwg = outG / OWN_COLS;
  const int unit = w.fmt == DT_MXFP4 ? 4 : (w.fmt == DT_Q8_0 || w.fmt == DT_FP8) ? 2 : 1;
  const int units = (w.KB + unit - 1) / unit;
  int nw = nwg >= 384 ? 4 : 8;
  if (units < nw) nw = 4;
  int per = (units + nw - 1) / nw * unit, lo = per;
  if (nw == 8) {
    // Waves 4..7 share their SIMDs with waves 0..3 and lose the issue
    // arbitration to the older waves (about a fifth slower on the same
    // k range, measured), so waves 0..3 take the larger share.
    const int hi_u = std::min(units, (int)std::ceil(units * OWN_SPLIT_HI / 4.0));
    const int lo_u = std::max(0, (units - 4 * hi_u + 3) / 4);
    per = hi_u * unit;
    lo = lo_u * unit;
  }
  p.hilo = 1;
  p.MT = 1;
  p.TPW = swiglu ? 4 : 2;
  p.nw = nw;
  p.grid_x = nwg;
  p.S = 1;
  p.ksteps_per_split = per;
  p.ksteps_lo = lo;
  p.amode = w.fmt == DT_Q8_0 ? 3 : 0;
  return p;
}

hipError_t launch_gemv_bf16(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st);
hipError_t launch_gemv_q8_0(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st);
hipError_t launch_gemv_fp8(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st);
hipError_t launch_gemv_mxfp4(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st);
hipError_t launch_gemv_f32(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st);

hipError_t launch_gemv(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st) {
  if (mode != GEMV_STORE && mode != GEMV_MARKOV && p.S != 1) return hipErrorInvalidValue;
  if ((mode == GEMV_OWN) != (p.nw > 0)) return hipErrorInvalidValue;
  switch (a.w.fmt) {
    case DT_BF16: return launch_gemv_bf16(a, p, mode, st);
    case DT_Q8_0: return launch_gemv_q8_0(a, p, mode, st);
    case DT_FP8: return launch_gemv_fp8(a, p, mode, st);
    case DT_MXFP4: return launch_gemv_mxfp4(a, p, mode, st);
    case DT_F32: return launch_gemv_f32(a, p, mode, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dspark
