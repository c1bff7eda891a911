// Skinny GEMM for the draft pass: M = 7 activation rows per sequence against a
// weight matrix streamed once from HBM (weight-only BF16 / Q8_0 / FP8 / MXFP4 / F32).
//
// Why MFMA for a 7-row product: with packed-fp32 VALU ops unavailable, a VALU
// dot product costs 7 FMAs plus a decode per weight element, about 700 us of
// issue time for the full-size pass against a 630 us HBM floor.  The
// v_mfma_f32_16x16x32_bf16 path costs ~1.5 VALU ops per element (decode only);
// the 16-row MFMA is mostly padding, so rows 8..15 carry the bf16 residual of
// the activations (hi/lo split) for near-fp32 accuracy at no extra cost.
//
// Work decomposition: each wave owns TPW consecutive 16-row tiles and one
// k range (split-K over blockIdx.y).  Weight chunks are read with non-temporal
// 16-byte loads (contiguous 1 KiB per wave per step); the small activation
// fragments stay L2 resident.  Split-K partial sums go to a workspace slice per
// split and are reduced, in a fixed order, by the consuming kernel.
#pragma once

#include <algorithm>

#include "kernels.h"

namespace dspark {

namespace {

template <typename T>
__device__ __forceinline__ T ntload(const T* p) {
  return __builtin_nontemporal_load(p);
}

// Buffer loads for the k loops.  Every stage issues the same loads whatever
// the k range: a load past the range (the last stage of a wave's k range
// may be partial) gets offset BUF_OOB, beyond the resource's size, so it
// returns zeros without touching memory.  The stage loop then has no
// conditional loads, and the compiler's wait counts stay exact (after a
// conditionally skipped load it must wait for every load in flight, which
// drains the prefetched stage).
constexpr uint32_t BUF_OOB = 0x80000000u;
constexpr int BUF_NT = 2;  // cache policy: non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Markov predecessor of position a.step for sequence m (callers treat values
// outside [0, vocab) as "no predecessor").
__device__ __forceinline__ int markov_prev(const GemvArgs& a, int m) {
  if (a.step == 0) return a.prev_token[m];
  if (a.forced) return a.forced[m * a.block + a.step - 1];
  const unsigned long long* k = a.keys + ((long long)m * a.block + a.step - 1) * KEY_SLOTS;
  unsigned long long best = 0;
#pragma unroll
  for (int i = 0; i < KEY_SLOTS; ++i) best = best > k[i] ? best : k[i];
  return key_index(best);
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int o) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, o, 64);
  hi = __shfl_xor(hi, o, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Row scales of this lane's output rows 16 mt + 4 (lane >> 4) + r, by the
// whole wave: the chunk sums of all 16 rows of an m-tile are loaded together
// (one memory round trip) and each is reduced by wave_sum (the same order,
// hence the same bits, as every other consumer of these chunk sums).
template <int MT>
__device__ __forceinline__ void gemv_row_scales(const RowScale& s, int M, int lane, float (&rsv)[MT][4]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float t[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int m = mt * 16 + j;
      t[j] = m < M ? chunk_lane_sum(s.ssq + (long long)m * SSQ_LD, s.nch, lane) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) t[j] = wave_sum(t[j]);
    const int q = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = q == 0 ? t[r] : q == 1 ? t[4 + r] : q == 2 ? t[8 + r] : t[12 + r];
      rsv[mt][r] = rsqrtf(x * s.invn + s.eps);
    }
  }
}

// Shared epilogue.  acc[mt][j] holds D[m][n] of tile t0 + j for this lane:
// m = 16 mt + 4 (lane >> 4) + r, n = lane & 15 (hi/lo: rows m and m + 8 are
// first summed, lanes 0..31 then hold rows 0..7).
template <int MT, int TPW, int MODE>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& a, f32x4 (&acc)[MT][TPW], bool active,
                                              int t0, int lane, int wave) {
  const int TG = a.w.TG, G = a.w.G;
  const int g = active ? t0 / TG : 0;
  if (MODE == GEMV_FRAG && MT == 1 && TPW % 2 == 0 && a.fd.i8) {
    // int8 fragments of the next GEMM: tiles (t, t + 1), t even, are one
    // 32-column block, whose per-row maximum is taken over lanes 0..15 of
    // each 16-lane group (one row per group and r after the hi/lo sum).
    float rsv[1][4] = {{1.f, 1.f, 1.f, 1.f}};
    if (a.rs.ssq) gemv_row_scales<1>(a.rs, a.M, lane, rsv);
    // FP8 column scales first: a load after the first store would make the
    // following wait cover the stores too
    float fsv[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) fsv[j] = 1.f;
    if (a.w.fmt == DT_FP8 && active) {
#pragma unroll
      for (int j = 0; j < TPW; ++j)
        fsv[j] = ((const float*)a.w.scales)[(long long)min(t0 + j, g * TG + TG - 1) * 16 + (lane & 15)];
    }
    f32x4 v[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      v[j] = acc[0][j];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[j][r] += __shfl_xor(v[j][r], 32, 64);
    }
#pragma unroll
    for (int jp = 0; jp < TPW; jp += 2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = (lane >> 4) * 4 + r;
        const float rsm = rsv[0][r];
        float x[2];
        bool ok[2];
        long long col[2];
        float bm = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = t0 + jp + h;
          const int cig = (t % TG) * 16 + (lane & 15);
          ok[h] = active && cig < G && lane < 32 && m < a.M;
          col[h] = (long long)g * G + cig;
          x[h] = v[jp + h][r] * rsm * fsv[jp + h];
          if (ok[h]) bm = fmaxf(bm, fabsf(x[h]));
        }
        bm = row16_max(bm);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (ok[h]) frag_put_i8(a.fd, 0, m, (int)col[h], x[h], bm);
      }
    }
  } else if (MODE != GEMV_MARKOV) {
    float* out = a.out + (long long)blockIdx.y * a.out_split_stride;
    float rsv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) rsv[mt][r] = 1.f;
    if (a.rs.ssq) gemv_row_scales<MT>(a.rs, a.M, lane, rsv);
    // FP8 column scales before the first store (see the fragment branch)
    float fsv[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) fsv[j] = 1.f;
    if (a.w.fmt == DT_FP8 && active) {
#pragma unroll
      for (int j = 0; j < TPW; ++j)
        fsv[j] = ((const float*)a.w.scales)[(long long)min(t0 + j, g * TG + TG - 1) * 16 + (lane & 15)];
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = t0 + j;
      const int cig = (t % TG) * 16 + (lane & 15);
      const bool colok = active && cig < G;
      const long long col = (long long)g * G + cig;
      const float fs = fsv[j];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 v = acc[mt][j];
        if (a.hilo) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] += __shfl_xor(v[r], 32, 64);
        }
        if (!colok) continue;
        if (a.hilo && lane >= 32) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mt * 16 + (lane >> 4) * 4 + r;
          if (m >= a.M) continue;
          const float val = v[r] * fs * rsv[mt][r];
          if (MODE == GEMV_STORE) {
            out[(long long)m * a.out_ld + col] = val;
          } else if (MODE == GEMV_QLAT) {
            const int s = m / a.block, i = m % a.block;
            const long long qi = ((long long)s * a.rows_pad + i * a.nh + g) * a.DQ + cig;
            if (a.q_f32) ((float*)a.q)[qi] = val;
            else ((uint16_t*)a.q)[qi] = (uint16_t)f32_to_bf16_bits(val);
          } else {
            frag_put(a.fd, 0, m, (int)col, val);
          }
        }
      }
    }
  } else {
    // Markov: l = z + W2 u for M = n_seq rows; argmax over the vocabulary.
    const long long V = G;
    unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = t0 + j;
      const int col = t * 16 + (lane & 15);
      if (!active || col >= G) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = (lane >> 4) * 4 + r;
        if (m >= a.M) continue;
        const long long row = (long long)m * a.block + a.step;
        const float v = acc[0][j][r] + a.z[row * V + col];
        if (a.logits) a.logits[row * V + col] = v;
        const unsigned long long k = argmax_key(v, (uint32_t)col);
        best[r] = best[r] > k ? best[r] : k;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const unsigned long long other = shfl_xor_u64(best[r], o);
        best[r] = best[r] > other ? best[r] : other;
      }
    }
    __shared__ unsigned long long red[4][16];
    if ((lane & 15) == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][(lane >> 4) * 4 + r] = best[r];
    }
    __syncthreads();
    const int m = threadIdx.x;
    if (m < 16 && m < a.M) {
      unsigned long long k = red[0][m];
#pragma unroll
      for (int w = 1; w < 4; ++w) k = k > red[w][m] ? k : red[w][m];
      if (k) atomicMax(a.keys + ((long long)m * a.block + a.step) * KEY_SLOTS + (blockIdx.x % KEY_SLOTS), k);
    }
  }
}

// Inputs of the column-owning epilogue that do not depend on the product,
// loaded by each epilogue wave before its weight stream starts (their latency
// then hides under the stream instead of following it).  Epilogue wave r
// (r < 4) finishes rows 4 (lane >> 4) + r, i.e. rows r and r + 4, of the
// workgroup's 32 columns: lane l < 32 holds column 16 jo + (l & 15).
struct OwnPre {
  float x[2];        // RESID: residual stream, columns jo = 0, 1
  float g1[2], dw[2];  // gain of the next input, confidence weights
  float ck[2];       // row-scale chunk sums of rows r and r + 4, per lane (summed over the wave later)
  float fs[4];       // FP8 column scales of the TPW tiles
};

template <int TPW>
__device__ __forceinline__ void own_prefetch(const GemvArgs& a, int t0, int lane, int r, OwnPre& pre) {
  const int M = a.M, G = a.w.G;
  constexpr int TO = 2;
  const bool swiglu = TPW == 2 * TO;
  const int outG = swiglu ? G / 2 : G;
  const int c0 = blockIdx.x * (16 * TO);
  const int m = (lane >> 4) * 4 + r;
#pragma unroll
  for (int jo = 0; jo < TO; ++jo) {
    const int col = c0 + 16 * jo + (lane & 15);
    const bool cok = col < outG;
    pre.g1[jo] = a.g1 && cok ? a.g1[col] : 0.f;
    pre.dw[jo] = a.dotw && cok ? a.dotw[col] : 0.f;
    const bool ok = lane < 32 && m < M && cok;
    pre.x[jo] = a.epi == OWN_RESID && ok ? a.x_in[(long long)m * outG + col] : 0.f;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int mr = r + 4 * h;
    pre.ck[h] = a.rs.ssq && mr < M ? chunk_lane_sum(a.rs.ssq + (long long)mr * SSQ_LD, a.rs.nch, lane) : 0.f;
  }
#pragma unroll
  for (int j = 0; j < TPW && j < 4; ++j)
    pre.fs[j] = a.w.fmt == DT_FP8 ? ((const float*)a.w.scales)[(long long)(t0 + j + (j >= TPW / 2 ? a.tile_jump : 0)) * 16 +
                                                                 (lane & 15)]
                                  : 1.f;
}

// Epilogue of the column-owning GEMM (NW waves share TPW tiles, each wave
// summed its own k range).  The waves' accumulators meet in LDS; waves 0..3
// each finish one accumulator row r = wave of the MFMA layout: they add the
// NW partial sums in wave order (fixed: deterministic), fold the hi/lo rows,
// and write the fused outputs of rows r and r + 4 of the workgroup's 32
// columns (for SWIGLU tiles 0, 1 are the gate and 2, 3 the up columns).
// Per-row sums over the 32 columns (RMSNorm statistics, the int8 block
// maximum) are taken over each 16-lane DPP row, every lane taking part.
template <int TPW, int NW>
__device__ __forceinline__ void own_epilogue(const GemvArgs& a, const f32x4 (&acc)[TPW], int t0, int lane, int wave,
                                             const OwnPre& pre) {
  extern __shared__ __attribute__((aligned(16))) unsigned char gemv_smem[];
  float* red = (float*)gemv_smem;  // [NW][TPW][4 accumulator rows][64 lanes]: both sides lane-contiguous
#pragma unroll
  for (int j = 0; j < TPW; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[((wave * TPW + j) * 4 + q) * 64 + lane] = acc[j][q];
  __syncthreads();
  if (wave >= 4) return;
  const int r = wave;
  float v[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    v[j] = red[(j * 4 + r) * 64 + lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) v[j] += red[((w * TPW + j) * 4 + r) * 64 + lane];
    v[j] += __shfl_xor(v[j], 32, 64);
  }
  const int M = a.M, G = a.w.G;
  constexpr int TO = 2;  // output tiles: 32 columns
  static_assert(TPW == TO || TPW == 2 * TO, "plain (2 tiles) or gate/up (2 + 2 tiles)");
  const bool swiglu = TPW == 2 * TO;
  const int outG = swiglu ? G / 2 : G;      // output columns of the matrix
  const int c0 = blockIdx.x * (16 * TO);    // first output column of the workgroup
  // row scale of this lane's row from the prefetched chunk sums (the order
  // gemv_row_scales uses)
  float rs = 1.f;
  if (a.rs.ssq) {
    const float t0s = wave_sum(pre.ck[0]), t1s = wave_sum(pre.ck[1]);
    rs = rsqrtf(((lane >> 4) == 0 ? t0s : t1s) * a.rs.invn + a.rs.eps);
  }
  const int m = (lane >> 4) * 4 + r;
  const bool rowok = lane < 32 && m < M;
  float fin[TO], sq = 0.f, dt = 0.f, bm = 0.f;
  int col[TO];
  bool ok[TO];
#pragma unroll
  for (int jo = 0; jo < TO; ++jo) {
    col[jo] = c0 + 16 * jo + (lane & 15);
    ok[jo] = rowok && col[jo] < outG;
    const long long xi = (long long)m * outG + col[jo];
    float y = 0.f;
    fin[jo] = 0.f;
    if (ok[jo]) {
      if (swiglu) {
        const float g = v[jo] * pre.fs[jo] * rs, u = v[jo + TO] * pre.fs[jo + TO] * rs;
        fin[jo] = g / (1.f + __expf(-g)) * u;
      } else {
        y = v[jo] * pre.fs[jo] * rs;
        if (a.epi == OWN_RESID) y += pre.x[jo];
        a.x_out[xi] = y;
        sq += y * y;
        if (a.g1) {
          fin[jo] = pre.g1[jo] * y;
          if (a.dotw) dt += fin[jo] * pre.dw[jo];
        }
      }
    }
    bm = fmaxf(bm, fabsf(fin[jo]));
  }
  if (a.ssq_out) {
    sq = row16_sum(sq);
    if ((lane & 15) == 0 && rowok) a.ssq_out[m * SSQ_LD + blockIdx.x] = sq;
  }
  if (a.dot_out) {
    dt = row16_sum(dt);
    if ((lane & 15) == 0 && rowok) a.dot_out[m * SSQ_LD + blockIdx.x] = dt;
  }
  if (a.fd.ptr && (swiglu || a.g1)) {
    if (a.fd.i8) {
      bm = row16_max(bm);
#pragma unroll
      for (int jo = 0; jo < TO; ++jo)
        if (ok[jo]) frag_put_i8(a.fd, 0, m, col[jo], fin[jo], bm);
    } else {
#pragma unroll
      for (int jo = 0; jo < TO; ++jo)
        if (ok[jo]) frag_put(a.fd, 0, m, col[jo], fin[jo]);
    }
  }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

enum { A_GLOBAL = 0, A_ROWS_BF = 1, A_ROWS_I8 = 2, A_GLOBAL_I8 = 3, A_LDS_I8 = 4, A_LDS_BF = 5 };

// Wait until at most N vector memory operations of this wave are outstanding:
// the compiler's own builtin (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt and lgkmcnt left at their maxima), so that it knows which loads are
// complete (its own analysis would wait for every load issued before the
// direct-to-LDS copies), and a scheduling barrier, so that no use of those
// loads is moved above it.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
}

// Eight fp32 activations of row `row` from column k0 (zero outside M x K).
__device__ __forceinline__ void load_row8(const GemvArgs& a, const float* rows, int row, int k0, float (&v)[8]) {
  const int K = a.w.K;
  if (row < a.M && k0 + 8 <= K && (a.act_ld & 3) == 0) {
    const f32x4 x0 = *(const f32x4*)(rows + (long long)row * a.act_ld + k0);
    const f32x4 x1 = *(const f32x4*)(rows + (long long)row * a.act_ld + k0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = x0[e];
      v[4 + e] = x1[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = (row < a.M && k0 + e < K) ? rows[(long long)row * a.act_ld + k0 + e] : 0.f;
  }
}

// bf16-family weights (BF16 / Q8_0 / FP8 / MXFP4).
//
// AMODE selects the activation operand:
//  A_GLOBAL:  prepared bf16 fragments read from global memory (L2 resident);
//  A_ROWS_BF: the workgroup converts its k range of the fp32 activation rows
//             into bf16 fragments in LDS (hi/lo split when M <= 8);
//  A_GLOBAL_I8: Q8_0 with M <= 8: int8 hi/lo activation codes with one
//             power-of-two scale per (row, 32-block), written by the producing
//             kernel (frag_put_i8) and read from global memory with the weight
//             stream; v_mfma_i32_16x16x32_i8 on the raw weight codes;
//  A_LDS_I8:  as A_GLOBAL_I8, but the workgroup first copies its k range of
//             the fragments into LDS (direct-to-LDS loads, overlapped with
//             the first weight stage) and the k loop reads them from there:
//             the weight stream keeps the memory pipeline to itself.
//  A_ROWS_I8: Q8_0 with M <= 8: each row's slice (the workgroup's k range)
//             is quantised with one scale s to an int8 hi code and an int8
//             residual code (scale s / 256), and the int8 weight codes feed
//             v_mfma_i32_16x16x32_i8 directly: no weight decode, exact
//             integer products, one convert and one fp32 fma per output per
//             block (factor d_w); s is applied once at the end.
//  A_LDS_BF:  FP8 or BF16 weights with several m-tiles (M > 8): the workgroup's
//             lds_bf_waves(FMT) waves share one k range, so the bf16 activation
//             fragments of a chunk of LDS_BF_CK k blocks (all m-tiles) are
//             loaded once per workgroup, a share per wave, one chunk ahead into
//             registers, then written to LDS (two buffers) and read from there
//             by every wave.  Ordinary loads return in order, so the chunk's
//             wait leaves the weight prefetch in flight (direct-to-LDS copies
//             would need a full wait).
// Weight loads are issued in stages of U k steps x TPW tiles before any of
// them is consumed.
//
// NW > 0 (GEMV_OWN): the workgroup's NW waves share its tiles and split the
// reduction (wave w takes k range w); see own_epilogue.  NW == 0: the four
// waves of a workgroup own consecutive tile sets and the k range is the
// workgroup's split-K slice (blockIdx.y).
template <int FMT, int MT, int TPW, int MODE, int AMODE, int NW = 0>
__global__ __launch_bounds__(NW ? 64 * NW : (AMODE == A_LDS_BF ? 64 * lds_bf_waves(FMT) : 256)) void k_gemv_bf(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char gemv_smem[];
  // wave index made wave-uniform (scalar): tile bases and buffer resources
  // derived from it live in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = a.w.ngroups * a.w.TG;
  constexpr int WPG = AMODE == A_LDS_BF ? lds_bf_waves(FMT) : 4;  // split-K: waves per workgroup
  const int t0 = NW ? blockIdx.x * (a.tile_jump ? TPW / 2 : TPW) : (blockIdx.x * WPG + wave) * TPW;
  const bool active = t0 < T;
  // tile j of this wave is t0 + tj(j); the span of tiles its loads cover
  const int jump = NW ? a.tile_jump : 0;
  auto tj = [&](int j) { return j + (j >= TPW / 2 ? jump : 0); };
  const int span = TPW + jump;
  const int KB = a.w.KB;
  // k range: split-K slice of the workgroup, or the wave's share (waves
  // 4..7 of eight take ksteps_lo, see plan_own)
  const int hi = a.ksteps_per_split, lo = NW == 8 ? a.ksteps_lo : hi;
  const int kb0 = min(KB, NW == 8 ? (wave < 4 ? wave * hi : 4 * hi + (wave - 4) * lo)
                                  : (NW ? wave : (int)blockIdx.y) * hi);
  const int kb1 = min(KB, kb0 + (NW == 8 && wave >= 4 ? lo : hi));
  OwnPre pre{};
  if constexpr (NW > 0) {
    if (wave < 4 && active) own_prefetch<TPW>(a, t0, lane, wave, pre);
  }
  const int nkb = kb1 - kb0;
  // activation group: the workgroup's for operands staged per workgroup (its
  // tiles lie in one group), else the wave's
  const int g = (AMODE == A_ROWS_BF || AMODE == A_ROWS_I8 || AMODE == A_LDS_BF)
                    ? min(blockIdx.x * WPG * TPW, T - 1) / a.w.TG
                    : (active ? t0 / a.w.TG : 0);

  // ---------------------------------------------------------- prologue --
  bf16x8* alds = (bf16x8*)gemv_smem;            // A_ROWS_BF: [MT][nkb][64]
  long* icode = (long*)gemv_smem;               // A_ROWS_I8: [nkb][64]
  float* iscale = (float*)(gemv_smem + (size_t)nkb * 512);  // [8] row maxima, then [4][8] partials
  const float* rows = (const float*)a.act + (long long)g * a.act_gstride;
  // Activation staging (all threads, ends with a barrier).  Weight loads do
  // not depend on it, so each wave issues its first weight stage before.
  auto stage_activations = [&]() {
    if (AMODE == A_ROWS_BF) {
      for (int i = threadIdx.x; i < MT * nkb * 64; i += 256) {
        const int mt = i / (nkb * 64), rem = i - mt * nkb * 64;
        const int kbl = rem >> 6, l = rem & 63;
        const int m16 = l & 15, k0 = 32 * (kb0 + kbl) + 8 * (l >> 4);
        const int row = a.hilo ? (m16 & 7) : mt * 16 + m16;
        const bool lo = a.hilo && m16 >= 8;
        float v[8];
        load_row8(a, rows, row, k0, v);
        u32x4 o;
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t h0 = f32_to_bf16_bits(v[2 * e]), h1 = f32_to_bf16_bits(v[2 * e + 1]);
          if (lo) {
            h0 = f32_to_bf16_bits(v[2 * e] - bf16_bits_to_f32(h0));
            h1 = f32_to_bf16_bits(v[2 * e + 1] - bf16_bits_to_f32(h1));
          }
          o[e] = h0 | (h1 << 16);
        }
        alds[i] = __builtin_bit_cast(bf16x8, o);
      }
      __syncthreads();
    } else if (AMODE == A_ROWS_I8) {
      // One scale per (row, this workgroup's k range): pass 1 finds each
      // row's largest magnitude, pass 2 writes the codes.  A thread's items
      // all belong to row (tid >> 2) & 7.
      float* wpart = iscale + 8;  // [4 waves][8 rows]
      float mx = 0.f;
      for (int it = threadIdx.x; it < nkb * 32; it += 256) {
        const int q = it & 3, row = (it >> 2) & 7, kbl = it >> 5;
        float v[8];
        load_row8(a, rows, row, 32 * (kb0 + kbl) + 8 * q, v);
  #pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if ((lane & 0x23) == 0) wpart[wave * 8 + ((lane >> 2) & 7)] = mx;
      __syncthreads();
      if (threadIdx.x < 8)
        iscale[threadIdx.x] = fmaxf(fmaxf(wpart[threadIdx.x], wpart[8 + threadIdx.x]),
                                    fmaxf(wpart[16 + threadIdx.x], wpart[24 + threadIdx.x]));
      __syncthreads();
      const float rmx = iscale[(threadIdx.x >> 2) & 7];
      const float sc = rmx * (1.f / 127.f);
      const float inv = rmx > 0.f ? 127.f / rmx : 0.f;
      for (int it = threadIdx.x; it < nkb * 32; it += 256) {
        const int q = it & 3, row = (it >> 2) & 7, kbl = it >> 5;
        float v[8];
        load_row8(a, rows, row, 32 * (kb0 + kbl) + 8 * q, v);
        uint32_t hw[2] = {0u, 0u}, lw[2] = {0u, 0u};
  #pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float qh = fminf(fmaxf(__builtin_rintf(v[e] * inv), -127.f), 127.f);
          const float ql = fminf(fmaxf(__builtin_rintf((v[e] - qh * sc) * inv * 256.f), -127.f), 127.f);
          hw[e >> 2] |= ((uint32_t)(int)qh & 0xFFu) << (8 * (e & 3));
          lw[e >> 2] |= ((uint32_t)(int)ql & 0xFFu) << (8 * (e & 3));
        }
        icode[kbl * 64 + q * 16 + row] = (long)(((unsigned long long)hw[1] << 32) | hw[0]);
        icode[kbl * 64 + q * 16 + 8 + row] = (long)(((unsigned long long)lw[1] << 32) | lw[0]);
      }
      __syncthreads();
    }
  };

  f32x4 acc[MT][TPW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < TPW; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool staged = false;
  if constexpr (FMT == DT_Q8_0 && (AMODE == A_GLOBAL_I8 || AMODE == A_LDS_I8)) {
    // Every wave runs this loop (inactive waves' loads fall outside their
    // buffer resources and read zeros), so all waves reach the barrier of the
    // LDS staging.  Stage = U pairs of k blocks; pair p of tile j: 1 KiB of
    // codes, 64 B of scales.
    constexpr bool SL = AMODE == A_LDS_I8;
    constexpr int U = 8 / TPW;
    const int KP = KB >> 1, P0 = kb0 >> 1, P1 = kb1 >> 1;
    const uint32_t wbytes = active ? (uint32_t)(span * KP * 1024) : 0u;
    const __amdgpu_buffer_rsrc_t wr = buf_rsrc((const unsigned char*)a.w.codes + (long long)(active ? t0 : 0) * KP * 1024, wbytes);
    const __amdgpu_buffer_rsrc_t sr = buf_rsrc((const unsigned char*)a.w.scales + (long long)(active ? t0 : 0) * KP * 64,
                                               active ? (uint32_t)(span * KP * 64) : 0u);
    const unsigned char* abase = (const unsigned char*)a.act + (long long)g * a.act_gstride;
    const __amdgpu_buffer_rsrc_t ar = buf_rsrc(abase, (uint32_t)(KB * 520));
    const uint32_t lw = lane * 16, ls = (lane & 15) * 4, la = lane * 8;
    const uint32_t le = KB * 512 + ((lane >> 4) & 1) * 4;  // this lane's exponent word, k block 0
    const int nkb = max(kb1 - kb0, 0);
    if constexpr (SL) {
      // codes [kb0, kb1) x 512 B, then exponents [kb0, kb1) x 8 B, 1 KiB per load
      const int ncode = nkb / 2, ebytes = nkb * 8;
      for (int ch = wave; ch < ncode; ch += 4)
        __builtin_amdgcn_global_load_lds(abase + (long long)kb0 * 512 + ch * 1024 + lane * 16, gemv_smem + ch * 1024, 16, 0, 0);
      for (int ch = wave; ch * 1024 < ebytes; ch += 4)
        if (ch * 1024 + lane * 16 < ebytes)
          __builtin_amdgcn_global_load_lds(abase + (long long)KB * 512 + kb0 * 8 + ch * 1024 + lane * 16,
                                           gemv_smem + nkb * 512 + ch * 1024, 16, 0, 0);
    }
    struct Stage {
      u32x4 w[U][TPW];
      uint32_t s[U][TPW];
      long c[U][2];
      uint32_t e[U][2];
    };
    auto load_stage = [&](Stage& st, int q0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = q0 + u;
        const bool ok = p < P1;
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
          st.w[u][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
              wr, ok ? (uint32_t)((tj(j) * KP + p) * 1024) + lw : BUF_OOB, 0, BUF_NT));
          st.s[u][j] = __builtin_amdgcn_raw_buffer_load_b32(sr, ok ? (uint32_t)((tj(j) * KP + p) * 64) + ls : BUF_OOB, 0, 0);
        }
        if constexpr (!SL) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            st.c[u][h] = __builtin_bit_cast(long, __builtin_amdgcn_raw_buffer_load_b64(
                ar, ok ? (uint32_t)((2 * p + h) * 512) + la : BUF_OOB, 0, 0));
            st.e[u][h] = __builtin_amdgcn_raw_buffer_load_b32(ar, ok ? (uint32_t)((2 * p + h) * 8) + le : BUF_OOB, 0, 0);
          }
        }
      }
    };
    auto compute_stage = [&](const Stage& st, int q0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = q0 + u;
        if (p >= P1) break;
        long c[2];
        uint32_t e[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if constexpr (SL) {
            const int kl = 2 * p + h - kb0;
            c[h] = *(const long*)(gemv_smem + kl * 512 + lane * 8);
            e[h] = *(const uint32_t*)(gemv_smem + nkb * 512 + kl * 8 + ((lane >> 4) & 1) * 4);
          } else {
            c[h] = st.c[u][h];
            e[h] = st.e[u][h];
          }
        }
        int e0[4], e1[4];  // activation exponents of this lane's 4 rows
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e0[r] = (int)(signed char)(e[0] >> (8 * r));
          e1[r] = (int)(signed char)(e[1] >> (8 * r));
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
          const long B0 = (long)(((unsigned long long)st.w[u][j][1] << 32) | st.w[u][j][0]);
          const long B1 = (long)(((unsigned long long)st.w[u][j][3] << 32) | st.w[u][j][2]);
          const float d0 = fp16_bits_to_f32(st.s[u][j] & 0xFFFFu);
          const float d1 = fp16_bits_to_f32(st.s[u][j] >> 16);
          const i32x4 z = {0, 0, 0, 0};
          const i32x4 p0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(c[0], B0, z, 0, 0, 0);
          const i32x4 p1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(c[1], B1, z, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[0][j][r] += ldexpf(d0, e0[r]) * (float)p0[r] + ldexpf(d1, e1[r]) * (float)p1[r];
        }
      }
    };
    Stage sa, sb;
    const int nst = (P1 - P0 + U - 1) / U;
    load_stage(sa, P0);
    if constexpr (SL) {
      // Direct-to-LDS copies complete in no fixed order with the other
      // vector memory operations, so only a count of zero proves this wave's
      // copies landed (the first weight stage, issued after them, is waited
      // for as well); the barrier then covers every wave's copies.  The
      // builtin lets the compiler know the copies are complete.
      vm_wait<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    int q = P0, st = 0;
    for (; st + 2 < nst; st += 2, q += 2 * U) {
      load_stage(sb, q + U);
      compute_stage(sa, q);
      load_stage(sa, q + 2 * U);
      compute_stage(sb, q + U);
    }
    if (st + 1 < nst) {
      load_stage(sb, q + U);
      compute_stage(sa, q);
      compute_stage(sb, q + U);
    } else if (nst > 0) {
      compute_stage(sa, q);
    }
    staged = true;
  } else if constexpr (AMODE == A_LDS_BF) {
    static_assert((FMT == DT_FP8 || FMT == DT_BF16) && MT > 1 && NW == 0 && MODE != GEMV_MARKOV,
                  "A_LDS_BF: FP8 or BF16 weights, several m-tiles, split-K");
    constexpr int WL = FMT == DT_FP8 ? 1 : 2;  // 16-byte weight loads per tile and pair of k blocks
    constexpr int CK = LDS_BF_CK;          // k blocks per chunk
    constexpr int D = CK / 2;              // pairs of k blocks per chunk = weight pairs in flight
    constexpr int NA = (MT * CK + WPG - 1) / WPG;  // activation fragments per wave per chunk
    const int KP = KB >> 1, P0 = kb0 >> 1, P1 = kb1 >> 1;
    const __amdgpu_buffer_rsrc_t wr = buf_rsrc((const unsigned char*)a.w.codes + (long long)(active ? t0 : 0) * KP * WL * 1024,
                                               active ? (uint32_t)(span * KP * WL * 1024) : 0u);
    const __amdgpu_buffer_rsrc_t ar = buf_rsrc((const bf16x8*)a.act + (long long)g * (a.act_gstride / 8),
                                               (uint32_t)(MT * KB * 1024));
    u32x4* lds_a = (u32x4*)gemv_smem;  // [2][MT][CK][64]
    const uint32_t l16 = lane * 16;
    u32x4 areg[NA];
    auto load_chunk = [&](int c) {
#pragma unroll
      for (int n = 0; n < NA; ++n) {
        const int i = wave + WPG * n, mt = i / CK, kk = i % CK, kb = kb0 + c * CK + kk;
        const bool ok = i < MT * CK && kb < kb1;
        areg[n] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
            ar, ok ? (uint32_t)((mt * KB + kb) * 1024) + l16 : BUF_OOB, 0, 0));
      }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
      for (int n = 0; n < NA; ++n) {
        const int i = wave + WPG * n;
        if (i < MT * CK) lds_a[((buf * MT + i / CK) * CK + i % CK) * 64 + lane] = areg[n];
      }
    };
    // LDS stores complete, then the barrier (no wait on the weight loads in
    // flight, which a __syncthreads would add)
    auto lds_barrier = [&]() {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    // weights: a ring of R = 2 D pairs (two chunks), slot r holding pair
    // P0 + 2 D c2 + r during chunks 2 c2, 2 c2 + 1, refilled with the same
    // slot's pair of the next two chunks as soon as it is consumed (R pairs
    // of matrix work hide each load)
    constexpr int R = 2 * D;
    u32x4 wring[R][TPW][WL];
    auto load_w = [&](u32x4 (&w)[TPW][WL], int p) {
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int h = 0; h < WL; ++h)  // FP8: one 1 KiB chunk per pair; BF16: one per k block
          w[j][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
              wr, p < P1 ? (uint32_t)(((tj(j) * KP + p) * WL + h) * 1024) + l16 : BUF_OOB, 0, BUF_NT));
    };
    const int nch = (kb1 - kb0 + CK - 1) / CK;
    if (nch > 0) {
      load_chunk(0);
#pragma unroll
      for (int r = 0; r < R; ++r) load_w(wring[r], P0 + r);
      store_chunk(0);
    }
    lds_barrier();
    for (int c2 = 0; 2 * c2 < nch; ++c2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // chunk c = 2 c2 + h in buffer h
        const int c = 2 * c2 + h;
        if (c >= nch) break;
        if (c + 1 < nch) load_chunk(c + 1);
#pragma unroll
        for (int pp = 0; pp < D; ++pp) {
          const int r = h * D + pp;
          bf16x8 B0[TPW], B1[TPW];
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            if constexpr (FMT == DT_FP8) {
              B0[j] = fp8x8_to_bf16x8(wring[r][j][0][0], wring[r][j][0][1]);
              B1[j] = fp8x8_to_bf16x8(wring[r][j][0][2], wring[r][j][0][3]);
            } else {
              B0[j] = __builtin_bit_cast(bf16x8, wring[r][j][0]);
              B1[j] = __builtin_bit_cast(bf16x8, wring[r][j][WL - 1]);
            }
          }
          load_w(wring[r], P0 + R * (c2 + 1) + r);  // out of range: zeros, no memory access
          __builtin_amdgcn_sched_barrier(0);  // issue the refill here, a whole ring ahead of its use
          // pairs past the k range: zero weights times zero fragments
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const bf16x8 A0 = __builtin_bit_cast(bf16x8, lds_a[((h * MT + mt) * CK + 2 * pp) * 64 + lane]);
            const bf16x8 A1 = __builtin_bit_cast(bf16x8, lds_a[((h * MT + mt) * CK + 2 * pp + 1) * 64 + lane]);
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
              acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B0[j], acc[mt][j], 0, 0, 0);
              acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B1[j], acc[mt][j], 0, 0, 0);
            }
          }
        }
        if (c + 1 < nch) {
          // every wave finished chunk c - 1 (the last barrier), whose buffer
          // takes chunk c + 1
          store_chunk(h ^ 1);
          lds_barrier();
        }
      }
    }
    staged = true;
  } else if (active) {
    const bf16x8* afrag = (const bf16x8*)a.act + (long long)g * (a.act_gstride / 8);
    const __bf16* gsrc = nullptr;
    if (MODE == GEMV_MARKOV) {
      const int m = lane & 15;
      const int tp = m < a.M ? markov_prev(a, m) : -1;
      if (tp >= 0 && tp < a.w.G) gsrc = (const __bf16*)a.act + (long long)tp * a.gather_ld + 8 * (lane >> 4);
    }
    auto load_a = [&](int mt, int kb) -> bf16x8 {
      if (MODE == GEMV_MARKOV) {
        if (!gsrc) return bf16x8{};
        return *(const bf16x8*)(gsrc + 32 * kb);
      }
      if (AMODE == A_ROWS_BF) return alds[(mt * nkb + (kb - kb0)) * 64 + lane];
      return afrag[((long long)mt * KB + kb) * 64 + lane];
    };

    // Weight stream, software pipelined: the loads of stage s+1 are issued
    // before stage s is consumed, so a wave always has loads in flight.
    if constexpr (FMT == DT_MXFP4) {
      // E2M1 codes decoded to bf16 with the block's E8M0 scale folded into
      // the conversion (exact), then the bf16 MFMA.  One 1 KiB chunk per
      // (tile, quad of k blocks) and one scale dword per (tile, quad, row).
      // Split-K ranges are whole quads (KB % 4 == 0, unit 4).
      const int KQ = KB >> 2, q1 = kb1 >> 2;
      const __amdgpu_buffer_rsrc_t wr = buf_rsrc((const unsigned char*)a.w.codes + (long long)t0 * KQ * 1024,
                                                 (uint32_t)(span * KQ * 1024));
      const __amdgpu_buffer_rsrc_t sr = buf_rsrc((const unsigned char*)a.w.scales + (long long)t0 * KQ * 64,
                                                 (uint32_t)(span * KQ * 64));
      const uint32_t l16 = lane * 16, ls = (lane & 15) * 4;
      auto scale = [](uint32_t w, int i) {
        return i == 0 ? e8m0_f32<0>(w) : i == 1 ? e8m0_f32<1>(w) : i == 2 ? e8m0_f32<2>(w) : e8m0_f32<3>(w);
      };
      if constexpr (MT == 1 && AMODE == A_GLOBAL && MODE != GEMV_MARKOV) {
        // prepared fragments: a quad's four activation fragments are loaded
        // with its weights, stage by stage (U quads x TPW tiles; one quad per
        // stage measured as fast as two or four, with fewer registers)
        constexpr int U = 1;
        const __amdgpu_buffer_rsrc_t ar = buf_rsrc(afrag, (uint32_t)(KB * 1024));
        struct Stage {
          u32x4 w[U][TPW];
          uint32_t s[U][TPW];
          u32x4 x[U][4];
        };
        auto load_stage = [&](Stage& st, int p0) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int p = p0 + u;
            const bool ok = p < q1;
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
              st.w[u][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                  wr, ok ? (uint32_t)((tj(j) * KQ + p) * 1024) + l16 : BUF_OOB, 0, BUF_NT));
              st.s[u][j] = __builtin_amdgcn_raw_buffer_load_b32(sr, ok ? (uint32_t)((tj(j) * KQ + p) * 64) + ls : BUF_OOB,
                                                                0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
              st.x[u][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                  ar, ok ? (uint32_t)((4 * p + i) * 1024) + l16 : BUF_OOB, 0, 0));
          }
        };
        auto compute_stage = [&](const Stage& st, int p0) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (p0 + u >= q1) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bf16x8 A = __builtin_bit_cast(bf16x8, st.x[u][i]);
#pragma unroll
              for (int j = 0; j < TPW; ++j)
                acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    A, fp4x8_to_bf16x8(st.w[u][j][i], scale(st.s[u][j], i)), acc[0][j], 0, 0, 0);
            }
          }
        };
        Stage sa, sb;
        const int p0 = kb0 >> 2;
        const int nst = (q1 - p0 + U - 1) / U;
        load_stage(sa, p0);
        int p = p0, st = 0;
        for (; st + 2 < nst; st += 2, p += 2 * U) {
          load_stage(sb, p + U);
          compute_stage(sa, p);
          load_stage(sa, p + 2 * U);
          compute_stage(sb, p + U);
        }
        if (st + 1 < nst) {
          load_stage(sb, p + U);
          compute_stage(sa, p);
          compute_stage(sb, p + U);
        } else if (nst > 0) {
          compute_stage(sa, p);
        }
      } else {
        // several m-tiles, or activations staged in LDS: weights by quad,
        // activations read as consumed
        stage_activations();
        staged = true;
        for (int p = kb0 >> 2; p < q1; ++p) {
          u32x4 w[TPW];
          uint32_t sc[TPW];
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            w[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                wr, (uint32_t)((j * KQ + p) * 1024) + l16, 0, BUF_NT));
            sc[j] = __builtin_amdgcn_raw_buffer_load_b32(sr, (uint32_t)((j * KQ + p) * 64) + ls, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bf16x8 A[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) A[mt] = load_a(mt, 4 * p + i);
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
              const bf16x8 B = fp4x8_to_bf16x8(w[j][i], scale(sc[j], i));
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt], B, acc[mt][j], 0, 0, 0);
            }
          }
        }
      }
    } else if constexpr (FMT == DT_FP8 && MT == 1 && AMODE == A_GLOBAL && MODE != GEMV_MARKOV) {
      // FP8 weights, prepared fragments: a 1 KiB chunk holds a pair of k
      // blocks of a tile; its two activation fragments are loaded with it,
      // stage by stage (U pairs x TPW tiles, 8 KiB of weights per stage).
      // The per-row scales are applied in the epilogue.
      constexpr int U = 8 / TPW;
      const int KP = KB >> 1, p1 = kb1 >> 1;
      const __amdgpu_buffer_rsrc_t wr = buf_rsrc((const unsigned char*)a.w.codes + (long long)t0 * KP * 1024,
                                                 (uint32_t)(span * KP * 1024));
      const __amdgpu_buffer_rsrc_t ar = buf_rsrc(afrag, (uint32_t)(KB * 1024));
      const uint32_t l16 = lane * 16;
      struct Stage {
        u32x4 w[U][TPW];
        u32x4 x[U][2];
      };
      auto load_stage = [&](Stage& st, int q0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int p = q0 + u;
          const bool ok = p < p1;
#pragma unroll
          for (int j = 0; j < TPW; ++j)
            st.w[u][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                wr, ok ? (uint32_t)((tj(j) * KP + p) * 1024) + l16 : BUF_OOB, 0, BUF_NT));
#pragma unroll
          for (int h = 0; h < 2; ++h)
            st.x[u][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                ar, ok ? (uint32_t)((2 * p + h) * 1024) + l16 : BUF_OOB, 0, 0));
        }
      };
      auto compute_stage = [&](const Stage& st, int q0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (q0 + u >= p1) break;
          const bf16x8 A0 = __builtin_bit_cast(bf16x8, st.x[u][0]), A1 = __builtin_bit_cast(bf16x8, st.x[u][1]);
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, fp8x8_to_bf16x8(st.w[u][j][0], st.w[u][j][1]),
                                                                acc[0][j], 0, 0, 0);
            acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, fp8x8_to_bf16x8(st.w[u][j][2], st.w[u][j][3]),
                                                                acc[0][j], 0, 0, 0);
          }
        }
      };
      Stage sa, sb;
      const int q0 = kb0 >> 1;
      const int nst = (p1 - q0 + U - 1) / U;
      load_stage(sa, q0);
      int q = q0, st = 0;
      for (; st + 2 < nst; st += 2, q += 2 * U) {
        load_stage(sb, q + U);
        compute_stage(sa, q);
        load_stage(sa, q + 2 * U);
        compute_stage(sb, q + U);
      }
      if (st + 1 < nst) {
        load_stage(sb, q + U);
        compute_stage(sa, q);
        compute_stage(sb, q + U);
      } else if (nst > 0) {
        compute_stage(sa, q);
      }
    } else if constexpr (FMT == DT_BF16 && AMODE == A_GLOBAL && MODE != GEMV_MARKOV) {
      // bf16 weights, prepared bf16 activation fragments: both loaded per
      // stage of U k blocks (tile j, k block kb: 1 KiB of weights; m-tile mt:
      // 1 KiB of activations).
      constexpr int U = (MT == 1 ? 8 : 4) / TPW;
      const __amdgpu_buffer_rsrc_t wr = buf_rsrc((const unsigned char*)a.w.codes + (long long)t0 * KB * 1024,
                                                 (uint32_t)(span * KB * 1024));
      const __amdgpu_buffer_rsrc_t ar = buf_rsrc(afrag, (uint32_t)(MT * KB * 1024));
      const uint32_t l16 = lane * 16;
      struct Stage {
        u32x4 w[U][TPW];
        u32x4 x[U][MT];
      };
      auto load_stage = [&](Stage& st, int k0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int kb = k0 + u;
          const bool ok = kb < kb1;
#pragma unroll
          for (int j = 0; j < TPW; ++j)
            st.w[u][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                wr, ok ? (uint32_t)((tj(j) * KB + kb) * 1024) + l16 : BUF_OOB, 0, BUF_NT));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            st.x[u][mt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                ar, ok ? (uint32_t)((mt * KB + kb) * 1024) + l16 : BUF_OOB, 0, 0));
        }
      };
      auto compute_stage = [&](const Stage& st, int k0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (k0 + u >= kb1) break;
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            const bf16x8 B = __builtin_bit_cast(bf16x8, st.w[u][j]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, st.x[u][mt]), B,
                                                                    acc[mt][j], 0, 0, 0);
          }
        }
      };
      Stage sa, sb;
      const int nst = (kb1 - kb0 + U - 1) / U;
      load_stage(sa, kb0);
      int kb = kb0, st = 0;
      for (; st + 2 < nst; st += 2, kb += 2 * U) {
        load_stage(sb, kb + U);
        compute_stage(sa, kb);
        load_stage(sa, kb + 2 * U);
        compute_stage(sb, kb + U);
      }
      if (st + 1 < nst) {
        load_stage(sb, kb + U);
        compute_stage(sa, kb);
        compute_stage(sb, kb + U);
      } else {
        compute_stage(sa, kb);
      }
    } else if (FMT == DT_BF16) {
      constexpr int U = (MT == 1 ? 8 : 4) / TPW;  // k blocks per stage
      const u32x4* wp = (const u32x4*)a.w.codes + (long long)t0 * KB * 64 + lane;
      auto load_stage = [&](u32x4 (&wr)[U][TPW], int kb) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (kb + u < kb1)
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
              // W2 is re-read by every Markov step: keep it cacheable
              const u32x4* src = wp + ((long long)j * KB + kb + u) * 64;
              wr[u][j] = MODE == GEMV_MARKOV ? *src : ntload(src);
            }
      };
      auto compute_stage = [&](const u32x4 (&wr)[U][TPW], int kb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (kb + u >= kb1) break;
          bf16x8 A[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) A[mt] = load_a(mt, kb + u);
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            const bf16x8 B = __builtin_bit_cast(bf16x8, wr[u][j]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt], B, acc[mt][j], 0, 0, 0);
          }
        }
      };
      u32x4 wa[U][TPW], wb[U][TPW];
      load_stage(wa, kb0);
      stage_activations();
      staged = true;
      for (int kb = kb0; kb < kb1; kb += 2 * U) {
        if (kb + U < kb1) load_stage(wb, kb + U);
        compute_stage(wa, kb);
        if (kb + U >= kb1) break;
        if (kb + 2 * U < kb1) load_stage(wa, kb + 2 * U);
        compute_stage(wb, kb + U);
      }
    } else {
      constexpr int U = (MT == 1 ? 8 : 4) / TPW;  // pairs of k blocks per stage
      const int KP = KB >> 1;
      const u32x4* wp = (const u32x4*)a.w.codes + (long long)t0 * KP * 64 + lane;
      const uint32_t* sp = (const uint32_t*)a.w.scales + (long long)t0 * KP * 16 + (lane & 15);
      auto load_stage = [&](u32x4 (&wr)[U][TPW], uint32_t (&sc)[U][TPW], int kb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (kb + 2 * u >= kb1) break;
          const int p = (kb >> 1) + u;
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            wr[u][j] = ntload(wp + ((long long)j * KP + p) * 64);
            if (FMT == DT_Q8_0) sc[u][j] = sp[((long long)j * KP + p) * 16];
          }
        }
      };
      auto compute_stage = [&](const u32x4 (&wr)[U][TPW], const uint32_t (&sc)[U][TPW], int kb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int k2 = kb + 2 * u;
          if (k2 >= kb1) break;
          if (AMODE == A_ROWS_I8) {
            const int kl = k2 - kb0;
            const long A0 = icode[kl * 64 + lane], A1 = icode[(kl + 1) * 64 + lane];
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
              const long B0 = (long)(((unsigned long long)wr[u][j][1] << 32) | wr[u][j][0]);
              const long B1 = (long)(((unsigned long long)wr[u][j][3] << 32) | wr[u][j][2]);
              const float d0 = fp16_bits_to_f32(sc[u][j] & 0xFFFFu);
              const float d1 = fp16_bits_to_f32(sc[u][j] >> 16);
              const i32x4 z = {0, 0, 0, 0};
              const i32x4 p0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(A0, B0, z, 0, 0, 0);
              const i32x4 p1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(A1, B1, z, 0, 0, 0);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[0][j][r] += d0 * (float)p0[r] + d1 * (float)p1[r];
            }
            continue;
          }
          bf16x8 A0[MT], A1[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            A0[mt] = load_a(mt, k2);
            A1[mt] = load_a(mt, k2 + 1);
          }
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            if (FMT == DT_Q8_0) {
              const bf16x8 B0 = i8x8_to_bf16x8(wr[u][j][0], wr[u][j][1]);
              const bf16x8 B1 = i8x8_to_bf16x8(wr[u][j][2], wr[u][j][3]);
              const float d0 = fp16_bits_to_f32(sc[u][j] & 0xFFFFu);
              const float d1 = fp16_bits_to_f32(sc[u][j] >> 16);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f32x4 p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[mt], B0, z, 0, 0, 0);
                const f32x4 p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[mt], B1, z, 0, 0, 0);
                acc[mt][j] += d0 * p0 + d1 * p1;
              }
            } else {
              const bf16x8 B0 = fp8x8_to_bf16x8(wr[u][j][0], wr[u][j][1]);
              const bf16x8 B1 = fp8x8_to_bf16x8(wr[u][j][2], wr[u][j][3]);
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) {
                acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[mt], B0, acc[mt][j], 0, 0, 0);
                acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[mt], B1, acc[mt][j], 0, 0, 0);
              }
            }
          }
        }
      };
      u32x4 wa[U][TPW], wb[U][TPW];
      uint32_t sa[U][TPW], sb[U][TPW];
      load_stage(wa, sa, kb0);
      stage_activations();
      staged = true;
      for (int kb = kb0; kb < kb1; kb += 4 * U) {
        if (kb + 2 * U < kb1) load_stage(wb, sb, kb + 2 * U);
        compute_stage(wa, sa, kb);
        if (kb + 2 * U >= kb1) break;
        if (kb + 4 * U < kb1) load_stage(wa, sa, kb + 4 * U);
        compute_stage(wb, sb, kb + 2 * U);
      }
    }
  }
  if (!staged) stage_activations();  // inactive waves still join the barrier
  if ((AMODE == A_GLOBAL_I8 || AMODE == A_LDS_I8) && lane >= 32) {
    // rows 8..15 carry the residual codes (scale 2^e / 256)
#pragma unroll
    for (int j = 0; j < TPW; ++j) acc[0][j] *= (1.f / 256.f);
  }
  if (AMODE == A_ROWS_I8) {
    // code units -> values: row scale max/127, residual rows (lanes 32..63) / 256
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float f = iscale[((lane >> 4) & 1) * 4 + r] * (lane >= 32 ? 1.f / (127.f * 256.f) : 1.f / 127.f);
#pragma unroll
      for (int j = 0; j < TPW; ++j) acc[0][j][r] *= f;
    }
  }
  if constexpr (NW > 0) {
    static_assert(MT == 1, "column-owning GEMMs take M <= 8 rows (hi/lo)");
    own_epilogue<TPW, NW>(a, acc[0], t0, lane, wave, pre);
  } else {
    gemv_epilogue<MT, TPW, MODE>(a, acc, active, t0, lane, wave);
  }
}

// F32 weights on v_mfma_f32_16x16x4_f32: four MFMAs per 16-wide k group.
template <int MT, int TPW, int MODE>
__global__ __launch_bounds__(256) void k_gemv_f32(GemvArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.w.ngroups * a.w.TG;
  const int t0 = (blockIdx.x * 4 + wave) * TPW;
  const bool active = t0 < T;
  const int KG = a.w.Kp >> 4;
  const int g0 = blockIdx.y * a.ksteps_per_split;
  const int g1 = min(KG, g0 + a.ksteps_per_split);

  f32x4 acc[MT][TPW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < TPW; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (active) {
    const int g = t0 / a.w.TG;
    const f32x4* afrag = (const f32x4*)a.act + (long long)g * (a.act_gstride / 4);
    const float* gsrc = nullptr;
    if (MODE == GEMV_MARKOV) {
      const int m = lane & 15;
      const int tp = m < a.M ? markov_prev(a, m) : -1;
      if (tp >= 0 && tp < a.w.G) gsrc = (const float*)a.act + (long long)tp * a.gather_ld + 4 * (lane >> 4);
    }
    const f32x4* wp = (const f32x4*)a.w.codes + (long long)t0 * KG * 64 + lane;
    for (int gk = g0; gk < g1; ++gk) {
      f32x4 W[TPW];
#pragma unroll
      for (int j = 0; j < TPW; ++j) W[j] = ntload(wp + ((long long)j * KG + gk) * 64);
      f32x4 A[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (MODE == GEMV_MARKOV) A[mt] = gsrc ? *(const f32x4*)(gsrc + 16 * gk) : f32x4{0.f, 0.f, 0.f, 0.f};
        else A[mt] = afrag[((long long)mt * KG + gk) * 64 + lane];
      }
#pragma unroll
      for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[mt][i], W[j][i], acc[mt][j], 0, 0, 0);
    }
  }
  gemv_epilogue<MT, TPW, MODE>(a, acc, active, t0, lane, wave);
}

// LDS bytes of the activation staging of one workgroup.
inline size_t gemv_lds_bytes(const GemvPlan& p) {
  if (p.amode == A_ROWS_BF) return (size_t)p.MT * p.ksteps_per_split * 64 * 16;
  if (p.amode == A_ROWS_I8) return (size_t)p.ksteps_per_split * 512 + 256;
  if (p.amode == A_GLOBAL_I8) return (size_t)p.ksteps_per_split * 520;  // the A_LDS_I8 copy
  if (p.amode == A_LDS_BF) return (size_t)2 * p.MT * LDS_BF_CK * 1024;
  return 0;
}

// int8 fragments staged in LDS when a workgroup's k range fits 32 KiB (the
// fc GEMM's 64 KiB k range measured slower staged than read with the weights)
inline bool gemv_lds_i8(const GemvPlan& p) { return p.ksteps_per_split * 520 <= 32768; }

template <int FMT, int MT, int TPW, int MODE>
hipError_t go(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  dim3 grid(p.grid_x, p.S), block(p.amode == A_LDS_BF ? 64 * lds_bf_waves(FMT) : 256);
  const size_t lds = gemv_lds_bytes(p);
  if (FMT == DT_F32) {
    hipLaunchKernelGGL((k_gemv_f32<MT, TPW, MODE>), grid, block, 0, st, a);
  } else if (p.amode == A_ROWS_BF) {
    hipLaunchKernelGGL((k_gemv_bf<FMT, MT, TPW, MODE, A_ROWS_BF>), grid, block, lds, st, a);
  } else if (FMT == DT_Q8_0 && MT == 1 && MODE != GEMV_MARKOV && p.amode == A_ROWS_I8) {
    hipLaunchKernelGGL((k_gemv_bf<FMT, 1, TPW, MODE, A_ROWS_I8>), grid, block, lds, st, a);
  } else if (FMT == DT_Q8_0 && MT == 1 && MODE != GEMV_MARKOV && p.amode == A_GLOBAL_I8) {
    if (gemv_lds_i8(p))
      hipLaunchKernelGGL((k_gemv_bf<FMT, 1, TPW, MODE, A_LDS_I8>), grid, block, lds, st, a);
    else
      hipLaunchKernelGGL((k_gemv_bf<FMT, 1, TPW, MODE, A_GLOBAL_I8>), grid, block, 0, st, a);
  } else if (p.amode == A_LDS_BF) {
    if constexpr ((FMT == DT_FP8 || FMT == DT_BF16) && MT > 1 && MODE != GEMV_MARKOV)
      hipLaunchKernelGGL((k_gemv_bf<FMT, MT, TPW, MODE, A_LDS_BF>), grid, block, lds, st, a);
    else
      return hipErrorInvalidValue;
  } else if (p.amode == A_GLOBAL) {
    hipLaunchKernelGGL((k_gemv_bf<FMT, MT, TPW, MODE, A_GLOBAL>), grid, block, 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT, int MODE>
hipError_t dispatch_out(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  if (p.MT == 1) {
    if (p.TPW == 4) return go<FMT, 1, 4, MODE>(a, p, st);
    if (p.TPW == 2) return go<FMT, 1, 2, MODE>(a, p, st);
    return go<FMT, 1, 1, MODE>(a, p, st);
  }
  if ((FMT == DT_FP8 || FMT == DT_BF16) && p.TPW == 2) {
    switch (p.MT) {
      case 2: return go<FMT, 2, 2, MODE>(a, p, st);
      case 3: return go<FMT, 3, 2, MODE>(a, p, st);
      case 4: return go<FMT, 4, 2, MODE>(a, p, st);
      case 5: return go<FMT, 5, 2, MODE>(a, p, st);
      case 6: return go<FMT, 6, 2, MODE>(a, p, st);
      case 7: return go<FMT, 7, 2, MODE>(a, p, st);
    }
    return hipErrorInvalidValue;
  }
  if (p.TPW == 4) {
    switch (p.MT) {
      case 2: return go<FMT, 2, 4, MODE>(a, p, st);
      case 3: return go<FMT, 3, 4, MODE>(a, p, st);
      case 4: return go<FMT, 4, 4, MODE>(a, p, st);
      case 5: return go<FMT, 5, 4, MODE>(a, p, st);
      case 6: return go<FMT, 6, 4, MODE>(a, p, st);
      case 7: return go<FMT, 7, 4, MODE>(a, p, st);
    }
    return hipErrorInvalidValue;
  }
  switch (p.MT) {
    case 2: return go<FMT, 2, 1, MODE>(a, p, st);
    case 3: return go<FMT, 3, 1, MODE>(a, p, st);
    case 4: return go<FMT, 4, 1, MODE>(a, p, st);
    case 5: return go<FMT, 5, 1, MODE>(a, p, st);
    case 6: return go<FMT, 6, 1, MODE>(a, p, st);
    case 7: return go<FMT, 7, 1, MODE>(a, p, st);
    case 8: return go<FMT, 8, 1, MODE>(a, p, st);
  }
  return hipErrorInvalidValue;
}

template <int FMT>
hipError_t dispatch_markov(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  if (p.MT != 1) return hipErrorInvalidValue;
  if (p.TPW == 4) return go<FMT, 1, 4, GEMV_MARKOV>(a, p, st);
  if (p.TPW == 2) return go<FMT, 1, 2, GEMV_MARKOV>(a, p, st);
  return go<FMT, 1, 1, GEMV_MARKOV>(a, p, st);
}

// Column-owning launches: one workgroup of 64 nw threads per 32 output
// columns; weights in bf16 fragments order (BF16 / FP8 / MXFP4 with bf16
// hi/lo activation fragments) or Q8_0 on int8 activation fragments.
template <int FMT, int TPW, int NW>
hipError_t go_own(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  const size_t lds = (size_t)NW * TPW * 64 * 16;
  if constexpr (FMT == DT_Q8_0)
    hipLaunchKernelGGL((k_gemv_bf<FMT, 1, TPW, GEMV_OWN, A_GLOBAL_I8, NW>), dim3(p.grid_x), dim3(64 * NW), lds, st, a);
  else
    hipLaunchKernelGGL((k_gemv_bf<FMT, 1, TPW, GEMV_OWN, A_GLOBAL, NW>), dim3(p.grid_x), dim3(64 * NW), lds, st, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t dispatch_own(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  if constexpr (FMT == DT_F32) {
    return hipErrorInvalidValue;
  } else {
    if (p.MT != 1 || p.S != 1 || (FMT == DT_Q8_0) != (p.amode == A_GLOBAL_I8)) return hipErrorInvalidValue;
    if (p.TPW == 2 && p.nw == 8) return go_own<FMT, 2, 8>(a, p, st);
    if (p.TPW == 2 && p.nw == 4) return go_own<FMT, 2, 4>(a, p, st);
    if (p.TPW == 4 && p.nw == 8) return go_own<FMT, 4, 8>(a, p, st);
    if (p.TPW == 4 && p.nw == 4) return go_own<FMT, 4, 4>(a, p, st);
    return hipErrorInvalidValue;
  }
}

template <int FMT>
hipError_t dispatch_fmt(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st) {
  switch (mode) {
    case GEMV_OWN: return dispatch_own<FMT>(a, p, st);
    case GEMV_STORE: return dispatch_out<FMT, GEMV_STORE>(a, p, st);
    case GEMV_QLAT: return dispatch_out<FMT, GEMV_QLAT>(a, p, st);
    case GEMV_FRAG: return dispatch_out<FMT, GEMV_FRAG>(a, p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

}  // namespace dspark
