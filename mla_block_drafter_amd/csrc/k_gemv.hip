// Skinny GEMM for the draft pass: M = 7 activation rows per sequence against a
// weight matrix streamed once from HBM (weight-only BF16 / Q8_0 / FP8 / F32).
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
#include "kernels.h"

namespace dspark {

namespace {

template <typename T>
__device__ __forceinline__ T ntload(const T* p) {
  return __builtin_nontemporal_load(p);
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

// Shared epilogue.  acc[mt][j] holds D[m][n] of tile t0 + j for this lane:
// m = 16 mt + 4 (lane >> 4) + r, n = lane & 15.
template <int MT, int TPW, int MODE>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& a, f32x4 (&acc)[MT][TPW], bool active,
                                              int t0, int lane, int wave) {
  const int TG = a.w.TG, G = a.w.G;
  const int g = active ? t0 / TG : 0;
  if (MODE == GEMV_STORE) {
    float* out = a.out + (long long)blockIdx.y * a.out_split_stride;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = t0 + j;
      const int cig = (t % TG) * 16 + (lane & 15);
      const bool colok = active && cig < G;
      const long long col = (long long)g * G + cig;
      float fs = 1.0f;
      if (a.w.fmt == DT_FP8 && colok) fs = ((const float*)a.w.scales)[(long long)t * 16 + (lane & 15)];
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
          if (m < a.M) out[(long long)m * a.out_ld + col] = v[r] * fs;
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

// bf16-family weights (BF16 / Q8_0 / FP8) on v_mfma_f32_16x16x32_bf16.
template <int FMT, int MT, int TPW, int MODE>
__global__ __launch_bounds__(256) void k_gemv_bf(GemvArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.w.ngroups * a.w.TG;
  const int t0 = (blockIdx.x * 4 + wave) * TPW;
  const bool active = t0 < T;
  const int KB = a.w.KB;
  const int kb0 = blockIdx.y * a.ksteps_per_split;
  const int kb1 = min(KB, kb0 + a.ksteps_per_split);

  f32x4 acc[MT][TPW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < TPW; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (active) {
    const int g = t0 / a.w.TG;
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
      return afrag[((long long)mt * KB + kb) * 64 + lane];
    };

    if (FMT == DT_BF16) {
      const u32x4* wp = (const u32x4*)a.w.codes + (long long)t0 * KB * 64 + lane;
      for (int kb = kb0; kb < kb1; ++kb) {
        u32x4 wr[TPW];
#pragma unroll
        for (int j = 0; j < TPW; ++j) wr[j] = ntload(wp + ((long long)j * KB + kb) * 64);
        bf16x8 A[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) A[mt] = load_a(mt, kb);
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
          const bf16x8 B = __builtin_bit_cast(bf16x8, wr[j]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt], B, acc[mt][j], 0, 0, 0);
        }
      }
    } else {
      const int KP = KB >> 1;
      const u32x4* wp = (const u32x4*)a.w.codes + (long long)t0 * KP * 64 + lane;
      const uint32_t* sp = (const uint32_t*)a.w.scales + (long long)t0 * KP * 16 + (lane & 15);
      for (int kb = kb0; kb < kb1; kb += 2) {
        const int p = kb >> 1;
        u32x4 wr[TPW];
        uint32_t sc[TPW];
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
          wr[j] = ntload(wp + ((long long)j * KP + p) * 64);
          if (FMT == DT_Q8_0) sc[j] = sp[((long long)j * KP + p) * 16];
        }
        bf16x8 A0[MT], A1[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          A0[mt] = load_a(mt, kb);
          A1[mt] = load_a(mt, kb + 1);
        }
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
          bf16x8 B0, B1;
          if (FMT == DT_Q8_0) {
            B0 = i8x8_to_bf16x8(wr[j][0], wr[j][1]);
            B1 = i8x8_to_bf16x8(wr[j][2], wr[j][3]);
            const float d0 = fp16_bits_to_f32(sc[j] & 0xFFFFu);
            const float d1 = fp16_bits_to_f32(sc[j] >> 16);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              const f32x4 z = {0.f, 0.f, 0.f, 0.f};
              const f32x4 p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[mt], B0, z, 0, 0, 0);
              const f32x4 p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[mt], B1, z, 0, 0, 0);
              acc[mt][j] += d0 * p0 + d1 * p1;
            }
          } else {
            B0 = fp8x8_to_bf16x8(wr[j][0], wr[j][1]);
            B1 = fp8x8_to_bf16x8(wr[j][2], wr[j][3]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[mt], B0, acc[mt][j], 0, 0, 0);
              acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[mt], B1, acc[mt][j], 0, 0, 0);
            }
          }
        }
      }
    }
  }
  gemv_epilogue<MT, TPW, MODE>(a, acc, active, t0, lane, wave);
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

template <int FMT, int MT, int TPW, int MODE>
hipError_t go(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  dim3 grid(p.grid_x, p.S), block(256);
  if (FMT == DT_F32)
    hipLaunchKernelGGL((k_gemv_f32<MT, TPW, MODE>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((k_gemv_bf<FMT, MT, TPW, MODE>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t dispatch_store(const GemvArgs& a, const GemvPlan& p, hipStream_t st) {
  if (p.MT == 1) {
    if (p.TPW == 4) return go<FMT, 1, 4, GEMV_STORE>(a, p, st);
    if (p.TPW == 2) return go<FMT, 1, 2, GEMV_STORE>(a, p, st);
    return go<FMT, 1, 1, GEMV_STORE>(a, p, st);
  }
  switch (p.MT) {
    case 2: return go<FMT, 2, 1, GEMV_STORE>(a, p, st);
    case 3: return go<FMT, 3, 1, GEMV_STORE>(a, p, st);
    case 4: return go<FMT, 4, 1, GEMV_STORE>(a, p, st);
    case 5: return go<FMT, 5, 1, GEMV_STORE>(a, p, st);
    case 6: return go<FMT, 6, 1, GEMV_STORE>(a, p, st);
    case 7: return go<FMT, 7, 1, GEMV_STORE>(a, p, st);
    case 8: return go<FMT, 8, 1, GEMV_STORE>(a, p, st);
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

}  // namespace

GemvPlan plan_gemv(const PackedMat& w, int M, bool markov) {
  GemvPlan p{};
  const bool f32 = w.fmt == DT_F32;
  p.hilo = (!f32 && !markov && M <= 8) ? 1 : 0;
  p.MT = p.hilo ? 1 : (M + 15) / 16;
  const int T = w.ngroups * w.TG;
  p.TPW = 1;
  if (p.MT == 1) {
    if (T >= 4096 && w.TG % 4 == 0) p.TPW = 4;
    else if (T >= 1024 && w.TG % 2 == 0) p.TPW = 2;
  }
  const int waves = T / p.TPW;
  p.grid_x = (waves + 3) / 4;
  const int ksteps = f32 ? (w.Kp >> 4) : w.KB;
  const int unit = (w.fmt == DT_Q8_0 || w.fmt == DT_FP8) ? 2 : 1;
  int S = 1;
  if (!markov) {
    const int target = 2048;  // waves in flight: 8 per CU
    while ((long long)waves * S < target && ksteps / (S * 2) >= 8) S *= 2;
  }
  int per = (ksteps + S - 1) / S;
  per = (per + unit - 1) / unit * unit;
  p.ksteps_per_split = per;
  p.S = (ksteps + per - 1) / per;
  return p;
}

hipError_t launch_gemv(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st) {
  if (mode == GEMV_MARKOV) {
    if (a.w.fmt == DT_BF16) return dispatch_markov<DT_BF16>(a, p, st);
    if (a.w.fmt == DT_F32) return dispatch_markov<DT_F32>(a, p, st);
    return hipErrorInvalidValue;
  }
  switch (a.w.fmt) {
    case DT_BF16: return dispatch_store<DT_BF16>(a, p, st);
    case DT_Q8_0: return dispatch_store<DT_Q8_0>(a, p, st);
    case DT_FP8: return dispatch_store<DT_FP8>(a, p, st);
    case DT_F32: return dispatch_store<DT_F32>(a, p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dspark
