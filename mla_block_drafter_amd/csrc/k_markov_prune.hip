// Markov rollout by exact candidate pruning (huggingface.co
// "Kimi-K3-DSpark-NVFP4", original card, "Model Overview": the low-rank
// sequential Markov head after the parallel backbone pass).
//
// Position i drafts t_i = argmax_v l_i[v] with l_i = z_i + W2 W1[t_{i-1}].
// By Cauchy-Schwarz |W2[v] . u| <= |W2[v]| |u| <= n2[v] B1, where n2[v] is
// the norm of W2's row v and B1 the largest row norm of W1 (both rounded up,
// computed once when the model is created).  So l_i[v] lies in
// [z_i[v] - n2[v] B1 - e_v, z_i[v] + n2[v] B1 + e_v], e_v bounding the fp32
// rounding of the dot product and of the add; a row whose upper end is below
// the largest lower end over the vocabulary can never be the argmax.  Only
// the remaining candidates are evaluated, sequentially, per sequence: a
// handful of 256-element dot products per position instead of the whole
// W2 product.  When any position keeps more candidates than fit, the
// rollout kernel does the whole product as before (a flag decides on the
// device; the pruning never changes which token is the argmax of the
// computed logits beyond rounding, and always the same way for the same
// inputs).
//
// Kernels: k_row_norms (model creation), k_markov_cand (per position and
// vocabulary chunk: the running largest lower end and the rows whose upper
// end reaches it, appended to the position's list), k_markov_prune (per
// sequence: the final threshold, the surviving candidates, the sequential
// rollout and the confidence, or the fallback flag).
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace dspark {

namespace {

// Rounding slack of l = z + W2[v] . u computed in fp32 from bf16 products
// (exact) over R <= 256 terms: |error| <= R 2^-24 sum |W2 u| <= 2^-16 n2 B1
// for the sum, 2^-24 |z + d| for the add; doubled for margin.
__device__ __forceinline__ float prune_slack(float z, float nb) {
  return 0x1p-15f * nb + 0x1p-22f * (fabsf(z) + nb);
}

// One thread per row: an upper bound of the row's L2 norm (fp64 sum of the
// exact squares, square root rounded up to fp32) and the running maximum
// (non-negative floats order as their bit patterns).
__global__ __launch_bounds__(256) void k_row_norms(const void* rows, int f32, long long ld, int R, int V, float* nrm,
                                                   unsigned* maxbits) {
  const long long v = (long long)blockIdx.x * 256 + threadIdx.x;
  if (v >= V) return;
  double ss = 0.0;
  for (int k = 0; k < R; ++k) {
    const double x = f32 ? (double)((const float*)rows)[v * ld + k]
                         : (double)bf16_bits_to_f32(((const uint16_t*)rows)[v * ld + k]);
    ss += x * x;
  }
  const double n = sqrt(ss) * (1.0 + 1e-12);
  float f = (float)n;
  if ((double)f < n) f = __uint_as_float(__float_as_uint(f) + 1u);  // next float up (f >= 0, finite)
  if (nrm) nrm[v] = f;
  if (maxbits) atomicMax(maxbits, __float_as_uint(f));
}

// Order-preserving bits of a float (larger float, larger unsigned).
__device__ __forceinline__ unsigned f2ord(float f) {
  const unsigned u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord2f(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Grid (chunks, rows m = s * block + i).  The chunk's largest lower end is
// merged into the row's running maximum (one atomic per workgroup); the
// chunk's rows whose upper end reaches the larger of the two are appended to
// the row's list as (row, z, bound).  The running maximum only grows, so the
// list holds every row whose upper end reaches the final maximum (the exact
// candidates) and some that do not, which the rollout drops.
__global__ __launch_bounds__(256) void k_markov_cand(MarkovPruneArgs a) {
  __shared__ float red[4];
  __shared__ float thr;
  const int c = blockIdx.x, m = blockIdx.y;
  const float B1 = __uint_as_float(*a.w1max);
  const float* z = a.z + (long long)m * a.vocab;
  float zv[MK_CHUNK / 256], nb[MK_CHUNK / 256];
  float lo = -INFINITY;
#pragma unroll
  for (int e = 0; e < MK_CHUNK / 256; ++e) {
    const int v = c * MK_CHUNK + e * 256 + threadIdx.x;
    const bool ok = v < a.vocab;
    zv[e] = ok ? z[v] : -INFINITY;
    nb[e] = ok ? a.n2[v] * B1 : 0.f;
    if (ok) lo = fmaxf(lo, zv[e] - nb[e] - prune_slack(zv[e], nb[e]));
  }
  const float L = block_max256(lo, red);
  if (threadIdx.x == 0) thr = fmaxf(L, ord2f(atomicMax(a.lmax + m, f2ord(L))));
  __syncthreads();
  const float T = thr;
#pragma unroll
  for (int e = 0; e < MK_CHUNK / 256; ++e) {
    const int v = c * MK_CHUNK + e * 256 + threadIdx.x;
    const float up = zv[e] + nb[e] + prune_slack(zv[e], nb[e]);
    if (v < a.vocab && up >= T) {
      const int k = atomicAdd(a.lcnt + m, 1);
      if (k < MK_CAPR) a.list[(long long)m * MK_CAPR + k] = u32x4{(unsigned)v, __float_as_uint(zv[e]), __float_as_uint(nb[e]), 0u};
    }
  }
}

// One workgroup per sequence: one memory round for every position's final
// threshold and list, one for the rows, then LDS only.
//  1. keep the list entries whose upper end reaches the final largest lower
//     end (too many anywhere: the fallback flag is raised, nothing written);
//  2. W2's row of every candidate and W1's row of every possible predecessor
//     (the candidates of the previous position, the last verified token, or
//     the forced predecessors) into LDS;
//  3. the positions in order: l = z + W2 row . u on each candidate, the
//     argmax key (lowest index on ties), the confidence as k_markov_final
//     computes it.
__global__ __launch_bounds__(256) void k_markov_prune(MarkovPruneArgs a) {
  constexpr int MB = MK_MAX_BLOCK, CG = MK_CAPG, EPT = MK_CAPR / 256;
  __shared__ __attribute__((aligned(16))) uint16_t w2c[MB][CG][256];  // W2 rows of the candidates
  __shared__ __attribute__((aligned(16))) uint16_t w1c[MB][CG][256];  // W1 rows of the candidates (predecessors)
  __shared__ __attribute__((aligned(16))) uint16_t w1p[MB][256];      // W1 rows of explicit predecessors
  __shared__ int lst[MB][CG];
  __shared__ float zc[MB][CG];
  __shared__ int nl[MB];
  __shared__ float rsp[MB], hdp[MB];
  __shared__ float red[4];
  __shared__ float uu[256];
  __shared__ unsigned long long kred[4];
  __shared__ int bad;
  const int s = blockIdx.x, B = a.block, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) bad = 0;
  if (threadIdx.x < MB) nl[threadIdx.x] = 0;
  // round 1: every position's threshold, count and list entries, row scale and dot
  float Lp[MB];
  int cntp[MB];
  u32x4 ent[MB][EPT];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const long long m = (long long)s * B + (i < B ? i : 0);
    Lp[i] = ord2f(a.lmax[m]);
    cntp[i] = a.lcnt[m];
#pragma unroll
    for (int q = 0; q < EPT; ++q) ent[i][q] = a.list[m * MK_CAPR + q * 256 + threadIdx.x];
  }
  for (int i = wave; i < B; i += 4) {
    const long long m = (long long)s * B + i;
    const float rs = row_scale_wave(a.rs_final, (int)m);
    const float hd = chunk_sum_wave(a.dot + m * SSQ_LD, a.nch_dot);
    if (lane == 0) {
      rsp[i] = rs;
      hdp[i] = hd;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    if (i >= B) break;
    if (cntp[i] > MK_CAPR) bad = 1;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int k = q * 256 + threadIdx.x;
      if (k >= cntp[i]) continue;
      const float zv = __uint_as_float(ent[i][q][1]), nb = __uint_as_float(ent[i][q][2]);
      if (zv + nb + prune_slack(zv, nb) >= Lp[i]) {
        const int j = atomicAdd(&nl[i], 1);
        if (j < CG) {
          lst[i][j] = (int)ent[i][q][0];
          zc[i][j] = zv;
        } else {
          bad = 1;
        }
      }
    }
  }
  __syncthreads();
  if (bad) {  // uniform (read after the barrier)
    if (threadIdx.x == 0) *a.fallback = 1;  // benign race: every writer stores 1
    return;
  }
  // round 2: rows into LDS, 16 bytes per thread and step: W2 rows (packed
  //    16-row tiles: dims 8 q .. 8 q + 7 of k block kb of row v at
  //    ((tile KB + kb) 64 + q 16 + v % 16) 16 bytes), W1 rows (plain, row
  //    stride w1_ld)
  const int R = a.R, KB = a.KB, nq = KB * 4;  // 16-byte pieces per row
  const uint16_t* w1 = (const uint16_t*)a.w1;
  for (int e = threadIdx.x; e < B * CG * nq; e += 256) {
    const int i = e / (CG * nq), r = e % (CG * nq), j = r / nq, p = r % nq;
    if (j >= nl[i]) continue;
    const int v = lst[i][j], kb = p >> 2, q = p & 3;
    *(u32x4*)&w2c[i][j][p * 8] =
        *(const u32x4*)((const uint16_t*)a.w2 + ((long long)(v >> 4) * KB * 64 + kb * 64 + q * 16 + (v & 15)) * 8);
    if (!a.forced && i + 1 < B) *(u32x4*)&w1c[i][j][p * 8] = *(const u32x4*)(w1 + (long long)v * a.w1_ld + p * 8);
  }
  for (int e = threadIdx.x; e < B * nq; e += 256) {
    const int i = e / nq, p = e % nq;
    if (i > 0 && !a.forced) continue;
    const int t = i == 0 ? a.prev_token[s] : a.forced[s * B + i - 1];
    const bool ok = t >= 0 && t < a.vocab;
    *(u32x4*)&w1p[i][p * 8] = ok ? *(const u32x4*)(w1 + (long long)t * a.w1_ld + p * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  // 3. the positions in order
  int jprev = -1;  // list index of the previous position's pick (free running)
  int tprev = -1;
  for (int i = 0; i < B; ++i) {
    const bool explicit_pred = i == 0 || a.forced;
    const int tp = explicit_pred ? (i == 0 ? a.prev_token[s] : a.forced[s * B + i - 1]) : tprev;
    const bool has = tp >= 0 && tp < a.vocab;
    const uint16_t* urow = explicit_pred ? w1p[i] : w1c[i - 1][jprev];
    uu[threadIdx.x] = has && (int)threadIdx.x < R ? bf16_bits_to_f32(urow[threadIdx.x]) : 0.f;
    __syncthreads();
    // candidate j: 16 threads (16 dims each), summed in a fixed butterfly
    const int n = nl[i];
    const int j = threadIdx.x >> 4, part = threadIdx.x & 15;
    float d = 0.f;
    if (j < n && part * 16 < KB * 32) {  // (the LDS rows hold the KB k blocks of the packed rank)
#pragma unroll
      for (int k = 0; k < 16; ++k) d += bf16_bits_to_f32(w2c[i][j][part * 16 + k]) * uu[part * 16 + k];
    }
    d = row16_sum(d);
    unsigned long long best = 0;
    if (j < n && part == 0) best = argmax_key(zc[i][j] + d, (uint32_t)lst[i][j]);
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long other = ((unsigned long long)__shfl_xor((unsigned)(best >> 32), o, 64) << 32) |
                                       (unsigned)__shfl_xor((unsigned)best, o, 64);
      best = best > other ? best : other;
    }
    if (lane == 0) kred[wave] = best;
    float dm = 0.f;
    if (has)
      for (int k = threadIdx.x; k < R; k += 256) dm += uu[k] * a.conf_wm[k];
    dm = block_sum256(dm, red);  // (its barriers also publish kred)
    best = kred[0];
    for (int q = 1; q < 4; ++q) best = best > kred[q] ? best : kred[q];
    const int t = key_index(best);
    int jt = 0;
    for (int q = 0; q < n; ++q) jt = lst[i][q] == t ? q : jt;
    const long long m = (long long)s * B + i;
    if (threadIdx.x == 0) {
      a.tokens[m] = t;
      const float x = rsp[i] * hdp[i] + dm + a.conf_b[0];
      a.conf[m] = 1.f / (1.f + __expf(-x));
      if (i == 0 && a.status && s == 0) *a.status = 2;  // drafted by the candidate rollout
    }
    tprev = t;
    jprev = jt;
    __syncthreads();  // uu and kred are rewritten by the next position
  }
}

}  // namespace

hipError_t launch_row_norms(const void* rows, int f32, long long ld, int R, int V, float* nrm, unsigned* maxbits,
                            hipStream_t st) {
  if (V <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_row_norms, dim3((V + 255) / 256), dim3(256), 0, st, rows, f32, ld, R, V, nrm, maxbits);
  return hipGetLastError();
}

bool markov_prune_supported(int R, int block, int vocab) {
  return R >= 1 && R <= 256 && block >= 1 && block <= MK_MAX_BLOCK && vocab >= 1;
}

hipError_t launch_markov_prune(const MarkovPruneArgs& a, hipStream_t st) {
  if (!markov_prune_supported(a.R, a.block, a.vocab) || a.n_seq < 1 || a.nch != markov_prune_chunks(a.vocab))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_markov_cand, dim3(a.nch, a.n_seq * a.block), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_markov_prune, dim3(a.n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
