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
// vocabulary chunk: the chunk's largest lower end and the rows whose upper
// end reaches it, in slots of their own), k_markov_prune (per sequence: the
// final threshold, the surviving candidates, the sequential rollout and the
// confidence, or the fallback flag).
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

// Grid (chunks, rows m = s * block + i), 1024 threads, 8 vocabulary rows per
// thread.  The chunk's largest lower end L and the count of its rows whose
// upper end reaches L go to (m, chunk); the first MK_CAPC of those rows to
// the chunk's slots.  Every row whose upper end reaches the final threshold
// (the largest L of the position) reaches its own chunk's L, so the slots
// hold every exact candidate unless a count exceeds MK_CAPC.
__global__ __launch_bounds__(1024) void k_markov_cand(MarkovPruneArgs a) {
  constexpr int E = MK_CHUNK / 1024;
  __shared__ float red[16];
  __shared__ int wcnt[16];
  const int c = blockIdx.x, m = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float B1 = __uint_as_float(*a.w1max);
  const float* z = a.z + (long long)m * a.vocab;
  float zv[E], nb[E];
  float lo = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int v = c * MK_CHUNK + e * 1024 + threadIdx.x;
    const bool ok = v < a.vocab;
    zv[e] = ok ? z[v] : -INFINITY;
    nb[e] = ok ? a.n2[v] * B1 : 0.f;
    if (ok) lo = fmaxf(lo, zv[e] - nb[e] - prune_slack(zv[e], nb[e]));
  }
  lo = wave_max(lo);
  if (lane == 0) red[wave] = lo;
  __syncthreads();
  float L = red[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) L = fmaxf(L, red[w]);
  unsigned long long pass[E];
  int wtot = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int v = c * MK_CHUNK + e * 1024 + threadIdx.x;
    pass[e] = __ballot(v < a.vocab && zv[e] + nb[e] + prune_slack(zv[e], nb[e]) >= L);
    wtot += __popcll(pass[e]);
  }
  if (lane == 0) wcnt[wave] = wtot;
  __syncthreads();
  int k = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    k += w < wave ? wcnt[w] : 0;
    tot += wcnt[w];
  }
  const long long mc = (long long)m * a.nch + c;
  if (threadIdx.x == 0) {
    a.lch[mc] = L;
    a.ccnt[mc] = tot;
  }
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int kk = k + __popcll(pass[e] & below);
    if (((pass[e] >> lane) & 1ull) && kk < MK_CAPC) {
      const int v = c * MK_CHUNK + e * 1024 + threadIdx.x;
      a.list[mc * MK_CAPC + kk] = u32x4{(unsigned)v, __float_as_uint(zv[e]), __float_as_uint(nb[e]), 0u};
    }
    k += __popcll(pass[e]);
  }
}

// Zero the dims from R on of a 16-byte piece (dims 8 p .. 8 p + 7, bf16).
__device__ __forceinline__ u32x4 mask_dims(u32x4 x, int p, int R) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int d = 8 * p + 2 * w;
    if (d >= R) x[w] = 0u;
    else if (d + 1 >= R) x[w] &= 0xFFFFu;
  }
  return x;
}

// w_m . u for a W1 row u, by the 16 lanes of one DPP row, in the order of a
// 256-thread block sum with thread k holding u[k] w_m[k] (the order
// k_markov_final uses): per 64-thread wave the four 16-lane row sums, paired
// (0 + 1) + (2 + 3); then the four waves left to right.
__device__ __forceinline__ float conf_dot16(const uint16_t* w1row, const float* wm, int q, int R) {
  float ws[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float r[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int k = w * 64 + h * 16 + q;
      float p = 0.f;
      if (k < R) p = fmaf(bf16_bits_to_f32(w1row[k]), wm[k], 0.f);
      r[h] = row16_sum(p);
    }
    ws[w] = (r[0] + r[1]) + (r[2] + r[3]);
  }
  return ((ws[0] + ws[1]) + ws[2]) + ws[3];
}

// One workgroup per sequence: one memory trip for every position's chunk
// thresholds and slots (and every small input), one for the rows, then LDS
// only (plus one sweep of the logits of any chunk whose candidates
// overflowed its slots).
//  1. the position's threshold is the largest chunk L; keep the slot entries
//     whose upper end reaches it, and rescan the chunks that had more
//     candidates than slots against it (more than MK_CAPG candidates for a
//     position, or none: the fallback flag is raised, nothing written);
//  2. W2's row of every candidate and W1's row of every possible predecessor
//     (the candidates of the previous position, the last verified token, or
//     the forced predecessors) into LDS;
//  3. in parallel, the Markov term of every (candidate, possible
//     predecessor) pair and w_m . u of every possible predecessor;
//  4. in parallel, for every position and possible predecessor: the argmax
//     of l = z + term over the candidates (lowest index on ties) and the
//     confidence as k_markov_final computes it;
//  5. one thread follows the picks from the first position on.
__global__ __launch_bounds__(256) void k_markov_prune(MarkovPruneArgs a) {
  constexpr int MB = MK_MAX_BLOCK, CG = MK_CAPG, NCH = MK_MAXCH, CC = MK_CAPC;
  constexpr int IPT = MB * NCH * CC / 256;  // slot entries per thread
  static_assert(MB <= 8, "two positions per wave in the first round");
  // rows (RS 16-byte pieces each, one more than a 256-dim row so that rows
  // start on different banks): W2 rows of the candidates [MB][CG], W1 rows
  // of the candidates (predecessors) [MB][CG], W1 rows of the explicit
  // predecessors [MB]
  constexpr int RS = 33, R1C = MB * CG, R1P = 2 * MB * CG;
  __shared__ u32x4 rows[(2 * MB * CG + MB) * RS];
  __shared__ float term[MB][CG][CG];  // [position][candidate][predecessor]
  __shared__ float cdot[MB][CG];      // w_m . u of position i's predecessor p
  __shared__ int pk_t[MB][CG], pk_j[MB][CG];  // pick given predecessor p: token, candidate index
  __shared__ float pk_c[MB][CG];              // and the confidence
  __shared__ int lst[MB][CG];
  __shared__ float zc[MB][CG];
  __shared__ unsigned Lord[MB];  // order-preserving bits of the position's threshold
  __shared__ unsigned ovf[MB];   // bit c: chunk c of the position had more candidates than slots
  __shared__ int nl[MB];
  __shared__ float rsp[MB], hdp[MB];
  __shared__ float cw[256];  // w_m
  __shared__ int tpx[MB];    // explicit predecessors: the last verified token, the forced ones
  __shared__ float cb;       // confidence bias
  __shared__ int bad;
  const int s = blockIdx.x, B = a.block, nch = a.nch, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) bad = 0;
  if (threadIdx.x < MB) {
    nl[threadIdx.x] = 0;
    Lord[threadIdx.x] = 0u;
    ovf[threadIdx.x] = 0u;
  }
  __syncthreads();
  // first memory trip: every global read before the rows, issued together
  const float cwv = (int)threadIdx.x < a.R ? a.conf_wm[threadIdx.x] : 0.f;
  const float cbv = a.conf_b[0];
  int tpv = -1;
  if ((int)threadIdx.x < B)
    tpv = threadIdx.x == 0 ? a.prev_token[s] : (a.forced ? a.forced[s * B + threadIdx.x - 1] : -1);
  u32x4 ent[IPT];
  int cnt[IPT];
  float lv[IPT];
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const int it = e * 256 + threadIdx.x, i = it / (NCH * CC), c = (it / CC) % NCH;
    const bool ok = i < B && c < nch;
    const long long mc = ((long long)s * B + (ok ? i : 0)) * nch + (ok ? c : 0);
    ent[e] = a.list[mc * CC + it % CC];
    cnt[e] = ok ? a.ccnt[mc] : 0;
    lv[e] = a.lch[mc];
  }
  // row scale and hidden dot of positions wave and wave + 4
  const int i0 = wave, i1 = wave + 4;
  const long long m0 = (long long)s * B + min(i0, B - 1), m1 = (long long)s * B + min(i1, B - 1);
  const float q0 = chunk_lane_sum(a.rs_final.ssq + m0 * SSQ_LD, a.rs_final.nch, lane);
  const float q1 = chunk_lane_sum(a.rs_final.ssq + m1 * SSQ_LD, a.rs_final.nch, lane);
  const float d0 = chunk_lane_sum(a.dot + m0 * SSQ_LD, a.nch_dot, lane);
  const float d1 = chunk_lane_sum(a.dot + m1 * SSQ_LD, a.nch_dot, lane);
  {
    const float rs0 = rsqrtf(wave_sum(q0) * a.rs_final.invn + a.rs_final.eps);
    const float rs1 = rsqrtf(wave_sum(q1) * a.rs_final.invn + a.rs_final.eps);
    const float hd0 = wave_sum(d0), hd1 = wave_sum(d1);
    if (lane == 0 && i0 < B) {
      rsp[i0] = rs0;
      hdp[i0] = hd0;
    }
    if (lane == 0 && i1 < B) {
      rsp[i1] = rs1;
      hdp[i1] = hd1;
    }
  }
  cw[threadIdx.x] = cwv;
  if (threadIdx.x == 0) cb = cbv;
  if ((int)threadIdx.x < B) tpx[threadIdx.x] = tpv;
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const int it = e * 256 + threadIdx.x, i = it / (NCH * CC), c = (it / CC) % NCH;
    if (i < B && c < nch && it % CC == 0) atomicMax(&Lord[i], f2ord(lv[e]));
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const int it = e * 256 + threadIdx.x, i = it / (NCH * CC), k = it % CC;
    if (cnt[e] > CC) {  // the slots hold only part of the chunk: rescanned below
      if (k == 0) atomicOr(&ovf[i], 1u << ((it / CC) % NCH));
      continue;
    }
    if (k >= cnt[e]) continue;  // (also every item outside the positions and chunks: cnt 0)
    const float zv = __uint_as_float(ent[e][1]), nb = __uint_as_float(ent[e][2]);
    if (zv + nb + prune_slack(zv, nb) >= ord2f(Lord[i])) {
      const int j = atomicAdd(&nl[i], 1);
      if (j < CG) {
        lst[i][j] = (int)ent[e][0];
        zc[i][j] = zv;
      } else {
        bad = 1;
      }
    }
  }
  __syncthreads();
  // Chunks with more candidates than slots: every row of the chunk against
  // the position's final threshold, its bound formed as k_markov_cand forms
  // it (the same candidates the slots would have held).
  {
    const float B1 = __uint_as_float(*a.w1max);
    for (int i = 0; i < B; ++i) {
      unsigned bits = ovf[i];  // uniform (after the barrier)
      const float L = ord2f(Lord[i]);
      const float* zr = a.z + ((long long)s * B + i) * a.vocab;
      while (bits) {
        const int c = __builtin_ctz(bits);
        bits &= bits - 1u;
        const int v1 = min((c + 1) * MK_CHUNK, a.vocab);
        for (int v = c * MK_CHUNK + (int)threadIdx.x; v < v1; v += 256) {
          const float zv = zr[v], nb = a.n2[v] * B1;
          if (zv + nb + prune_slack(zv, nb) >= L) {
            const int j = atomicAdd(&nl[i], 1);
            if (j < CG) {
              lst[i][j] = v;
              zc[i][j] = zv;
            } else {
              bad = 1;
            }
          }
        }
      }
    }
  }
  __syncthreads();
  // flat offsets per position (registers, constant indices only): candidates,
  // predecessors (one explicit row, or the previous position's candidates)
  const bool forced = a.forced != nullptr;
  int nlv[MB], off[MB + 1], pb[MB + 1];
  bool give_up = bad != 0;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    nlv[i] = i < B ? nl[i] : 0;
    give_up |= i < B && nlv[i] == 0;  // (NaN logits only)
  }
  off[0] = pb[0] = 0;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int npi = i < B ? ((forced || i == 0) ? 1 : nlv[i > 0 ? i - 1 : 0]) : 0;
    off[i + 1] = off[i] + nlv[i];
    pb[i + 1] = pb[i] + npi;
  }
  if (give_up) {  // uniform (read after the barrier)
    if (threadIdx.x == 0) *a.fallback = 1;  // benign race: every writer stores 1
    return;
  }
  // segment of a flat index x in a prefix array and its start
  auto seg = [](const int (&v)[MB + 1], int x, int& i, int& base) {
    i = 0;
    base = 0;
#pragma unroll
    for (int t = 1; t < MB; ++t)
      if (x >= v[t]) {
        i = t;
        base = v[t];
      }
  };
  // second memory trip: rows into LDS, 16 bytes per piece.  W2 rows are packed in
  //    16-row tiles: dims 8 q .. 8 q + 7 of k block kb of row v sit at
  //    ((tile KB + kb) 64 + q 16 + v % 16) 16 bytes.  W1 rows are plain
  //    (row stride w1_ld).  Pieces: [0, n2p) W2 rows of the candidates,
  //    [n2p, n2p + n1p) W1 rows of the candidates that can precede a position
  //    (free running), then the explicit predecessors; all loads of a thread
  //    are issued before the first store.
  const int R = a.R, KB = a.KB, nq = KB * 4;  // 16-byte pieces per row
  int nc = 0, ncp = 0, npred = 0;
#pragma unroll
  for (int i = 0; i <= MB; ++i) {
    nc = i == B ? off[i] : nc;
    ncp = (i == B - 1 && !forced) ? off[i] : ncp;  // candidates of positions 0 .. B-2 (predecessors)
    npred = i == B ? pb[i] : npred;
  }
  const int nexp = forced ? B : 1;
  const int n2p = nc * nq, n1p = ncp * nq, np = n2p + n1p + nexp * nq;
  const uint16_t* w1 = (const uint16_t*)a.w1;
  constexpr int U = 8;
  for (int e0 = 0; e0 < np; e0 += 256 * U) {
    u32x4 buf[U];
    int dst[U];  // 16-byte slot in rows, -1: none
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * 256 + (int)threadIdx.x;
      dst[u] = -1;
      buf[u] = u32x4{0u, 0u, 0u, 0u};
      if (e < n2p + n1p) {
        const bool is2 = e < n2p;
        const int f = is2 ? e / nq : (e - n2p) / nq, p = is2 ? e % nq : (e - n2p) % nq;
        int i, base;
        seg(off, f, i, base);
        const int j = f - base, v = lst[i][j];
        if (is2) {
          const int kb = p >> 2, q = p & 3;
          buf[u] = *(const u32x4*)((const uint16_t*)a.w2 + ((long long)(v >> 4) * KB * 64 + kb * 64 + q * 16 + (v & 15)) * 8);
          dst[u] = (i * CG + j) * RS + p;
        } else {
          buf[u] = *(const u32x4*)(w1 + (long long)v * a.w1_ld + p * 8);
          dst[u] = (R1C + i * CG + j) * RS + p;
        }
        buf[u] = mask_dims(buf[u], p, R);
      } else if (e < np) {
        const int i = (e - n2p - n1p) / nq, p = (e - n2p - n1p) % nq;
        const int t = tpx[i];
        if (t >= 0 && t < a.vocab) buf[u] = mask_dims(*(const u32x4*)(w1 + (long long)t * a.w1_ld + p * 8), p, R);
        dst[u] = (R1P + i) * RS + p;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (dst[u] >= 0) rows[dst[u]] = buf[u];
  }
  __syncthreads();
  // 3. the (candidate, predecessor) pairs on the matrix cores, one wave per
  //    position: A = W1 rows of the predecessors, B = W2 rows of the
  //    candidates, accumulated over the k blocks in order from zero, as the
  //    full rollout does (the same products and sums for every pair); then
  //    the predecessors' w_m . u, one 16-lane row each
  for (int i = wave; i < B; i += 4) {
    const bool ex = forced || i == 0;
    const int npi = ex ? 1 : nl[i - 1], n = nl[i];
    const int l16 = lane & 15, qa = lane >> 4;
    const u32x4* arow = ex ? &rows[(R1P + i) * RS] : &rows[(R1C + (i - 1) * CG + l16) * RS];
    const u32x4* brow = &rows[(i * CG + l16) * RS];
    // all operand reads first (KB <= 8), then the products
    u32x4 av[8], bv[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      av[kb] = kb < KB ? arow[kb * 4 + qa] : u32x4{0u, 0u, 0u, 0u};
      bv[kb] = kb < KB ? brow[kb * 4 + qa] : u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
      if (kb < KB)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[kb]), __builtin_bit_cast(bf16x8, bv[kb]),
                                                      acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = qa * 4 + r;  // output row: predecessor; column: candidate l16
      if (l16 < n && p < npi) term[i][l16][p] = acc[r];
    }
  }
  const int q = threadIdx.x & 15;
  for (int r0 = 0; r0 < npred; r0 += 16) {
    const int r = r0 + (int)(threadIdx.x >> 4);  // uniform across the 16-lane row
    if (r < npred) {
      int i, base;
      seg(pb, r, i, base);
      const int p = r - base;
      const u32x4* u = (forced || i == 0) ? &rows[(R1P + i) * RS] : &rows[(R1C + (i - 1) * CG + p) * RS];
      const float d = conf_dot16((const uint16_t*)u, cw, q, R);
      if (q == 0) cdot[i][p] = d;
    }
  }
  __syncthreads();
  // 4. one thread per (position, possible predecessor)
  if ((int)threadIdx.x < npred) {
    int i, base;
    seg(pb, threadIdx.x, i, base);
    const int p = threadIdx.x - base;
    const int n = nl[i];
    unsigned long long best = 0;
    int jt = 0;
#pragma unroll
    for (int j = 0; j < CG; ++j) {
      const unsigned long long key = argmax_key(zc[i][j] + term[i][j][p], (uint32_t)lst[i][j]);
      if (j < n && key > best) {
        best = key;
        jt = j;
      }
    }
    const bool explicit_pred = forced || i == 0;
    const bool has = !explicit_pred || (tpx[i] >= 0 && tpx[i] < a.vocab);
    const float x = rsp[i] * hdp[i] + (has ? cdot[i][p] : 0.f) + cb;
    pk_t[i][p] = key_index(best);
    pk_j[i][p] = jt;
    pk_c[i][p] = 1.f / (1.f + __expf(-x));
  }
  __syncthreads();
  // 5. the picks in order
  if (threadIdx.x == 0) {
    int p = 0;
    for (int i = 0; i < B; ++i) {
      const long long m = (long long)s * B + i;
      a.tokens[m] = pk_t[i][p];
      a.conf[m] = pk_c[i][p];
      p = forced ? 0 : pk_j[i][p];
    }
    if (a.status && s == 0) *a.status = 2;  // drafted by the candidate rollout
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
  return R >= 1 && R <= 256 && block >= 1 && block <= MK_MAX_BLOCK && vocab >= 1 &&
         markov_prune_chunks(vocab) <= MK_MAXCH;
}

hipError_t launch_markov_prune(const MarkovPruneArgs& a, hipStream_t st) {
  if (!markov_prune_supported(a.R, a.block, a.vocab) || a.n_seq < 1 || a.nch != markov_prune_chunks(a.vocab))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_markov_cand, dim3(a.nch, a.n_seq * a.block), dim3(1024), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_markov_prune, dim3(a.n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
