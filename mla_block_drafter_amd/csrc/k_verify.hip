// Verification of a drafted block under sampling (huggingface.co
// "Kimi-K3-DSpark-NVFP4", "Sampling options": the draft sampled from its own
// distribution, and the block verified token by token or as a unit).
//
// With q_i = softmax(l_i / T) the draft's and p_i = softmax(t_i / T) the
// target's distribution at position i (p_B after the whole block):
//  * token: accept x_i while r_i < min(1, p_i(x_i) / q_i(x_i)); at the first
//    rejection draw from max(p_i - q_i, 0), else from p_B;
//  * block: prefix weights w_0 = 1, w_k = min(w_{k-1} p_{k-1}(x_{k-1}) /
//    q_{k-1}(x_{k-1}), 1); residual res_k = max(w_k p_k - q_k, 0) of mass
//    S_k; k is accepted when r_{k-1} < h_k with h_k = S_k / (S_k + 1 - w_k)
//    (h_B = w_B); the accepted length is the largest accepted k; then a draw
//    from res_k (or p_B when k = B).
// Draws use the inverse CDF: the lowest index whose cumulative mass exceeds
// u times the total.
//
// Four launches: (1) per (sequence, position, vocabulary chunk) the running
// maximum and sum of exp of the tempered logits (one pass, online); (2) per
// sequence, one wave: the row normalisers, the drafted tokens' probabilities
// and the prefix weights; (3) per (sequence, position < B, chunk) the
// residual masses of both rules; (4) per sequence the decision and the draw:
// the chunk masses locate the threshold's chunk, one workgroup scans it.
#include "kernels.h"

namespace dspark {

namespace {

// vocabulary chunks per row in launches 1 and 3 (at most 64: launch 4 holds
// one chunk per lane of a wave)
constexpr int VF_NCH = 64;

// (max, sum) merge of two partial softmax normalisers
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  const float mx = fmaxf(m, m2);
  s = s * __expf(m - mx) + s2 * __expf(m2 - mx);
  m = mx;
}

__device__ void block_ms(float& m, float& s, float* red) {
  // wave merge by DPP-free shuffles (once per launch), then across the 4 waves
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ms_merge(m, s, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[2 * w] = m;
    red[2 * w + 1] = s;
  }
  __syncthreads();
  m = red[0];
  s = red[1];
  for (int i = 1; i < 4; ++i) ms_merge(m, s, red[2 * i], red[2 * i + 1]);
}

// (max, sum of exp(x - max)) of this thread's entries c0 + tid, + 256, ...
// below c1 of the tempered row: the maximum first, then one exp per entry
__device__ __forceinline__ void thread_ms(const float* row, int c0, int c1, float inv_temp, float& m, float& s) {
  m = -INFINITY;
  s = 0.f;
#pragma unroll 4
  for (int v = c0 + threadIdx.x; v < c1; v += 256) m = fmaxf(m, row[v] * inv_temp);
  if (m == -INFINITY) return;
#pragma unroll 4
  for (int v = c0 + threadIdx.x; v < c1; v += 256) s += __expf(row[v] * inv_temp - m);
}

// stats layout per (sequence, row): [chunk][4] = target (m, s), draft (m, s)
__global__ __launch_bounds__(256) void k_verify_norm(VerifyArgs a) {
  __shared__ float red[8];
  const int s = blockIdx.x, i = blockIdx.y, ch = blockIdx.z;
  const int B = a.block, V = a.vocab;
  const int c0 = (int)((long long)V * ch / VF_NCH), c1 = (int)((long long)V * (ch + 1) / VF_NCH);
  const float* t = a.tlog + ((long long)s * (B + 1) + i) * V;
  float mt, st, md = -INFINITY, sd = 0.f;
  thread_ms(t, c0, c1, a.inv_temp, mt, st);
  block_ms(mt, st, red);
  if (i < B) {
    thread_ms(a.dlog + ((long long)s * B + i) * V, c0, c1, a.inv_temp, md, sd);
    block_ms(md, sd, red);
  }
  if (threadIdx.x == 0) {
    float* o = a.stats + (((long long)s * (B + 1) + i) * VF_NCH + ch) * 4;
    o[0] = mt;
    o[1] = st;
    o[2] = md;
    o[3] = sd;
  }
}

// Per-row scalars of one sequence: the tempered normalisers of both models
// (each wave merges a row's chunk partials, one chunk per lane), then, on
// wave 0 with lane i holding row i <= B, the probabilities of the drafted
// token under each model and the block rule's prefix weight w_i.
__global__ __launch_bounds__(256) void k_verify_probs(VerifyArgs a) {
  __shared__ float nrm[64][4];
  const int s = blockIdx.x, B = a.block, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long V = a.vocab;
  for (int row = wave; row <= B; row += 4) {
    const float* o = a.stats + (((long long)s * (B + 1) + row) * VF_NCH + lane) * 4;
    float mt = -INFINITY, st = 0.f, md = -INFINITY, sd = 0.f;
    if (lane < VF_NCH) {
      mt = o[0];
      st = o[1];
      md = o[2];
      sd = o[3];
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) {
      ms_merge(mt, st, __shfl_xor(mt, x, 64), __shfl_xor(st, x, 64));
      ms_merge(md, sd, __shfl_xor(md, x, 64), __shfl_xor(sd, x, 64));
    }
    if (lane == 0) {
      nrm[row][0] = mt;
      nrm[row][1] = st;
      nrm[row][2] = md;
      nrm[row][3] = sd;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const int i = lane;
  float mt = -INFINITY, st = 0.f, md = -INFINITY, sd = 0.f, pt = 0.f, pq = 1.f;
  if (i <= B) {
    mt = nrm[i][0];
    st = nrm[i][1];
    md = nrm[i][2];
    sd = nrm[i][3];
  }
  if (i < B) {
    const int x = a.draft[(long long)s * B + i];
    if (x >= 0 && x < V) {  // else not a token: the target never emits it, so it is rejected
      pt = __expf(a.tlog[((long long)s * (B + 1) + i) * V + x] * a.inv_temp - mt) / st;
      pq = __expf(a.dlog[((long long)s * B + i) * V + x] * a.inv_temp - md) / sd;
    }
  }
  // w_0 = 1, w_k = min(w_{k-1} p_{k-1}(x) / q_{k-1}(x), 1): every lane runs the
  // chain and keeps its own entry
  float w = 1.f, wi = 1.f;
  for (int k = 1; k <= B; ++k) {
    const float ptk = __shfl(pt, k - 1, 64), pqk = __shfl(pq, k - 1, 64);
    w = fminf(w * ptk / pqk, 1.f);
    if (k == i) wi = w;
  }
  if (i <= B) {
    float* o = a.probs + ((long long)s * (B + 1) + i) * 8;
    o[0] = mt;
    o[1] = st;
    o[2] = md;
    o[3] = sd;
    o[4] = pt;
    o[5] = pq;
    o[6] = wi;
    o[7] = 0.f;
  }
}

// residual masses at position i < B, chunk ch: token rule (w = 1) and block rule (w = w_i)
__global__ __launch_bounds__(256) void k_verify_resid(VerifyArgs a) {
  __shared__ float red[4];
  const int s = blockIdx.x, i = blockIdx.y, ch = blockIdx.z;
  const int B = a.block, V = a.vocab;
  const float* pr = a.probs + ((long long)s * (B + 1) + i) * 8;
  const float mt = pr[0], it = 1.f / pr[1], md = pr[2], id = 1.f / pr[3], w = pr[6];
  const int c0 = (int)((long long)V * ch / VF_NCH), c1 = (int)((long long)V * (ch + 1) / VF_NCH);
  const float* t = a.tlog + ((long long)s * (B + 1) + i) * V;
  const float* d = a.dlog + ((long long)s * B + i) * V;
  float rt = 0.f, rb = 0.f;
#pragma unroll 4
  for (int v = c0 + threadIdx.x; v < c1; v += 256) {
    const float p = __expf(t[v] * a.inv_temp - mt) * it, q = __expf(d[v] * a.inv_temp - md) * id;
    rt += fmaxf(p - q, 0.f);
    rb += fmaxf(w * p - q, 0.f);
  }
  rt = block_sum256(rt, red);
  rb = block_sum256(rb, red);
  if (threadIdx.x == 0) {
    float* o = a.resid + (((long long)s * B + i) * VF_NCH + ch) * 2;
    o[0] = rt;
    o[1] = rb;
  }
}

constexpr int VD_THREADS = 1024, VD_PER = 4;  // draw: 4 consecutive entries per thread per tile

// Decision and draw, one workgroup per sequence.  Wave 0 takes the decision
// (lane k looks at position k), then locates the vocabulary chunk holding the
// threshold from the chunk masses of launches 1 and 2; the workgroup then
// scans that chunk tile by tile for the first entry whose cumulative mass
// exceeds the threshold.
__global__ __launch_bounds__(VD_THREADS) void k_verify_decide(VerifyArgs a) {
  __shared__ int sh_tau, sh_ch, sh_first, sh_last;
  __shared__ float sh_thr;
  __shared__ float wsum[VD_THREADS / 64];
  __shared__ float Ssh[64];
  const int s = blockIdx.x, B = a.block, V = a.vocab;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool token = a.method == DSPARK_VERIFY_TOKEN_C;
  const float* r = a.u + (long long)s * (B + 1);
  const float* P = a.probs + (long long)s * (B + 1) * 8;
  if (!token) {  // block rule: residual masses S_k, 0 < k < B, one wave per row, one chunk per lane
    for (int k = wave + 1; k < B; k += VD_THREADS / 64) {
      float v = lane < VF_NCH ? a.resid[(((long long)s * B + k) * VF_NCH + lane) * 2 + 1] : 0.f;
#pragma unroll
      for (int x = 32; x >= 1; x >>= 1) v += __shfl_xor(v, x, 64);
      if (lane == 0) Ssh[k] = v;
    }
    __syncthreads();
  }
  if (tid < 64) {
    int tau;
    if (token) {  // the first rejected position, else B
      const bool rej = lane < B && !(r[lane] < fminf(1.f, P[lane * 8 + 4] / P[lane * 8 + 5]));
      const unsigned long long m = __ballot(rej);
      tau = m ? __builtin_ctzll(m) : B;
    } else {  // the largest k in 1..B with r_{k-1} < h_k, else 0
      bool acc = false;
      if (lane >= 1 && lane <= B) {
        const float w = P[lane * 8 + 6];
        float h = w;
        if (lane < B) {
          const float S = Ssh[lane];
          h = S + 1.f - w > 0.f ? S / (S + 1.f - w) : 1.f;
        }
        acc = r[lane - 1] < h;
      }
      const unsigned long long m = __ballot(acc);
      tau = m ? 63 - __builtin_clzll(m) : 0;
    }
    // chunk masses of the distribution drawn from: the residual of row tau,
    // or p_B after a full block
    float mass = 0.f;
    if (lane < VF_NCH) {
      if (tau < B) {
        mass = a.resid[(((long long)s * B + tau) * VF_NCH + lane) * 2 + (token ? 0 : 1)];
      } else {
        const float* o = a.stats + (((long long)s * (B + 1) + B) * VF_NCH + lane) * 4;
        mass = o[0] == -INFINITY ? 0.f : o[1] * __expf(o[0] - P[B * 8]) / P[B * 8 + 1];
      }
    }
    float incl = mass;
#pragma unroll
    for (int o = 1; o < VF_NCH; o <<= 1) {
      const float y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    static_assert(VF_NCH <= 64, "one chunk per lane");
    const float total = __shfl(incl, VF_NCH - 1, 64);
    const float thr = r[B] * total;
    const unsigned long long hit = __ballot(lane < VF_NCH && mass > 0.f && incl > thr);
    const unsigned long long pos = __ballot(lane < VF_NCH && mass > 0.f);
    // past the total by rounding: the last chunk with mass (its scan then
    // finds no crossing and takes its last entry with mass)
    const int ch = hit ? __builtin_ctzll(hit) : pos ? 63 - __builtin_clzll(pos) : -1;
    const float excl = __shfl(incl - mass, ch < 0 ? 0 : ch, 64);
    if (lane == 0) {
      sh_tau = tau;
      sh_ch = ch;
      sh_thr = thr - excl;
      sh_first = 0x7FFFFFFF;
      sh_last = -1;
    }
  }
  __syncthreads();
  const int tau = sh_tau, ch = sh_ch;
  if (ch < 0) {  // nothing to draw from (all mass zero): the last index, as the inverse CDF gives
    if (tid == 0) {
      a.out_len[s] = tau;
      a.out_token[s] = V - 1;
    }
    return;
  }
  const float* pr = P + tau * 8;
  const float mt = pr[0], it = 1.f / pr[1];
  const bool resid = tau < B;
  const float md = resid ? pr[2] : 0.f, id = resid ? 1.f / pr[3] : 0.f;
  const float w = token ? 1.f : pr[6];
  const float* t = a.tlog + ((long long)s * (B + 1) + tau) * V;
  const float* d = a.dlog + ((long long)s * B + (resid ? tau : 0)) * V;
  const int c0 = (int)((long long)V * ch / VF_NCH), c1 = (int)((long long)V * (ch + 1) / VF_NCH);
  const float thr = sh_thr;
  float base = 0.f;
  for (int t0 = c0; t0 < c1; t0 += VD_THREADS * VD_PER) {  // uniform trip count
    const int v0 = t0 + tid * VD_PER;
    float x[VD_PER];
#pragma unroll
    for (int e = 0; e < VD_PER; ++e) {
      const int v = v0 + e;
      float p = 0.f;
      if (v < c1) {
        p = __expf(t[v] * a.inv_temp - mt) * it;
        if (resid) p = fmaxf(w * p - __expf(d[v] * a.inv_temp - md) * id, 0.f);
      }
      x[e] = p;
    }
    float own = 0.f;
#pragma unroll
    for (int e = 0; e < VD_PER; ++e) own += x[e];
    float inc = own;  // inclusive over this wave's threads
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[tid >> 6] = inc;
    __syncthreads();
    float c = base;
    for (int q = 0; q < (tid >> 6); ++q) c += wsum[q];
    float tile = 0.f;
    for (int q = 0; q < VD_THREADS / 64; ++q) tile += wsum[q];
    c += inc - own;  // cumulative mass before this thread's first entry
    // this thread's first entry past the threshold and last entry with mass;
    // the cumulative mass only grows, so the wave's first crossing is its
    // lowest lane's (one LDS atomic per wave)
    int first = 0x7FFFFFFF, last = -1;
#pragma unroll
    for (int e = 0; e < VD_PER; ++e) {
      c += x[e];
      if (x[e] > 0.f) {
        if (c > thr && first == 0x7FFFFFFF) first = v0 + e;
        last = v0 + e;
      }
    }
    const unsigned long long mf = __ballot(first != 0x7FFFFFFF), ml = __ballot(last >= 0);
    if (mf && lane == __builtin_ctzll(mf)) atomicMin(&sh_first, first);
    if (ml && lane == 63 - __builtin_clzll(ml)) atomicMax(&sh_last, last);
    __syncthreads();
    if (sh_first != 0x7FFFFFFF) break;
    base += tile;
  }
  if (tid == 0) {
    a.out_len[s] = tau;
    a.out_token[s] = sh_first != 0x7FFFFFFF ? sh_first : sh_last >= 0 ? sh_last : c1 - 1;
  }
}

}  // namespace

int verify_nch() { return VF_NCH; }

hipError_t launch_verify(const VerifyArgs& a, hipStream_t st) {
  if (a.block < 1 || a.vocab < 1 || a.n_seq < 1) return hipErrorInvalidValue;
  if (a.block > 63) return hipErrorInvalidValue;  // rows 0..block on the lanes of one wave
  hipLaunchKernelGGL(k_verify_norm, dim3(a.n_seq, a.block + 1, VF_NCH), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_verify_probs, dim3(a.n_seq), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_verify_resid, dim3(a.n_seq, a.block, VF_NCH), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_verify_decide, dim3(a.n_seq), dim3(VD_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
