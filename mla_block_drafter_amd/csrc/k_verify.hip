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
// Three launches: (1) per (sequence, position, vocabulary chunk) the running
// maximum and sum of exp of the tempered logits (one pass, online); (2) per
// (sequence, position < B, chunk) the residual masses, after every workgroup
// rebuilds the position's normalisers and the prefix weights from (1);
// (3) per sequence the decision and the draw, a chunked scan over the
// vocabulary by one workgroup.
#include "kernels.h"

namespace dspark {

namespace {

constexpr int VF_NCH = 16;  // vocabulary chunks per row in launches 1 and 2

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

// stats layout per (sequence, row): [chunk][4] = target (m, s), draft (m, s)
__global__ __launch_bounds__(256) void k_verify_norm(VerifyArgs a) {
  __shared__ float red[8];
  const int s = blockIdx.x, i = blockIdx.y, ch = blockIdx.z;
  const int B = a.block, V = a.vocab;
  const int c0 = (int)((long long)V * ch / VF_NCH), c1 = (int)((long long)V * (ch + 1) / VF_NCH);
  const float* t = a.tlog + ((long long)s * (B + 1) + i) * V;
  float mt = -INFINITY, st = 0.f, md = -INFINITY, sd = 0.f;
  for (int v = c0 + threadIdx.x; v < c1; v += 256) ms_merge(mt, st, t[v] * a.inv_temp, 1.f);
  block_ms(mt, st, red);
  if (i < B) {
    const float* d = a.dlog + ((long long)s * B + i) * V;
    for (int v = c0 + threadIdx.x; v < c1; v += 256) ms_merge(md, sd, d[v] * a.inv_temp, 1.f);
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

// normalisers of row i of sequence s from the chunk partials
__device__ void row_norm(const VerifyArgs& a, int s, int i, float& mt, float& st, float& md, float& sd) {
  mt = -INFINITY, st = 0.f, md = -INFINITY, sd = 0.f;
  const float* o = a.stats + ((long long)s * (a.block + 1) + i) * VF_NCH * 4;
  for (int c = 0; c < VF_NCH; ++c) {
    ms_merge(mt, st, o[4 * c], o[4 * c + 1]);
    ms_merge(md, sd, o[4 * c + 2], o[4 * c + 3]);
  }
}

// probability of token x at row i under the target (pt) and the draft (pq)
__device__ void gathered(const VerifyArgs& a, int s, int i, float& pt, float& pq) {
  float mt, st, md, sd;
  row_norm(a, s, i, mt, st, md, sd);
  const int x = a.draft[(long long)s * a.block + i];
  const long long V = a.vocab;
  if (x < 0 || x >= V) {  // not a token: the target never emits it, so it is rejected
    pt = 0.f;
    pq = 1.f;
    return;
  }
  pt = __expf(a.tlog[((long long)s * (a.block + 1) + i) * V + x] * a.inv_temp - mt) / st;
  pq = __expf(a.dlog[((long long)s * a.block + i) * V + x] * a.inv_temp - md) / sd;
}

// prefix weight w_k of the block rule
__device__ float prefix_weight(const VerifyArgs& a, int s, int k) {
  float w = 1.f;
  for (int j = 0; j < k; ++j) {
    float pt, pq;
    gathered(a, s, j, pt, pq);
    w = fminf(w * pt / pq, 1.f);
  }
  return w;
}

// residual masses at position i < B, chunk ch: token rule (w = 1) and block rule (w = w_i)
__global__ __launch_bounds__(256) void k_verify_resid(VerifyArgs a) {
  __shared__ float red[4];
  __shared__ float sh[5];
  const int s = blockIdx.x, i = blockIdx.y, ch = blockIdx.z;
  const int B = a.block, V = a.vocab;
  if (threadIdx.x == 0) {
    float mt, st, md, sd;
    row_norm(a, s, i, mt, st, md, sd);
    sh[0] = mt;
    sh[1] = st;
    sh[2] = md;
    sh[3] = sd;
    sh[4] = prefix_weight(a, s, i);
  }
  __syncthreads();
  const float mt = sh[0], it = 1.f / sh[1], md = sh[2], id = 1.f / sh[3], w = sh[4];
  const int c0 = (int)((long long)V * ch / VF_NCH), c1 = (int)((long long)V * (ch + 1) / VF_NCH);
  const float* t = a.tlog + ((long long)s * (B + 1) + i) * V;
  const float* d = a.dlog + ((long long)s * B + i) * V;
  float rt = 0.f, rb = 0.f;
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

// decision and draw, one workgroup of 1024 threads per sequence
__global__ __launch_bounds__(1024) void k_verify_decide(VerifyArgs a) {
  __shared__ int sh_tau;
  __shared__ float sh_w, sh_mt, sh_it, sh_md, sh_id, sh_tot;
  __shared__ float part[1024];
  __shared__ int sh_hit;
  const int s = blockIdx.x, B = a.block, V = a.vocab;
  const float* r = a.u + (long long)s * (B + 1);
  if (threadIdx.x == 0) {
    int tau = 0;
    float w = 1.f;
    if (a.method == DSPARK_VERIFY_TOKEN_C) {
      tau = B;
      for (int i = 0; i < B; ++i) {
        float pt, pq;
        gathered(a, s, i, pt, pq);
        if (!(r[i] < fminf(1.f, pt / pq))) {
          tau = i;
          break;
        }
      }
    } else {
      for (int k = 1; k <= B; ++k) {
        float pt, pq;
        gathered(a, s, k - 1, pt, pq);
        w = fminf(w * pt / pq, 1.f);
        float h = w;
        if (k < B) {
          float S = 0.f;
          for (int c = 0; c < VF_NCH; ++c) S += a.resid[(((long long)s * B + k) * VF_NCH + c) * 2 + 1];
          h = S + 1.f - w > 0.f ? S / (S + 1.f - w) : 1.f;
        }
        if (r[k - 1] < h) tau = k;
      }
      w = prefix_weight(a, s, tau);
    }
    float mt, st, md, sd;
    row_norm(a, s, tau, mt, st, md, sd);
    sh_tau = tau;
    sh_w = a.method == DSPARK_VERIFY_TOKEN_C ? 1.f : w;
    sh_mt = mt;
    sh_it = 1.f / st;
    sh_md = md;
    sh_id = 1.f / sd;
  }
  __syncthreads();
  const int tau = sh_tau;
  const bool resid = tau < B;
  const float* t = a.tlog + ((long long)s * (B + 1) + tau) * V;
  const float* d = a.dlog + ((long long)s * B + (resid ? tau : 0)) * V;
  auto weight = [&](int v) {
    const float p = __expf(t[v] * a.inv_temp - sh_mt) * sh_it;
    if (!resid) return p;
    return fmaxf(sh_w * p - __expf(d[v] * a.inv_temp - sh_md) * sh_id, 0.f);
  };
  // chunk masses (contiguous chunks, one per thread), exclusive scan, then
  // the chunk holding the threshold walks its entries in order
  const int per = (V + 1023) / 1024;
  const int v0 = threadIdx.x * per, v1 = min(V, v0 + per);
  float cm = 0.f;
  for (int v = v0; v < v1; ++v) cm += weight(v);
  part[threadIdx.x] = cm;
  __syncthreads();
  if (threadIdx.x == 0) {
    float acc = 0.f;
    for (int c = 0; c < 1024; ++c) {
      const float x = part[c];
      part[c] = acc;
      acc += x;
    }
    sh_tot = acc;
    sh_hit = -1;
  }
  __syncthreads();
  const float thr = a.u[(long long)s * (B + 1) + B] * sh_tot;
  const float base = part[threadIdx.x];
  if (base <= thr && thr < base + cm) sh_hit = threadIdx.x;  // at most one chunk (masses >= 0)
  __syncthreads();
  if ((int)threadIdx.x == sh_hit) {
    float c = base;
    int y = v1 - 1;
    for (int v = v0; v < v1; ++v) {
      c += weight(v);
      if (c > thr) {
        y = v;
        break;
      }
    }
    a.out_token[s] = y;
  }
  if (threadIdx.x == 0) {
    a.out_len[s] = tau;
    if (sh_hit < 0) a.out_token[s] = V - 1;  // rounding put the threshold past the total mass
  }
}

}  // namespace

int verify_nch() { return VF_NCH; }

hipError_t launch_verify(const VerifyArgs& a, hipStream_t st) {
  if (a.block < 1 || a.vocab < 1 || a.n_seq < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_verify_norm, dim3(a.n_seq, a.block + 1, VF_NCH), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_verify_resid, dim3(a.n_seq, a.block, VF_NCH), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_verify_decide, dim3(a.n_seq), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
