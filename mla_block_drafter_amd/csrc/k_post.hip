// Column-parallel kernels between the GEMMs of the draft pass.
//
// RMSNorm(x; g) = g * x * rs with one scale rs = 1/sqrt(mean(x^2) + eps) per
// row.  Because rs is a per-row constant it commutes with the next matrix
// product: W (g * x * rs) = rs * (W (g * x)).  So a producer never waits for a
// whole-row reduction: it writes the fragments of g * x for the next GEMM
// plus one partial sum of squares per (row, 256-column chunk); the consumer
// sums the chunks in a fixed order (deterministic) and applies rs to the GEMM
// output.  Every kernel here therefore spreads over column chunks x row
// groups instead of one workgroup per row.
#include "kernels.h"

namespace dspark {

namespace {

// One row per workgroup (blockIdx.y), 256 columns per workgroup (blockIdx.x).

// Row scale of row m (computed by wave 0), broadcast through LDS, in two
// steps: wave 0 requests the chunk sums first, the kernel then issues its own
// loads (split-K partials, inputs), and the scale is formed after them, so the
// two requests share one memory round trip.  The arithmetic is
// row_scale_wave's.
struct RowScaleLoads {
  float t[4];
};
__device__ __forceinline__ RowScaleLoads row_scale_issue(const RowScale& s, int m) {
  RowScaleLoads l{{0.f, 0.f, 0.f, 0.f}};
  if (threadIdx.x < 64 && s.ssq) {
    const float* row = s.ssq + (long long)m * SSQ_LD;
#pragma unroll
    for (int i = 0; i < 4; ++i) l.t[i] = (int)threadIdx.x + 64 * i < s.nch ? row[threadIdx.x + 64 * i] : 0.f;
  }
  return l;
}
__device__ __forceinline__ float row_scale_finish(const RowScale& s, const RowScaleLoads& l, float* slot) {
  if (threadIdx.x < 64) {
    const float v = s.ssq ? rsqrtf(wave_sum((l.t[0] + l.t[1]) + (l.t[2] + l.t[3])) * s.invn + s.eps) : 1.f;
    if (threadIdx.x == 0) *slot = v;
  }
  __syncthreads();
  return *slot;
}

// Sums of the split-K partials of elements (m, c[u]), u < N, columns with
// c[u] < 0 skipped: R splits per column are loaded together (every load of a
// round, all N columns, is in flight at once; the loads are unconditional, at
// clamped in-range addresses, so none waits on a branch), each column summed
// in a fixed order, hence deterministic.
template <int N, int R>
__device__ __forceinline__ void part_sum_r(const PartIn& p, int m, const int (&c)[N], float (&out)[N]) {
  const float* q = p.part + (long long)m * p.ld;
  float v[N][R];
#pragma unroll
  for (int n = 0; n < N; ++n)
#pragma unroll
    for (int u = 0; u < R; ++u) v[n][u] = 0.f;
  for (int s = 0; s < p.S; s += R) {
    float x[N][R];
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
      for (int u = 0; u < R; ++u) x[n][u] = q[(long long)min(s + u, p.S - 1) * p.ss + max(c[n], 0)];
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
      for (int u = 0; u < R; ++u) v[n][u] += (c[n] >= 0 && s + u < p.S) ? x[n][u] : 0.f;
  }
#pragma unroll
  for (int n = 0; n < N; ++n) {
#pragma unroll
    for (int w = R / 2; w >= 1; w >>= 1)
#pragma unroll
      for (int u = 0; u < w; ++u) v[n][u] += v[n][u + w];
    out[n] = v[n][0];
  }
}
// Splits per round: the smallest of 2, 4 and 8 that covers S (8 beyond), so
// that few loads repeat the last split (the fused gate/up GEMM has two
// splits: its SwiGLU post went from 11.1 to 8.5 us per launch at M = 112).
// The sums equal those of eight splits per round: the tree levels that pair
// a split with an absent one add zeros.  (Sixteen per round, one round trip
// for up to 16 splits, measured slower for the q_a / kv_a post.)
template <int N>
__device__ __forceinline__ void part_sum_n(const PartIn& p, int m, const int (&c)[N], float (&out)[N]) {
  if (p.S <= 2) part_sum_r<N, 2>(p, m, c, out);
  else if (p.S <= 4) part_sum_r<N, 4>(p, m, c, out);
  else part_sum_r<N, 8>(p, m, c, out);
}

__device__ __forceinline__ float part_sum(const PartIn& p, int m, int c) {
  const int cc[1] = {c};
  float o[1];
  part_sum_n<1>(p, m, cc, o);
  return o[0];
}

// Rotation of the pair (x0, x1) by the angle whose (cos, sin) is cs.
__device__ __forceinline__ void rope_pair(float x0, float x1, const float* cs, float& y0, float& y1) {
  const float c = cs[0], s = cs[1];
  y0 = x0 * c - x1 * s;
  y1 = x0 * s + x1 * c;
}

// Latent row of activation row m from the split-K partials of its columns
// col0 .. col0 + latent - 1 (scaled by r): c = RMSNorm(first rr columns; g)
// and the rotated rope pairs (cos, sin per pair in cs), written as one row
// at element offset `at` of dst (fp32 or bf16).  All threads of the block.
__device__ __forceinline__ void latent_row(const PartIn& p, int m, int col0, const RowScale& rs_in,
                                           const RowScaleLoads& rl, float* rs_slot, int latent, int rr, int dr,
                                           const float* g, float eps, const float* cs, void* dst, long long at,
                                           int f32, float* red, float* lat) {
  // latent columns k = tid + 256 u (latent <= 1024), all partial loads in flight together
  float s2 = 0.f;
  {
    int cc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) cc[u] = (int)threadIdx.x + 256 * u < latent ? col0 + (int)threadIdx.x + 256 * u : -1;
    float v[4];
    part_sum_n<4>(p, m, cc, v);
    const float r = row_scale_finish(rs_in, rl, rs_slot);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = threadIdx.x + 256 * u;
      if (k >= latent) continue;
      lat[k] = r * v[u];
      if (k < rr) s2 += lat[k] * lat[k];
    }
  }
  const float rc = rsqrtf(block_sum256(s2, red) / rr + eps);  // also orders lat[]
  for (int k = threadIdx.x; k < latent; k += 256) {
    float v;
    if (k < rr) {
      v = g[k] * (lat[k] * rc);
    } else {
      const int e = k - rr, pr = e >> 1;
      float y0, y1;
      rope_pair(lat[rr + 2 * pr], lat[rr + 2 * pr + 1], cs + 2 * pr, y0, y1);
      v = (e & 1) ? y1 : y0;
    }
    if (f32) ((float*)dst)[at + k] = v;
    else ((uint16_t*)dst)[at + k] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// ------------------------------------------------------------- residual --
__global__ __launch_bounds__(256) void k_post_resid(ResidPost a) {
  __shared__ float red[4];
  __shared__ float rs;
  const int m = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  float sq = 0.f, dt = 0.f;
  const bool ok = c < a.H;
  float x = 0.f;
  if (a.mode == RP_NORM) {
    const RowScaleLoads rl = row_scale_issue(a.rs_in, m);
    const float xi = ok ? a.x_in[(long long)m * a.H + c] : 0.f, g0 = ok ? a.g0[c] : 0.f;
    const float r = row_scale_finish(a.rs_in, rl, &rs);
    x = g0 * (xi * r);
  }
  if (ok) {
    const long long i = (long long)m * a.H + c;
    switch (a.mode) {
      case RP_SUM: x = part_sum(a.p, m, c); break;
      case RP_ADD: x = a.x_in[i] + part_sum(a.p, m, c); break;
      case RP_NORM: break;
      default: x = a.x_in[i]; break;
    }
    a.x_out[i] = x;
    sq = x * x;
  }
  if (a.g1) {
    const float v = ok ? a.g1[c] * x : 0.f;
    frag_put_wave(a.fd, 0, m, c, v, ok);
    if (a.dotw && ok) dt = v * a.dotw[c];
  }
  if (a.ssq_out) {
    sq = block_sum256(sq, red);
    if (threadIdx.x == 0) a.ssq_out[m * SSQ_LD + blockIdx.x] = sq;
  }
  if (a.dot_out) {
    dt = block_sum256(dt, red);
    if (threadIdx.x == 0) a.dot_out[m * SSQ_LD + blockIdx.x] = dt;
  }
}

// ------------------------------------------------------ fused q_a / kv_a --
// x-chunks 0..ncq-1: the q_lora columns; chunk ncq: the latent columns of the
// row (kv_a norm over kv_lora, rope of the rope part) -> block keys.
__global__ __launch_bounds__(256) void k_post_qkva(QkvaPost a) {
  __shared__ float red[4];
  __shared__ float rs;
  __shared__ float lat[1024];
  const int m = blockIdx.y;
  const RowScaleLoads rl = row_scale_issue(a.rs_in, m);
  const int ncq = (a.q_lora + 255) / 256;
  if ((int)blockIdx.x < ncq) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    const bool ok = c < a.q_lora;
    const float ps = ok ? part_sum(a.p, m, c) : 0.f;
    const float r = row_scale_finish(a.rs_in, rl, &rs);
    float sq = 0.f, v = 0.f;
    if (ok) {
      v = r * ps;
      sq = v * v;
    }
    frag_put_wave(a.fd_qb, 0, m, c, ok ? a.g_qa[c] * v : 0.f, ok);
    sq = block_sum256(sq, red);
    if (threadIdx.x == 0) a.ssq_cq[m * SSQ_LD + blockIdx.x] = sq;
    return;
  }
  latent_row(a.p, m, a.q_lora, a.rs_in, rl, &rs, a.latent, a.r, a.dr, a.g_kva, a.eps,
             a.rope + (long long)m * (a.dr / 2) * 2, a.bkeys, (long long)m * a.latent, a.kv_f32, red, lat);
}

// ---------------------------------------------------------- cache append --
// One workgroup per new row: its latent row into the cache row slot[m].
__global__ __launch_bounds__(256) void k_post_kv_rows(KvRowPost a) {
  __shared__ float red[4];
  __shared__ float rs;
  __shared__ float lat[1024];
  const int m = blockIdx.x;
  const RowScaleLoads rl = row_scale_issue(a.rs_in, m);
  latent_row(a.p, m, 0, a.rs_in, rl, &rs, a.latent, a.r, a.dr, a.g_kva, a.eps, a.rope + (long long)m * (a.dr / 2) * 2,
             a.dst, a.slot[m] * a.latent, a.dst_f32, red, lat);
}

// ------------------------------------------------------------------ q_b --
// One thread per column pair: nope pairs -> absorb fragments (group = head),
// rope pairs -> rotated into the query buffer.
__global__ __launch_bounds__(256) void k_post_qb(QbPost a) {
  __shared__ float rs;
  const int m = blockIdx.y;
  const RowScaleLoads rl = row_scale_issue(a.rs, m);
  const int hd = a.dn + a.dr;
  const int c0 = 2 * (blockIdx.x * 256 + threadIdx.x);
  const bool live = c0 < a.nh * hd;
  float v[2];
  {
    const int cc[2] = {live ? c0 : -1, live ? c0 + 1 : -1};
    part_sum_n<2>(a.p, m, cc, v);
  }
  const float r = row_scale_finish(a.rs, rl, &rs);  // every thread reaches the barrier
  if (!live) return;
  const int h = c0 / hd, e = c0 % hd;
  const float v0 = r * v[0], v1 = r * v[1];
  if (e < a.dn) {
    frag_put(a.fd_uk, h, m, e, v0);
    frag_put(a.fd_uk, h, m, e + 1, v1);
  } else {
    const int s = m / a.block, i = m % a.block;
    const int er = e - a.dn;
    float y0, y1;
    rope_pair(v0, v1, a.rope + ((long long)m * (a.dr / 2) + (er >> 1)) * 2, y0, y1);
    const long long qi = ((long long)s * a.rows_pad + i * a.nh + h) * a.DQ + a.r + er;
    if (a.q_f32) {
      ((float*)a.q)[qi] = y0;
      ((float*)a.q)[qi + 1] = y1;
    } else {
      ((uint32_t*)a.q)[qi >> 1] = f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
    }
  }
}

// --------------------------------------------------------------- SwiGLU --
__global__ __launch_bounds__(256) void k_post_swiglu(SwigluPost a) {
  __shared__ float rs;
  const int m = blockIdx.y;
  const RowScaleLoads rl = row_scale_issue(a.rs, m);
  const int c = blockIdx.x * 256 + threadIdx.x;
  const bool ok = c < a.inter;
  float gu[2];
  {
    const int cc[2] = {ok ? c : -1, ok ? a.inter + c : -1};
    part_sum_n<2>(a.p, m, cc, gu);
  }
  const float r = row_scale_finish(a.rs, rl, &rs);
  float h = 0.f;
  if (ok) {
    const float g = r * gu[0], u = r * gu[1];
    h = g / (1.f + __expf(-g)) * u;
  }
  frag_put_wave(a.fd, 0, m, c, h, ok);
}

}  // namespace

hipError_t launch_post_resid(const ResidPost& a, hipStream_t st) {
  dim3 grid((a.H + 255) / 256, a.M);
  if (grid.x > SSQ_LD) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_post_resid, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_post_qkva(const QkvaPost& a, hipStream_t st) {
  if (a.latent > 1024 || (a.q_lora + 255) / 256 > SSQ_LD) return hipErrorInvalidValue;
  dim3 grid((a.q_lora + 255) / 256 + 1, a.M);
  hipLaunchKernelGGL(k_post_qkva, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_post_kv_rows(const KvRowPost& a, hipStream_t st) {
  if (a.latent > 1024 || a.M < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_post_kv_rows, dim3(a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_post_qb(const QbPost& a, hipStream_t st) {
  const int pairs = a.nh * (a.dn + a.dr) / 2;
  dim3 grid((pairs + 255) / 256, a.M);
  hipLaunchKernelGGL(k_post_qb, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_post_swiglu(const SwigluPost& a, hipStream_t st) {
  dim3 grid((a.inter + 255) / 256, a.M);
  hipLaunchKernelGGL(k_post_swiglu, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
