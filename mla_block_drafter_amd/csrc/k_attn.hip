// Absorbed MLA attention of the draft block over the latent cache.
//
// Every query row (token i, head h) of a sequence attends, without a mask
// (non-causal block, huggingface.co card "Model Overview"), to all of that
// sequence's cache rows plus the block's own 7 latent rows.  With kv_b
// absorbed, query row = [q_lat (kv_lora) | q_pe (qk_rope)] and key row =
// the stored latent [c_kv | k_pe]; the value is c_kv itself.  All 64 x 7
// query rows share one 576-element key row, so the product is dense:
// ~846 flop per key byte, above the MI355X bf16 ridge, hence MFMA.
//
// bf16 path (split-K, flash-decoding style): a workgroup of 4 waves owns 64
// query rows and one slot of C keys.  Key tiles of 32 rows are staged in LDS
// row-major.  S^T = K Q^T takes the key rows as the A operand (16-byte LDS
// reads), so the probabilities land with one query row per lane column,
// which is already the B-operand layout of P^T for O^T = V^T P^T: the
// probabilities never leave registers (the 32 keys' order inside the MFMA
// reduction is permuted identically on both operands).  The V^T operand is
// gathered from the same row-major tile with 2-byte LDS reads (the value is
// c_kv, the first kv_lora columns of the key row), so no transposed copy is
// staged.  Online softmax state (m, l) is per lane column.  Partials per slot
// are merged by k_attn_combine in a fixed order.
#include "kernels.h"

namespace dspark {

namespace {

constexpr int KT = 32;  // keys per LDS tile
constexpr int MAX_COMBINE_SLOTS = 4096;

__device__ __forceinline__ void slot_lookup(const AttnArgs& a, int slot, int& s, int& p, int& len,
                                            int& off, int& J) {
  int base = 0;
  for (s = 0; s < a.n_seq; ++s) {
    off = a.offs[s];
    len = a.offs[s + 1] - off;
    J = len + a.block;
    const int ns = (J + a.C - 1) / a.C;
    if (slot < base + ns) {
      p = slot - base;
      return;
    }
    base += ns;
  }
  s = -1;
}

template <int NKB, int NDT>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(AttnArgs a) {
  constexpr int DQ = NKB * 32;
  constexpr int R = NDT * 16;
  constexpr int KLD = DQ + 8;   // padded LDS row (elements), 16-byte aligned rows
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[KT * KLD];

  int s, p, len, off, J;
  slot_lookup(a, blockIdx.y, s, p, len, off, J);
  if (s < 0) return;  // uniform over the workgroup
  const int k_begin = p * a.C;
  const int k_end = min(J, k_begin + a.C);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * 64 + wave * 16;
  const int myrow = row0 + (lane & 15);

  // Q fragments (B operand of S^T = K Q^T): row myrow, dims 32kb + 8(lane>>4).
  bf16x8 qf[NKB];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((long long)s * a.rows_pad + myrow) * DQ + 8 * (lane >> 4);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) qf[kb] = *(const bf16x8*)(qrow + 32 * kb);
  }

  f32x4 acc[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* cache = (const uint16_t*)a.cache;
  const uint16_t* bk = (const uint16_t*)a.bkeys;
  constexpr int CHUNKS_PER_KEY = DQ / 8;

  for (int kt0 = k_begin; kt0 < k_end; kt0 += KT) {
    // ---- stage the key tile (row-major) and its transpose (value part) ----
    for (int c = threadIdx.x; c < KT * CHUNKS_PER_KEY; c += 256) {
      const int kk = c / CHUNKS_PER_KEY, d8 = (c % CHUNKS_PER_KEY) * 8;
      const int j = kt0 + kk;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (j < k_end && d8 < a.latent) {
        const uint16_t* src = j < len ? cache + (long long)(off + j) * a.latent + d8
                                      : bk + (long long)(s * a.block + (j - len)) * a.latent + d8;
        v = *(const u32x4*)src;
      }
      *(u32x4*)(k_lds + kk * KLD + d8) = v;
    }
    __syncthreads();

    // ---- S^T for 32 keys x 16 rows: two 16-key MFMA tiles ----
    f32x4 st[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = k_lds + (16 * h + (lane & 15)) * KLD + 8 * (lane >> 4);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(krow + 32 * kb);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kb], c, 0, 0, 0);
      }
      st[h] = c;
    }
    // lane holds keys kt0 + 16h + 4(lane>>4) + r for query row myrow
    float tmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kt0 + 16 * h + 4 * (lane >> 4) + r;
        const float v = j < k_end ? st[h][r] * a.tau : -INFINITY;
        st[h][r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float corr = m_new == -INFINITY ? 1.f : __expf(m_run - m_new);
    float psum = 0.f;
    u32x4 pw;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = m_new == -INFINITY ? 0.f : __expf(st[h][r] - m_new);
        psum += pr[r];
      }
      pw[2 * h] = f32_to_bf16_bits(pr[0]) | (f32_to_bf16_bits(pr[1]) << 16);
      pw[2 * h + 1] = f32_to_bf16_bits(pr[2]) | (f32_to_bf16_bits(pr[3]) << 16);
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * corr + psum;
    m_run = m_new;
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);

    // ---- O^T += V^T P^T: lane's k slots map to keys 4(lane>>4)+{0..3} and
    //      16 + 4(lane>>4) + {0..3}, matching the P fragment above; the A
    //      operand holds V[key][dim = 16d + (lane & 15)] for those keys ----
    const uint16_t* vbase = k_lds + 4 * (lane >> 4) * KLD + (lane & 15);
#pragma unroll
    for (int d = 0; d < NDT; ++d) {
      const uint16_t* vcol = vbase + 16 * d;
      u32x4 vv;
      vv[0] = (uint32_t)vcol[0] | ((uint32_t)vcol[KLD] << 16);
      vv[1] = (uint32_t)vcol[2 * KLD] | ((uint32_t)vcol[3 * KLD] << 16);
      vv[2] = (uint32_t)vcol[16 * KLD] | ((uint32_t)vcol[17 * KLD] << 16);
      vv[3] = (uint32_t)vcol[18 * KLD] | ((uint32_t)vcol[19 * KLD] << 16);
      acc[d] *= corr;
      acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, acc[d], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- partials: O^T[dim = 16d + 4(lane>>4) + r][row = myrow]; layout
  //      [row][slot][dim] so the combine of one row reads contiguous memory ----
  const long long prow = (long long)myrow * a.slots + blockIdx.y;
  float* op = a.o_part + prow * a.r + 4 * (lane >> 4);
#pragma unroll
  for (int d = 0; d < NDT; ++d) *(f32x4*)(op + 16 * d) = acc[d];
  if ((lane >> 4) == 0) {
    a.ml_part[prow * 2] = m_run;
    a.ml_part[prow * 2 + 1] = l_run;
  }
}

// Merge the slots of each (sequence, row) in slot order and write the
// un-absorb fragments: O = sum_p exp(m_p - M) O_p / sum_p exp(m_p - M) l_p.
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
  __shared__ float wgt[MAX_COMBINE_SLOTS];
  __shared__ float red[4];
  const int row = blockIdx.x;  // i * nh + h
  const int s = blockIdx.y;
  if (row >= a.rows) return;
  int base = 0;
  for (int t = 0; t < s; ++t) {
    const int J = a.offs[t + 1] - a.offs[t] + a.block;
    base += (J + a.C - 1) / a.C;
  }
  const int J = a.offs[s + 1] - a.offs[s] + a.block;
  const int ns = (J + a.C - 1) / a.C;
  const float* ml = a.ml_part + ((long long)row * a.slots + base) * 2;
  float mx = -INFINITY;
  for (int p = threadIdx.x; p < ns; p += 256) mx = fmaxf(mx, ml[2 * p]);
  mx = block_max256(mx, red);
  float l = 0.f;
  for (int p = threadIdx.x; p < ns; p += 256) {
    const float w = __expf(ml[2 * p] - mx);
    wgt[p] = w;
    l += ml[2 * p + 1] * w;
  }
  l = block_sum256(l, red);  // also orders the wgt writes before the reads below
  const float invL = 1.f / l;
  const int i = row / a.nh, h = row % a.nh;
  const int m = s * a.block + i;
  const float* op = a.o_part + ((long long)row * a.slots + base) * a.r;
  for (int d = threadIdx.x; d < a.r; d += 256) {
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int p = 0;
    for (; p + 8 <= ns; p += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] += wgt[p + u] * op[(long long)(p + u) * a.r + d];
    }
    for (; p < ns; ++p) o[0] += wgt[p] * op[(long long)p * a.r + d];
    const float t = ((o[0] + o[1]) + (o[2] + o[3])) + ((o[4] + o[5]) + (o[6] + o[7]));
    frag_put(a.fd_uv, h, m, d, t * invL);
  }
}

// fp32 path (small all-fp32 configurations): one workgroup per (row, sequence),
// keys in chunks of 256 with online softmax; writes the un-absorb fragments.
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  __shared__ float qs[1024];
  __shared__ float ps[256];
  __shared__ float red[4];
  const int row = blockIdx.x, s = blockIdx.y;
  if (row >= a.rows) return;
  const int off = a.offs[s], len = a.offs[s + 1] - off, J = len + a.block;
  const float* q = (const float*)a.q + ((long long)s * a.rows_pad + row) * a.DQ;
  for (int d = threadIdx.x; d < a.latent; d += 256) qs[d] = q[d];
  __syncthreads();
  const float* cache = (const float*)a.cache;
  const float* bk = (const float*)a.bkeys;
  auto keyrow = [&](int j) -> const float* {
    return j < len ? cache + (long long)(off + j) * a.latent
                   : bk + (long long)(s * a.block + (j - len)) * a.latent;
  };
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  for (int c0 = 0; c0 < J; c0 += 256) {
    const int j = c0 + threadIdx.x;
    float sc = -INFINITY;
    if (j < J) {
      const float* kr = keyrow(j);
      float acc = 0.f;
      for (int d = 0; d < a.latent; ++d) acc += qs[d] * kr[d];
      sc = acc * a.tau;
    }
    const float cmax = block_max256(sc, red);
    const float m_new = fmaxf(m_run, cmax);
    const float corr = __expf(m_run - m_new);
    const float pj = j < J ? __expf(sc - m_new) : 0.f;
    ps[threadIdx.x] = pj;
    const float csum = block_sum256(pj, red);
    l_run = l_run * corr + csum;
    m_run = m_new;
    const int nk = min(256, J - c0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = threadIdx.x + 256 * u;
      if (d >= a.r) continue;
      float acc = o[u] * corr;
      for (int t = 0; t < nk; ++t) acc += ps[t] * keyrow(c0 + t)[d];
      o[u] = acc;
    }
    __syncthreads();
  }
  const int i = row / a.nh, h = row % a.nh;
  const int m = s * a.block + i;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = threadIdx.x + 256 * u;
    if (d < a.r) frag_put(a.fd_uv, h, m, d, o[u] / l_run);
  }
}

}  // namespace

bool attn_bf16_supported(int DQ, int r) {
  return (DQ == 576 && r == 512) || (DQ == 96 && r == 64);
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.rows_pad / 64, a.slots), block(256);
  if (a.DQ == 576 && a.r == 512)
    hipLaunchKernelGGL((k_attn_bf16<18, 32>), grid, block, 0, st, a);
  else if (a.DQ == 96 && a.r == 64)
    hipLaunchKernelGGL((k_attn_bf16<3, 4>), grid, block, 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t st) {
  if (a.slots > MAX_COMBINE_SLOTS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_combine, dim3(a.rows, a.n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st) {
  if (a.latent > 1024 || a.r > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_f32, dim3(a.rows, a.n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
