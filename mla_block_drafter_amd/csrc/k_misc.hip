// Row-wise kernels of the draft pass: split-K reduction + residual + RMSNorm,
// q/kv norms and (YaRN) rope, fragment writers for the next GEMM, the Markov
// finaliser (tokens, confidence), acceptance length, weight repack / decode.
//
// RMSNorm: g * x / sqrt(mean(x^2) + eps) in fp32.  RoPE rotates consecutive
// pairs (2k, 2k+1) by pos * theta'_k, with theta'_k precomputed on the host in
// fp64 (YaRN NTK-by-parts) and the angle reduced and evaluated in fp64.
#include "kernels.h"

namespace dspark {

namespace {

// ------------------------------------------------------------------ init --
__global__ __launch_bounds__(256) void k_init(InitArgs a) {
  const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long nthr = (long long)gridDim.x * 256;
  u32x4* z = (u32x4*)a.zero_ptr;
  const long long n16 = a.zero_bytes / 16;
  for (long long i = tid; i < n16; i += nthr) z[i] = u32x4{0u, 0u, 0u, 0u};
  if (!a.captured) return;
  // fc input: row m = s*block + i, column k = c*H + h of captured[s][c][i][h];
  // every element of the fragment buffer is written (zeros outside M x K).
  const FragDesc& fd = a.fd_fc;
  const int M = a.n_seq * a.block;
  const int K = a.ncap * a.H;
  const int Kp = fd.f32 ? fd.KG * 16 : fd.KB * 32;
  const int rows = fd.hilo ? 8 : fd.MT * 16;
  const long long total = (long long)rows * Kp;
  for (long long e = tid; e < total; e += nthr) {
    const int m = (int)(e / Kp), k = (int)(e % Kp);
    float v = 0.f;
    if (m < M && k < K) {
      const int s = m / a.block, i = m % a.block, c = k / a.H, h = k % a.H;
      const long long idx = (((long long)s * a.ncap + c) * a.block + i) * a.H + h;
      v = a.cap_f32 ? ((const float*)a.captured)[idx]
                    : bf16_bits_to_f32(((const uint16_t*)a.captured)[idx]);
    }
    frag_put(fd, 0, m, k, v);
  }
}

// ------------------------------------------------------------- residual --
__global__ __launch_bounds__(256) void k_resid_norm(ResidArgs a) {
  extern __shared__ float xs[];  // H floats
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int H = a.H;
  float ss = 0.f;
  for (int k = threadIdx.x; k < H; k += 256) {
    float v;
    if (a.mode == RESID_COPY) {
      v = a.x_in[(long long)m * H + k];
    } else {
      float sum = 0.f;
      for (int sp = 0; sp < a.S; ++sp) sum += a.part[sp * a.part_ss + (long long)m * a.part_ld + k];
      v = a.mode == RESID_ADD ? a.x_in[(long long)m * H + k] + sum : sum;
    }
    xs[k] = v;
    ss += v * v;
  }
  if (a.mode == RESID_NORM_FIRST) {
    const float tot = block_sum256(ss, red);
    const float rs = rsqrtf(tot / H + a.eps);
    ss = 0.f;
    for (int k = threadIdx.x; k < H; k += 256) {
      const float v = a.g0[k] * (xs[k] * rs);
      xs[k] = v;
      ss += v * v;
    }
  }
  for (int k = threadIdx.x; k < H; k += 256) a.x_out[(long long)m * H + k] = xs[k];
  if (!a.g1) return;
  const float tot = block_sum256(ss, red);
  const float rs = rsqrtf(tot / H + a.eps);
  float dot = 0.f;
  for (int k = threadIdx.x; k < H; k += 256) {
    const float v = a.g1[k] * (xs[k] * rs);
    if (a.fd.ptr) frag_put(a.fd, 0, m, k, v);
    if (a.hidden_out) a.hidden_out[(long long)m * H + k] = v;
    if (a.conf_wh) dot += v * a.conf_wh[k];
  }
  if (a.conf_wh) {
    dot = block_sum256(dot, red);
    if (threadIdx.x == 0) a.hconf[m] = dot;
  }
}

__device__ __forceinline__ void rope_pair(float x0, float x1, double pos, double f, float& y0, float& y1) {
  double sn, cs;
  sincos(pos * f, &sn, &cs);
  const float c = (float)cs, s = (float)sn;
  y0 = x0 * c - x1 * s;
  y1 = x0 * s + x1 * c;
}

// --------------------------------------------------- fused q_a / kv_a post --
__global__ __launch_bounds__(256) void k_qkva_post(QkvaArgs a) {
  extern __shared__ float buf[];  // q_lora + latent
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int N = a.q_lora + a.latent;
  for (int k = threadIdx.x; k < N; k += 256) {
    float sum = 0.f;
    for (int sp = 0; sp < a.S; ++sp) sum += a.part[sp * a.part_ss + (long long)m * a.part_ld + k];
    buf[k] = sum;
  }
  __syncthreads();
  float sq = 0.f, sc = 0.f;
  for (int k = threadIdx.x; k < a.q_lora; k += 256) sq += buf[k] * buf[k];
  for (int k = threadIdx.x; k < a.r; k += 256) sc += buf[a.q_lora + k] * buf[a.q_lora + k];
  const float rq = rsqrtf(block_sum256(sq, red) / a.q_lora + a.eps);
  const float rc = rsqrtf(block_sum256(sc, red) / a.r + a.eps);
  for (int k = threadIdx.x; k < a.q_lora; k += 256) frag_put(a.fd_qb, 0, m, k, a.g_qa[k] * (buf[k] * rq));
  const int s = m / a.block, i = m % a.block;
  const double pos = (double)(a.offs[s + 1] - a.offs[s] + i);
  const long long ob = (long long)m * a.latent;
  for (int k = threadIdx.x; k < a.latent; k += 256) {
    float v;
    if (k < a.r) {
      v = a.g_kva[k] * (buf[a.q_lora + k] * rc);
    } else {
      const int e = k - a.r, pr = e >> 1;
      float y0, y1;
      rope_pair(buf[a.q_lora + a.r + 2 * pr], buf[a.q_lora + a.r + 2 * pr + 1], pos, a.freqs[pr], y0, y1);
      v = (e & 1) ? y1 : y0;
    }
    if (a.kv_f32) ((float*)a.bkeys)[ob + k] = v;
    else ((uint16_t*)a.bkeys)[ob + k] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// ------------------------------------------------------------- q_b post --
__global__ __launch_bounds__(256) void k_qb_post(QbArgs a) {
  const int m = blockIdx.x;
  const int s = m / a.block, i = m % a.block;
  const double pos = (double)(a.offs[s + 1] - a.offs[s] + i);
  const int hd = a.dn + a.dr;
  const int N = a.nh * hd;
  for (int k = threadIdx.x; k < N; k += 256) {
    const int h = k / hd, e = k % hd;
    auto val = [&](int kk) {
      float sum = 0.f;
      for (int sp = 0; sp < a.S; ++sp) sum += a.part[sp * a.part_ss + (long long)m * a.part_ld + kk];
      return sum;
    };
    if (e < a.dn) {
      frag_put(a.fd_uk, h, m, e, val(k));
    } else {
      const int er = e - a.dn, pr = er >> 1;
      const int kb = h * hd + a.dn + 2 * pr;
      float y0, y1;
      rope_pair(val(kb), val(kb + 1), pos, a.freqs[pr], y0, y1);
      const float v = (er & 1) ? y1 : y0;
      const long long qi = ((long long)s * a.rows_pad + i * a.nh + h) * a.DQ + a.r + er;
      if (a.q_f32) ((float*)a.q)[qi] = v;
      else ((uint16_t*)a.q)[qi] = (uint16_t)f32_to_bf16_bits(v);
    }
  }
}

// ------------------------------------------------------------ absorb post --
__global__ __launch_bounds__(256) void k_absorb_post(AbsorbArgs a) {
  const int m = blockIdx.x;
  const int s = m / a.block, i = m % a.block;
  const int N = a.nh * a.r;
  for (int k = threadIdx.x; k < N; k += 256) {
    const int h = k / a.r, c = k % a.r;
    const float v = a.part[(long long)m * a.part_ld + k];
    const long long qi = ((long long)s * a.rows_pad + i * a.nh + h) * a.DQ + c;
    if (a.q_f32) ((float*)a.q)[qi] = v;
    else ((uint16_t*)a.q)[qi] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// ------------------------------------------------------ plain / SwiGLU copy --
__global__ __launch_bounds__(256) void k_to_frag(FragArgs a) {
  const int m = blockIdx.x;
  for (int k = threadIdx.x; k < a.K; k += 256) {
    float v = 0.f, u = 0.f;
    for (int sp = 0; sp < a.S; ++sp) {
      const float* p = a.part + sp * a.part_ss + (long long)m * a.part_ld;
      v += p[k];
      if (a.swiglu) u += p[a.K + k];
    }
    if (a.swiglu) v = v / (1.f + __expf(-v)) * u;
    frag_put(a.fd, 0, m, k, v);
  }
}

// ------------------------------------------------------------ Markov final --
__global__ __launch_bounds__(256) void k_markov_final(MarkovFinalArgs a) {
  __shared__ float red[4];
  __shared__ int toks[64];
  const int s = blockIdx.x;
  if (threadIdx.x < a.block) {
    const unsigned long long* k = a.keys + ((long long)s * a.block + threadIdx.x) * KEY_SLOTS;
    unsigned long long best = 0;
    for (int i = 0; i < KEY_SLOTS; ++i) best = best > k[i] ? best : k[i];
    toks[threadIdx.x] = key_index(best);
    a.tokens[s * a.block + threadIdx.x] = key_index(best);
  }
  __syncthreads();
  for (int i = 0; i < a.block; ++i) {
    int tp;
    if (i == 0) tp = a.prev_token[s];
    else tp = a.forced ? a.forced[s * a.block + i - 1] : toks[i - 1];
    float d = 0.f;
    if (tp >= 0 && tp < a.vocab) {
      for (int k = threadIdx.x; k < a.R; k += 256) {
        const long long idx = (long long)tp * a.w1_ld + k;
        const float u = a.w1_f32 ? ((const float*)a.w1)[idx] : bf16_bits_to_f32(((const uint16_t*)a.w1)[idx]);
        d += u * a.conf_wm[k];
      }
    }
    d = block_sum256(d, red);
    if (threadIdx.x == 0) {
      const float x = a.hconf[s * a.block + i] + d + a.conf_b[0];
      a.conf[s * a.block + i] = 1.f / (1.f + __expf(-x));
    }
  }
}

// ------------------------------------------------------------ acceptance --
__global__ void k_accept(const int32_t* d, const int32_t* v, int n_seq, int block, int32_t* out) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_seq) return;
  int k = 0;
  while (k < block && d[(long long)s * block + k] == v[(long long)s * block + k]) ++k;
  out[s] = k;
}

// ---------------------------------------------------------------- repack --
// Destination logical row n and column k -> packed byte offset of the code.
__device__ __forceinline__ long long code_offset(const PackedMat& w, int n, int k, int& tile, int& r16) {
  const int g = n / w.G, j = n % w.G;
  tile = g * w.TG + j / 16;
  r16 = j % 16;
  if (w.fmt == DT_F32) {
    const int grp = k >> 4, q = (k >> 2) & 3, i = k & 3;
    return (((long long)tile * (w.Kp >> 4) + grp) * 64 + q * 16 + r16) * 16 + i * 4;
  }
  const int kb = k >> 5, q = (k >> 3) & 3, i = k & 7;
  if (w.fmt == DT_BF16) return (((long long)tile * w.KB + kb) * 64 + q * 16 + r16) * 16 + i * 2;
  return (((long long)tile * (w.KB >> 1) + (kb >> 1)) * 64 + q * 16 + r16) * 16 + (kb & 1) * 8 + i;
}

// One thread per (destination row, 32-wide k block).
__global__ __launch_bounds__(256) void k_repack(RepackArgs a) {
  const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  const int K = a.dst.K;
  const int nkb = (K + 31) / 32;
  if (id >= (long long)a.nrows * nkb) return;
  const int lr = (int)(id / nkb), kb = (int)(id % nkb);
  int n;  // destination logical row
  if (a.xf == XF_NORMAL) n = a.row0 + lr;
  else n = lr;
  for (int kk = 0; kk < 32; ++kk) {
    const int k = kb * 32 + kk;
    if (k >= K) break;
    long long sr, sc;  // source row / column
    if (a.xf == XF_NORMAL) { sr = lr; sc = k; }
    else if (a.xf == XF_UK) {  // row (h, c), col d  <-  kv_b[h*(dn+dv) + d][c]
      const int h = n / a.r, c = n % a.r;
      sr = (long long)h * (a.dn + a.dv) + k; sc = c;
    } else {                   // row (h, v), col c  <-  kv_b[h*(dn+dv) + dn + v][c]
      const int h = n / a.dv, v = n % a.dv;
      sr = (long long)h * (a.dn + a.dv) + a.dn + v; sc = k;
    }
    int tile, r16;
    const long long off = code_offset(a.dst, n, k, tile, r16);
    switch (a.src_fmt) {
      case DT_F32:
        *(float*)(a.codes + off) = ((const float*)a.src)[sr * a.src_cols + sc];
        break;
      case DT_BF16:
        *(uint16_t*)(a.codes + off) = ((const uint16_t*)a.src)[sr * a.src_cols + sc];
        break;
      case DT_FP8:
        a.codes[off] = ((const unsigned char*)a.src)[sr * a.src_cols + sc];
        break;
      case DT_Q8_0: {
        const unsigned char* blk = (const unsigned char*)a.src + sr * (a.src_cols / 32 * 34) + (sc / 32) * 34;
        a.codes[off] = blk[2 + (sc % 32)];
        break;
      }
    }
  }
  int tile, r16;
  code_offset(a.dst, n, kb * 32, tile, r16);
  if (a.src_fmt == DT_Q8_0) {
    const unsigned char* blk = (const unsigned char*)a.src + (long long)lr * (a.src_cols / 32 * 34) + kb * 34;
    const uint16_t d = (uint16_t)(blk[0] | (blk[1] << 8));
    uint16_t* sp = (uint16_t*)a.scales;
    sp[(((long long)tile * (a.dst.KB >> 1) + (kb >> 1)) * 16 + r16) * 2 + (kb & 1)] = d;
  } else if (a.src_fmt == DT_FP8 && kb == 0) {
    ((float*)a.scales)[(long long)tile * 16 + r16] = a.src_scales[lr];
  }
}

// Decode the packed matrix back to [rows][K] floats with the GEMM's decoders.
__global__ __launch_bounds__(256) void k_dequant(PackedMat w, float* out) {
  const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long rows = (long long)w.ngroups * w.G;
  const int nkb = w.Kp / 32;
  if (id >= rows * nkb) return;
  const int n = (int)(id / nkb), kb = (int)(id % nkb);
  for (int q = 0; q < 4; ++q) {  // 8 elements at a time, as one lane of the GEMM reads them
    const int k0 = kb * 32 + q * 8;
    if (k0 >= w.K) break;
    int tile, r16;
    const long long off = code_offset(w, n, k0, tile, r16);
    float v[8];
    if (w.fmt == DT_F32) {
      for (int i = 0; i < 8; ++i) {
        const long long o2 = code_offset(w, n, k0 + i, tile, r16);
        v[i] = *(const float*)(w.codes + o2);
      }
    } else {
      bf16x8 b;
      float sc = 1.f;
      if (w.fmt == DT_BF16) {
        b = *(const bf16x8*)(w.codes + off);
      } else {
        const u32x2 c = *(const u32x2*)(w.codes + off);
        if (w.fmt == DT_Q8_0) {
          b = i8x8_to_bf16x8(c[0], c[1]);
          const uint32_t s2 = ((const uint32_t*)w.scales)[((long long)tile * (w.KB >> 1) + (kb >> 1)) * 16 + r16];
          sc = fp16_bits_to_f32((kb & 1) ? (s2 >> 16) : (s2 & 0xFFFFu));
        } else {
          b = fp8x8_to_bf16x8(c[0], c[1]);
          sc = ((const float*)w.scales)[(long long)tile * 16 + r16];
        }
      }
      for (int i = 0; i < 8; ++i) v[i] = (float)b[i] * sc;
    }
    for (int i = 0; i < 8; ++i)
      if (k0 + i < w.K) out[(long long)n * w.K + k0 + i] = v[i];
  }
}

}  // namespace

hipError_t launch_init(const InitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_init, dim3(512), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_resid_norm(const ResidArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_resid_norm, dim3(a.M), dim3(256), a.H * sizeof(float), st, a);
  return hipGetLastError();
}

hipError_t launch_qkva_post(const QkvaArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_qkva_post, dim3(a.M), dim3(256), (a.q_lora + a.latent) * sizeof(float), st, a);
  return hipGetLastError();
}

hipError_t launch_qb_post(const QbArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_qb_post, dim3(a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_absorb_post(const AbsorbArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_absorb_post, dim3(a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_to_frag(const FragArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_to_frag, dim3(a.M), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_markov_final(const MarkovFinalArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_markov_final, dim3(a.n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_accept_len(const int32_t* d, const int32_t* v, int n_seq, int block, int32_t* out,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_accept, dim3((n_seq + 255) / 256), dim3(256), 0, st, d, v, n_seq, block, out);
  return hipGetLastError();
}

hipError_t launch_repack(const RepackArgs& a, hipStream_t st) {
  const long long n = (long long)a.nrows * ((a.dst.K + 31) / 32);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_repack, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dequant(const PackedMat& w, float* out, hipStream_t st) {
  const long long n = (long long)w.ngroups * w.G * (w.Kp / 32);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, w, out);
  return hipGetLastError();
}

}  // namespace dspark
