// Small kernels of the draft pass: workspace init and fc input fragments, the
// Markov finaliser (tokens, confidence, hidden output), acceptance length, and
// weight repack / decode.
#include "gemv_impl.h"

namespace dspark {

namespace {

// ------------------------------------------------------------------ init --
__global__ __launch_bounds__(256) void k_init(InitArgs a) {
  const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long nthr = (long long)gridDim.x * 256;
  u32x4* z = (u32x4*)a.zero_ptr;
  const long long n16 = a.zero_bytes / 16;
  for (long long i = tid; i < n16; i += nthr) z[i] = u32x4{0u, 0u, 0u, 0u};
  if (a.rope) {
    // angles in float64 (positions reach 2^20 and more), stored as fp32 pairs
    const long long nr = (long long)a.n_seq * a.block * a.npairs;
    for (long long e = tid; e < nr; e += nthr) {
      const int m = (int)(e / a.npairs), p = (int)(e % a.npairs);
      const int s = m / a.block, i = m % a.block;
      double sn, cs;
      const long long pos = a.positions ? (long long)a.positions[m] : (long long)(a.offs[s + 1] - a.offs[s] + i);
      sincos((double)pos * a.freqs[p], &sn, &cs);
      a.rope[2 * e] = (float)cs;
      a.rope[2 * e + 1] = (float)sn;
    }
  }
  if (!a.captured) return;
  // fc input: row m = s*block + i, column k = c*H + h of captured[s][c][i][h];
  // every element of the fragment buffer is written (zeros outside M x K).
  const FragDesc& fd = a.fd_fc;
  const int M = a.n_seq * a.block;
  const int K = a.ncap * a.H;
  const int Kp = fd.rows ? K : fd.f32 ? fd.KG * 16 : fd.KB * 32;
  const int rows = fd.rows ? M : (fd.hilo || fd.i8) ? 8 : fd.MT * 16;
  if (!fd.rows && !fd.f32 && a.H % 8 == 0) {
    // bf16 / int8 fragments keep eight consecutive columns of a row together:
    // one thread per (row, 8 columns), one 8- or 16-byte store per code row.
    // K8 is a multiple of 4 and the thread count of 64, so each quad of lanes
    // holds one 32-column block of one row (its int8 scale: a quad maximum).
    const int K8 = Kp / 8;
    const long long total8 = (long long)rows * K8;
    const bool al16 = ((uintptr_t)a.captured & 15) == 0;  // idx is a multiple of 8
    for (long long e = tid; e < total8; e += nthr) {
      const int m = (int)(e / K8), k0 = (int)(e % K8) * 8;
      float v[8];
      const bool in = m < M && k0 < K;
      const int s = m / a.block, i = m % a.block, c = k0 / a.H, h = k0 % a.H;
      const long long idx = in ? (((long long)s * a.ncap + c) * a.block + i) * a.H + h : 0;
      if (!in) {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = 0.f;
      } else if (al16 && a.cap_f32) {
        const f32x4 x0 = *(const f32x4*)((const float*)a.captured + idx);
        const f32x4 x1 = *(const f32x4*)((const float*)a.captured + idx + 4);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[u] = x0[u];
          v[4 + u] = x1[u];
        }
      } else if (al16) {
        const u32x4 x = *(const u32x4*)((const uint16_t*)a.captured + idx);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[2 * u] = bf16_bits_to_f32(x[u] & 0xFFFFu);
          v[2 * u + 1] = bf16_bits_to_f32(x[u] >> 16);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = a.cap_f32 ? ((const float*)a.captured)[idx + u]
                           : bf16_bits_to_f32(((const uint16_t*)a.captured)[idx + u]);
      }
      if (fd.i8) {
        float bm = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) bm = fmaxf(bm, fabsf(v[u]));
        bm = fmaxf(bm, dpp_mov<DPP_XOR1>(bm));
        bm = fmaxf(bm, dpp_mov<DPP_XOR2>(bm));
        frag_put_i8_x8(fd, 0, m, k0, v, frag_i8_exp(bm));
      } else {
        const int kb = k0 >> 5, q = (k0 >> 3) & 3;
        uint16_t* p = (uint16_t*)fd.ptr;
        u32x4 hw, lw;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t h0 = f32_to_bf16_bits(v[2 * u]), h1 = f32_to_bf16_bits(v[2 * u + 1]);
          hw[u] = h0 | (h1 << 16);
          lw[u] = f32_to_bf16_bits(v[2 * u] - bf16_bits_to_f32(h0)) |
                  (f32_to_bf16_bits(v[2 * u + 1] - bf16_bits_to_f32(h1)) << 16);
        }
        if (fd.hilo) {
          *(u32x4*)(p + ((long long)kb * 64 + q * 16 + m) * 8) = hw;
          *(u32x4*)(p + ((long long)kb * 64 + q * 16 + 8 + m) * 8) = lw;
        } else {
          const int mt = m >> 4;
          *(u32x4*)(p + ((long long)(mt * fd.KB + kb) * 64 + q * 16 + (m & 15)) * 8) = hw;
        }
      }
    }
    return;
  }
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
    // int8 fragments: Kp and the thread count are multiples of 64, so every
    // wave walks whole 64-column runs of one row together
    frag_put_wave(fd, 0, m, k, v, true);
  }
}

// ------------------------------------------------------------ Markov final --
// Tokens from the argmax keys, confidence sigmoid(w_h . hf_i + w_m . u_i + b)
// with hf_i = rs_final * g_final * x, and the optional hidden output.
__global__ __launch_bounds__(256) void k_markov_final(MarkovFinalArgs a) {
  if (a.fallback && *a.fallback == 0) return;  // the candidate rollout wrote tokens and confidences
  __shared__ float red[4];
  __shared__ unsigned long long kred[4];
  const int s = blockIdx.x, i = blockIdx.y;  // one workgroup per (sequence, position)
  const long long m = (long long)s * a.block + i;
  // argmax key of position pos (all threads take part)
  auto token_at = [&](int pos) {
    unsigned long long best = 0;
    if (a.slots) {
      const unsigned long long* sl = a.slots + ((long long)pos * a.n_seq + s) * a.nwg;
      for (int w = threadIdx.x; w < a.nwg; w += 256) best = best > sl[w] ? best : sl[w];
    } else if (threadIdx.x < KEY_SLOTS) {
      best = a.keys[((long long)s * a.block + pos) * KEY_SLOTS + threadIdx.x];
    }
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long other = ((unsigned long long)__shfl_xor((unsigned)(best >> 32), o, 64) << 32) |
                                       (unsigned)__shfl_xor((unsigned)best, o, 64);
      best = best > other ? best : other;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) kred[threadIdx.x >> 6] = best;
    __syncthreads();
    for (int q = 0; q < 4; ++q) best = best > kred[q] ? best : kred[q];
    return key_index(best);
  };
  const bool failed = a.rollout_err && *a.rollout_err;
  int tp;
  if (i == 0) tp = a.prev_token[s];
  else if (a.forced) tp = a.forced[s * a.block + i - 1];
  else tp = token_at(i - 1);
  const int ti = token_at(i);
  // every wave computes the row scale and the dot-chunk sum (same bits in all)
  const float rs = row_scale_wave(a.rs_final, (int)m);
  const float hd = chunk_sum_wave(a.dot + m * SSQ_LD, a.nch);
  if (a.hidden)
    for (int k = threadIdx.x; k < a.H; k += 256) a.hidden[m * a.H + k] = a.g_final[k] * a.x[m * a.H + k] * rs;
  float d = 0.f;
  if (tp >= 0 && tp < a.vocab) {
    for (int k = threadIdx.x; k < a.R; k += 256) {
      const long long idx = (long long)tp * a.w1_ld + k;
      const float u = a.w1_f32 ? ((const float*)a.w1)[idx] : bf16_bits_to_f32(((const uint16_t*)a.w1)[idx]);
      d += u * a.conf_wm[k];
    }
  }
  d = block_sum256(d, red);
  if (a.status && s == 0 && i == 0 && threadIdx.x == 0) *a.status = failed ? 1 : 0;
  if (threadIdx.x == 0) {
    a.tokens[m] = failed ? -1 : ti;
    const float x = rs * hd + d + a.conf_b[0];
    a.conf[m] = 1.f / (1.f + __expf(-x));
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
  if (w.fmt == DT_MXFP4)  // byte holding element k (low nibble when k is even)
    return (((long long)tile * (w.KB >> 2) + (kb >> 2)) * 64 + q * 16 + r16) * 16 + (kb & 3) * 4 + (i >> 1);
  return (((long long)tile * (w.KB >> 1) + (kb >> 1)) * 64 + q * 16 + r16) * 16 + (kb & 1) * 8 + i;
}

// Byte offset of the E8M0 scale code of (tile, row r16, k block kb).
__device__ __forceinline__ long long mx_scale_offset(const PackedMat& w, int tile, int r16, int kb) {
  return (((long long)tile * (w.KB >> 2) + (kb >> 2)) * 16 + r16) * 4 + (kb & 3);
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
  if (a.src_fmt == DT_MXFP4) {  // whole bytes (element pairs) and the block's scale code
    const unsigned char* blk = (const unsigned char*)a.src + (long long)lr * (a.src_cols / 32 * 17) + kb * 17;
    int tile, r16;
    for (int kk = 0; kk < 32; kk += 2) {
      const long long off = code_offset(a.dst, n, kb * 32 + kk, tile, r16);
      a.codes[off] = blk[1 + kk / 2];
    }
    code_offset(a.dst, n, kb * 32, tile, r16);
    ((unsigned char*)a.scales)[mx_scale_offset(a.dst, tile, r16, kb)] = blk[0];
    return;
  }
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
      } else if (w.fmt == DT_MXFP4) {
        const uint32_t c = *(const uint32_t*)(w.codes + off);
        const uint32_t sw = ((const uint32_t*)w.scales)[((long long)tile * (w.KB >> 2) + (kb >> 2)) * 16 + r16];
        const int j = kb & 3;
        b = fp4x8_to_bf16x8(c, j == 0 ? e8m0_f32<0>(sw) : j == 1 ? e8m0_f32<1>(sw) : j == 2 ? e8m0_f32<2>(sw)
                                                                                            : e8m0_f32<3>(sw));
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

// Streaming read laid out as the weight-streaming GEMMs read: each wave owns
// one contiguous range of 1 KiB chunks (64 lanes x 16 bytes) and keeps eight
// chunks in flight with non-temporal buffer loads (loads past the buffer
// return zeros without a memory access); each workgroup folds what it read
// into one XOR word.
__global__ __launch_bounds__(256) void k_read_probe(const unsigned char* p, long long bytes, uint32_t* out) {
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long nchunk = (bytes + 1023) / 1024, nw = (long long)gridDim.x * 4;
  const long long per = (nchunk + nw - 1) / nw, c0 = min(nchunk, ((long long)blockIdx.x * 4 + wave) * per);
  const long long c1 = min(nchunk, c0 + per);
  const long long rbytes = max(0ll, min(bytes - c0 * 1024, (c1 - c0) * 1024));  // 0 for waves past the data
  const __amdgpu_buffer_rsrc_t r = buf_rsrc(p + c0 * 1024, (uint32_t)rbytes);
  u32x4 x = {0u, 0u, 0u, 0u};
  for (long long c = 0; c < c1 - c0; c += 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, c + u < c1 - c0 ? (uint32_t)((c + u) * 1024 + lane * 16) : BUF_OOB, 0, BUF_NT));
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u];
  }
  uint32_t v = x[0] ^ x[1] ^ x[2] ^ x[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v ^= (uint32_t)__shfl_xor((int)v, o, 64);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t st) {
  if (bytes / 1024 / (READ_PROBE_WGS * 4) >= (1ll << 22)) return hipErrorInvalidValue;  // a wave's range < 4 GiB
  hipLaunchKernelGGL(k_read_probe, dim3(READ_PROBE_WGS), dim3(256), 0, st, (const unsigned char*)buf, (long long)bytes, out);
  return hipGetLastError();
}

hipError_t launch_init(const InitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_init, dim3(512), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_markov_final(const MarkovFinalArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_markov_final, dim3(a.n_seq, a.block), dim3(256), 0, st, a);
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
