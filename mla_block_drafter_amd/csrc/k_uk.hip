// q_b post fused with the absorb GEMM (huggingface.co "Kimi-K3-DSpark-NVFP4",
// "Model Overview": MLA with the k_nope half of kv_b absorbed into the query,
// q_lat[i,h] = W_UK[h]^T q_nope[i,h]), for M <= 8 block rows.
//
// q = rs_cq * (sum of the q_b split-K partials); per head h the 128 nope
// columns become the MFMA A operand (bf16 hi rows 0..7, residual lo rows
// 8..15) in LDS, and the first workgroup of the head writes the rotated rope
// columns into the query buffer.  Each workgroup multiplies by 8 tiles (128
// outputs) of the head's W_UK and writes q_lat into the query buffer.  The
// W_UK tiles are requested first, so the partial sums overlap their latency.
// This replaces a separate kernel that wrote the nope fragments to memory for
// the GEMM to read back.
#include "gemv_impl.h"

namespace dspark {

namespace {

constexpr int QBA_TPW = 2;  // W_UK tiles per wave
constexpr int QBA_KB = 4;   // k blocks of 32 (qk_nope = 128)
constexpr int QBA_NI = 3;   // column pairs per thread: M (dn + dr) / 2 <= 768
// A fragments in LDS: 16 bytes per (k block, lane), one pad unit after every
// 16 lanes, so that the 4-byte writes of one row's columns (consecutive
// threads: consecutive column pairs) fall on distinct banks; the MFMA reads
// of 16 consecutive lanes stay contiguous.
constexpr int QBA_AKB = 68;  // 16-byte units per k block
__device__ __forceinline__ int qba_pos(int kb, int l) { return kb * QBA_AKB + (l >> 4) * 17 + (l & 15); }

__global__ __launch_bounds__(256) void k_qb_absorb(QbAbsorbArgs a) {
  __shared__ __attribute__((aligned(16))) u32x4 afr[QBA_KB * QBA_AKB];  // A fragments (qba_pos)
  const GemvArgs& g = a.g;
  const QbPost& p = a.qb;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int TG = g.w.TG, M = g.M;
  const int wph = (TG + 4 * QBA_TPW - 1) / (4 * QBA_TPW);  // workgroups per head
  const int h = blockIdx.x / wph, quarter = blockIdx.x % wph;
  const int tl0 = (quarter * 4 + wave) * QBA_TPW;  // first tile of this wave within the head
  const bool active = tl0 < TG;
  const int t0 = h * TG + tl0;

  // 1. this wave's W_UK tiles, all k blocks
  u32x4 w[QBA_KB][QBA_TPW];
  {
    const __amdgpu_buffer_rsrc_t wr = buf_rsrc(g.w.codes + (long long)(active ? t0 : 0) * QBA_KB * 1024,
                                               active ? (uint32_t)(QBA_TPW * QBA_KB * 1024) : 0u);
#pragma unroll
    for (int kb = 0; kb < QBA_KB; ++kb)
#pragma unroll
      for (int j = 0; j < QBA_TPW; ++j)
        w[kb][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
            wr, (uint32_t)((j * QBA_KB + kb) * 1024 + lane * 16), 0, BUF_NT));
  }

  // 2. the chunk sums of cq^2 of every row, requested together (each wave
  //    computes all row scales itself, in the order row_scale_wave uses)
  float ck[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float* r = p.rs.ssq + (long long)min(m, M - 1) * SSQ_LD;
    const float c0 = r[min(lane, p.rs.nch - 1)], c1 = r[min(lane + 64, p.rs.nch - 1)];  // unconditional loads
    ck[m] = (lane < p.rs.nch ? c0 : 0.f) + (lane + 64 < p.rs.nch ? c1 : 0.f);
  }

  // 3. the head's columns: thread item it -> (row m, column pair e, e + 1);
  //    the rope pairs only in the head's first workgroup.  All split loads of
  //    a round (8 splits x 2 columns x QBA_NI items) are in flight together.
  const int hd = p.dn + p.dr;
  const int npair = (quarter == 0 ? hd : p.dn) / 2;
  const int nitem = M * npair;
  int im[QBA_NI], ie[QBA_NI];
  bool iok[QBA_NI];
#pragma unroll
  for (int k = 0; k < QBA_NI; ++k) {
    const int it = threadIdx.x + 256 * k;
    iok[k] = it < nitem;
    const int itc = iok[k] ? it : 0;
    im[k] = itc / npair;
    ie[k] = 2 * (itc % npair);
  }
  float acc2[QBA_NI][2][8];
#pragma unroll
  for (int k = 0; k < QBA_NI; ++k)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int u = 0; u < 8; ++u) acc2[k][c][u] = 0.f;
  for (int s0 = 0; s0 < p.p.S; s0 += 8) {
    float x[QBA_NI][2][8];
#pragma unroll
    for (int k = 0; k < QBA_NI; ++k)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* q = p.p.part + (long long)im[k] * p.p.ld + (long long)min(s0 + u, p.p.S - 1) * p.p.ss +
                         (long long)h * hd + ie[k];
        x[k][0][u] = q[0];
        x[k][1][u] = q[1];
      }
#pragma unroll
    for (int k = 0; k < QBA_NI; ++k)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int u = 0; u < 8; ++u) acc2[k][c][u] += s0 + u < p.p.S ? x[k][c][u] : 0.f;
  }
  float rsm[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) rsm[m] = rsqrtf(wave_sum(ck[m]) * p.rs.invn + p.rs.eps);
  // fragment rows M..7 are zero (entries no item writes)
  for (int i = threadIdx.x; i < QBA_KB * 4 * 8; i += 256) {
    const int row = i & 7, q = (i >> 3) & 3, kb = i >> 5;
    if (row >= M) {
      afr[qba_pos(kb, q * 16 + row)] = u32x4{0u, 0u, 0u, 0u};
      afr[qba_pos(kb, q * 16 + 8 + row)] = u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int k = 0; k < QBA_NI; ++k) {
    if (!iok[k]) continue;
    const int mk = im[k];
    float rk = rsm[0];
#pragma unroll
    for (int m = 1; m < 8; ++m) rk = mk == m ? rsm[m] : rk;
    float v[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float* t = acc2[k][c];
      v[c] = rk * (((t[0] + t[4]) + (t[2] + t[6])) + ((t[1] + t[5]) + (t[3] + t[7])));
    }
    const int m = im[k], e = ie[k];
    if (e < p.dn) {
      // A fragment: k = e -> block e / 32, lane (e / 8 % 4) * 16 + row, word (e % 8) / 2
      const uint32_t hi = pack_bf16x2(v[0], v[1]);
      const uint32_t lo = pack_bf16x2(v[0] - bf16_bits_to_f32(hi & 0xFFFFu), v[1] - bf16_bits_to_f32(hi >> 16));
      const int kb = e >> 5, q = (e >> 3) & 3, wd = (e & 7) >> 1;
      ((uint32_t*)&afr[qba_pos(kb, q * 16 + m)])[wd] = hi;
      ((uint32_t*)&afr[qba_pos(kb, q * 16 + 8 + m)])[wd] = lo;
    } else {
      const int s = m / p.block, i = m % p.block, er = e - p.dn;
      float y0, y1;
      const float* cs = p.rope + ((long long)m * (p.dr / 2) + (er >> 1)) * 2;
      y0 = v[0] * cs[0] - v[1] * cs[1];
      y1 = v[0] * cs[1] + v[1] * cs[0];
      const long long qi = ((long long)s * p.rows_pad + i * p.nh + h) * p.DQ + p.r + er;
      if (p.q_f32) {
        ((float*)p.q)[qi] = y0;
        ((float*)p.q)[qi + 1] = y1;
      } else {
        ((uint32_t*)p.q)[qi >> 1] = f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
      }
    }
  }
  __syncthreads();

  // 4. the GEMM over all k blocks, then the query-buffer epilogue
  f32x4 acc[1][QBA_TPW];
#pragma unroll
  for (int j = 0; j < QBA_TPW; ++j) acc[0][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < QBA_KB; ++kb) {
    const bf16x8 A = __builtin_bit_cast(bf16x8, afr[qba_pos(kb, lane)]);
#pragma unroll
    for (int j = 0; j < QBA_TPW; ++j)
      acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, w[kb][j]), acc[0][j], 0, 0, 0);
  }
  gemv_epilogue<1, QBA_TPW, GEMV_QLAT>(g, acc, active, t0, lane, wave);
}

}  // namespace

bool qb_absorb_supported(const GemvArgs& g, const QbPost& p) {
  return g.M >= 1 && g.M <= 8 && g.hilo && g.w.fmt == DT_BF16 && g.w.KB == QBA_KB && g.w.K == 32 * QBA_KB &&
         p.dn == 32 * QBA_KB && p.dr % 2 == 0 && g.w.TG % QBA_TPW == 0 && g.w.G == 16 * g.w.TG &&
         g.w.ngroups == p.nh && p.M == g.M && g.M * (p.dn + p.dr) / 2 <= 256 * QBA_NI && !g.rs.ssq && p.rs.ssq;
}

hipError_t launch_qb_absorb(const QbAbsorbArgs& a, hipStream_t st) {
  if (!qb_absorb_supported(a.g, a.qb)) return hipErrorInvalidValue;
  const int wph = (a.g.w.TG + 4 * QBA_TPW - 1) / (4 * QBA_TPW);
  hipLaunchKernelGGL(k_qb_absorb, dim3(a.g.w.ngroups * wph), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
