// Attention combine fused with the un-absorb GEMM (o[i,h] = W_UV[h] O[i,h];
// huggingface.co "Kimi-K3-DSpark-NVFP4", "What is quantized to what": kv_b
// is used through absorption), for one sequence of block rows (M <= 8).
//
// One workgroup of 8 waves per head.  Wave w merges row w of the head: lane l
// owns dims 8l .. 8l + 7 and requests the stored Ohat_p = O_p / l_p of every
// slot at once; the slot weights w_p = exp(m_p - M) l_p / sum are computed
// meanwhile (O = sum_p w_p Ohat_p, in slot order).  Those loads are issued
// first, then the head's W_UV tiles are copied into LDS (direct-to-LDS loads),
// so the merge waits only for its own data.  The merged rows become the MFMA
// A operand in LDS (bf16 hi rows 0..7, residual lo rows 8..15), and waves
// 0..3 multiply them by two W_UV tiles each; the GEMM's fragment epilogue
// writes the o_proj input.  This replaces a separate combine kernel whose
// output the un-absorb GEMM then read back.
#include "gemv_impl.h"

namespace dspark {

namespace {

constexpr int UVC_TPW = 2;    // W_UV tiles per GEMM wave (waves 0..3)
constexpr int UVC_CHUNK = 40; // slots whose partials are requested together

template <int KB>
__device__ __forceinline__ void uv_combine(const UvCombineArgs& a, unsigned char* wlds, bf16x8 (*afr)[64]) {
  constexpr int TGMAX = 4 * UVC_TPW;
  const GemvArgs& g = a.g;
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int TG = g.w.TG, M = g.M;
  const int J = a.len1 + a.block;
  const int ns = (J + a.C - 1) / a.C;
  const int m = wave;  // the row this wave merges
  constexpr int NLANE = KB * 4;  // lanes that own 8 dims each (r = 32 KB)
  const bool merge = m < M && lane < NLANE;
  const long long arow = (long long)(m < M ? m : 0) * a.nh + h;  // attention row of (token m, head h)
  // this row's partials; slots past ns fall outside the resource and read zeros
  const __amdgpu_buffer_rsrc_t orow = buf_rsrc(a.o_part + arow * a.slots * a.r, (uint32_t)(ns * a.r * 2));
  const uint32_t ol = 16 * (lane < NLANE ? lane : 0);

  // 1. this thread's partials of the first chunk of slots, then the slot
  //    statistics of this wave's row, then the W_UV copy (issued last, so
  //    the merge does not wait for it)
  u32x4 x[UVC_CHUNK];
#pragma unroll
  for (int u = 0; u < UVC_CHUNK; ++u)
    x[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(orow, ol, u * a.r * 2, 0));
  const float* ml = a.ml_part + arow * a.slots * 2;
  float mp[UVC_MAX_SLOTS / 64], lp[UVC_MAX_SLOTS / 64];
#pragma unroll
  for (int i = 0; i < UVC_MAX_SLOTS / 64; ++i) {
    const int p = lane + 64 * i;
    const bool ok = p < ns;
    mp[i] = ok ? ml[2 * min(p, ns - 1)] : -INFINITY;
    lp[i] = ok ? ml[2 * min(p, ns - 1) + 1] : 0.f;
  }
  {
    // every copy is issued (a head with fewer tiles repeats its last chunk
    // into unused space), so the compiler's wait counts stay exact
    const unsigned char* wsrc = g.w.codes + (long long)h * TG * KB * 1024;
    const int nch = TG * KB;  // 1 KiB chunks
#pragma unroll
    for (int i = 0; i < TGMAX * KB / 8; ++i) {
      const int ch = wave + 8 * i;
      __builtin_amdgcn_global_load_lds(wsrc + min(ch, nch - 1) * 1024 + lane * 16, wlds + ch * 1024, 16, 0, 0);
    }
  }

  // 2. slot weights of row m, kept in this wave's registers (lane p % 64 of
  //    e[p / 64] holds w_p)
  float e[UVC_MAX_SLOTS / 64];
  {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < UVC_MAX_SLOTS / 64; ++i) mx = fmaxf(mx, mp[i]);
    mx = wave_max(mx);
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < UVC_MAX_SLOTS / 64; ++i) {
      e[i] = lp[i] > 0.f ? __expf(mp[i] - mx) * lp[i] : 0.f;
      l += e[i];
    }
    const float inv = m < M ? 1.f / wave_sum(l) : 0.f;
#pragma unroll
    for (int i = 0; i < UVC_MAX_SLOTS / 64; ++i) e[i] *= inv;
  }

  // 3. merged row m, dims 8 lane .. 8 lane + 7, in slot order
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < ns; p0 += UVC_CHUNK) {
    if (p0 > 0) {
#pragma unroll
      for (int u = 0; u < UVC_CHUNK; ++u)
        x[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(orow, ol, (p0 + u) * a.r * 2, 0));
    }
#pragma unroll
    for (int u = 0; u < UVC_CHUNK; ++u) {
      const int p = p0 + u;
      if (p >= ns) break;
      const int i = p >> 6;
      const float ei = i == 0 ? e[0] : i == 1 ? e[1] : i == 2 ? e[2] : e[3];
      static_assert(UVC_MAX_SLOTS == 256, "four weight registers");
      const float wt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ei), p & 63));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] += wt * fp16_bits_to_f32(x[u][e] & 0xFFFFu);
        v[2 * e + 1] += wt * fp16_bits_to_f32(x[u][e] >> 16);
      }
    }
  }
  // A fragments: row m hi at lane q*16 + m, lo at q*16 + 8 + m (rows >= M zero)
  if (lane < NLANE) {
    u32x4 hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a0 = merge ? v[2 * e] : 0.f, a1 = merge ? v[2 * e + 1] : 0.f;
      hi[e] = pack_bf16x2(a0, a1);
      lo[e] = pack_bf16x2(a0 - bf16_bits_to_f32(hi[e] & 0xFFFFu), a1 - bf16_bits_to_f32(hi[e] >> 16));
    }
    const int kb = lane >> 2, q = lane & 3;
    afr[kb][q * 16 + m] = __builtin_bit_cast(bf16x8, hi);
    afr[kb][q * 16 + 8 + m] = __builtin_bit_cast(bf16x8, lo);
  }
  __syncthreads();  // fragments written, every wave's W_UV copies complete

  // 4. waves 0..3: two W_UV tiles each, then the fragment epilogue
  if (wave >= 4) return;
  const int t0 = h * TG + wave * UVC_TPW;
  const bool active = wave * UVC_TPW < TG;
  f32x4 acc[1][UVC_TPW];
#pragma unroll
  for (int j = 0; j < UVC_TPW; ++j) acc[0][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 A = afr[kb][lane];
#pragma unroll
      for (int j = 0; j < UVC_TPW; ++j) {
        const bf16x8 B = *(const bf16x8*)(wlds + (((wave * UVC_TPW + j) * KB + kb) * 64 + lane) * 16);
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[0][j], 0, 0, 0);
      }
    }
  }
  gemv_epilogue<1, UVC_TPW, GEMV_FRAG>(g, acc, active, t0, lane, wave);
}

template <int KB>
__global__ __launch_bounds__(512) void k_uv_combine(UvCombineArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char wlds[4 * UVC_TPW * KB * 1024];  // W_UV tiles of the head
  __shared__ __attribute__((aligned(16))) bf16x8 afr[KB][64];                           // A fragments [k block][lane]
  uv_combine<KB>(a, wlds, afr);
}

}  // namespace

bool uv_combine_supported(const GemvArgs& g, int n_seq, int slots) {
  return n_seq == 1 && g.M <= 8 && g.hilo && g.w.fmt == DT_BF16 && (g.w.KB == 16 || g.w.KB == 2) &&
         g.w.K == 32 * g.w.KB && g.w.TG <= 4 * UVC_TPW && g.w.TG % 2 == 0 && slots <= UVC_MAX_SLOTS;
}

hipError_t launch_uv_combine(const UvCombineArgs& a, hipStream_t st) {
  if (!uv_combine_supported(a.g, 1, a.slots) || a.r != 32 * a.g.w.KB || a.len1 < 0) return hipErrorInvalidValue;
  if (a.g.w.KB == 16)
    hipLaunchKernelGGL(k_uv_combine<16>, dim3(a.g.w.ngroups), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL(k_uv_combine<2>, dim3(a.g.w.ngroups), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
