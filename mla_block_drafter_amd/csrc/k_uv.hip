// Attention combine fused with the un-absorb GEMM (o[i,h] = W_UV[h] O[i,h];
// huggingface.co "Kimi-K3-DSpark-NVFP4", "What is quantized to what": kv_b
// is used through absorption), for one sequence of block rows (M <= 8).
//
// One workgroup of 8 waves per (head, pair of block rows): the merge reads
// each row's partials once, and splitting the rows spreads those reads over
// four times as many CUs (a CU's own load path, not HBM, bounds this step);
// the head's 128 KiB of W_UV is read by the four workgroups of the head,
// which sit on one XCD, so it leaves HBM once.
//
// Wave w < 2 merges row 2 part + w: lane l owns dims 8l .. 8l + 7 and
// requests the stored Ohat_p = O_p / l_p of every slot at once; the slot
// weights w_p = exp(m_p - max) l_p / sum are computed while those loads are
// in flight, and each slot is added as soon as its data is there (in slot
// order: O = sum_p w_p Ohat_p).  Waves 2..7 meanwhile copy the head's W_UV
// tiles into LDS (direct-to-LDS loads).  The merged rows become
// the MFMA A operand in LDS (bf16 hi rows, residual lo rows 8 apart); wave w
// multiplies them by W_UV tile w, the outputs go through LDS, and 128 threads
// write the o_proj input fragments, eight columns each.  This replaces a
// separate combine kernel whose output the un-absorb GEMM then read back.
#include "gemv_impl.h"

namespace dspark {

namespace {

constexpr int UVC_TILES = 8;   // W_UV tiles per head at most (one per wave)
constexpr int UVC_CHUNK = 40;  // slots whose partials are requested together
constexpr int UVC_OLD = UVC_TILES * 16 + 4;  // LDS row stride of the GEMM outputs
constexpr int UVC_RPW = 2;     // block rows per workgroup
// A fragments in LDS: 16 bytes per (k block, lane), one pad unit after every
// 16 lanes, so that the writes of one row (lanes q 16 + w over the k blocks)
// spread over the banks; the MFMA reads of 16 consecutive lanes stay
// contiguous.
constexpr int UVC_AKB = 68;    // 16-byte units per k block
__device__ __forceinline__ int afr_pos(int kb, int l) { return kb * UVC_AKB + (l >> 4) * 17 + (l & 15); }

// Slot U of the first chunk (weight in lane U of e0), then the next slot:
// each waits only for its own partials (issued in slot order, NAFTER more
// operations issued after the chunk).
template <int U, int NU, int NAFTER>
__device__ __forceinline__ void merge_chunk0(float (&v)[8], const u32x4 (&x)[NU], float e0) {
  if constexpr (U < NU) {
    vm_wait<NU - 1 - U + NAFTER>();
    const float wt = lane_value(e0, U);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] += wt * fp16_bits_to_f32(x[U][q] & 0xFFFFu);
      v[2 * q + 1] += wt * fp16_bits_to_f32(x[U][q] >> 16);
    }
    merge_chunk0<U + 1, NU, NAFTER>(v, x, e0);
  }
}

template <int KB>
__device__ __forceinline__ void uv_combine(const UvCombineArgs& a, unsigned char* wlds, bf16x8* afr,
                                           float (*olds)[UVC_OLD]) {
  constexpr int NCOPYW = 8 - UVC_RPW;        // waves that copy W_UV
  constexpr int NCH = UVC_TILES * KB;        // 1 KiB chunks of W_UV space in LDS
  constexpr int NCOPY = (NCH + NCOPYW - 1) / NCOPYW;  // copies per copying wave
  constexpr int NW = UVC_MAX_SLOTS / 64;
  const GemvArgs& g = a.g;
  // workgroup (part, head): rows UVC_RPW part .. + UVC_RPW - 1 of head h; the
  // parts of a head are 64 workgroups apart (a multiple of 8: same XCD, so
  // the head's W_UV is read from HBM once and then from that XCD's L2)
  const int h = blockIdx.x % g.w.ngroups, part = blockIdx.x / g.w.ngroups;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int TG = g.w.TG;
  const int row0 = part * UVC_RPW, nrows = min(UVC_RPW, g.M - row0);
  const int J = a.len1 + a.block;
  const int ns = (J + a.C - 1) / a.C;
  const int m = row0 + wave;  // the row this wave merges (waves < nrows)
  constexpr int NLANE = KB * 4;  // lanes that own 8 dims each (r = 32 KB)

  if (wave < nrows) {
    const long long arow = (long long)m * a.nh + h;  // attention row of (token m, head h)
    // this row's partials and slot statistics; slots past ns fall outside
    // the resources and read zeros
    const __amdgpu_buffer_rsrc_t orow = buf_rsrc(a.o_part + arow * a.slots * a.r, (uint32_t)(ns * a.r * 2));
    const __amdgpu_buffer_rsrc_t mlr = buf_rsrc(a.ml_part + arow * a.slots * 2, (uint32_t)(ns * 8));
    const uint32_t ol = 16 * (lane < NLANE ? lane : 0);

    // 1. loads in the order they are needed (vector memory counts complete
    //    in issue order): the slot statistics (m, l), then this thread's
    //    partials of the first chunk of slots.  The other waves copy W_UV
    //    meanwhile.
    u32x2 mlv[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i)
      mlv[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(mlr, (uint32_t)(lane + 64 * i) * 8, 0, 0));
    u32x4 x[UVC_CHUNK];
#pragma unroll
    for (int u = 0; u < UVC_CHUNK; ++u) {
      x[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(orow, ol, u * a.r * 2, 0));
      __builtin_amdgcn_sched_barrier(0);  // keep the issue order (the waits count on it)
    }

    // 2. slot weights of row m, kept in this wave's registers (lane p % 64
    //    of e[p / 64] holds w_p)
    vm_wait<UVC_CHUNK>();
    float e[NW];
    {
      float mp[NW], lp[NW];
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        lp[i] = __uint_as_float(mlv[i][1]);
        mp[i] = lp[i] > 0.f ? __uint_as_float(mlv[i][0]) : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < NW; ++i) mx = fmaxf(mx, mp[i]);
      mx = wave_max(mx);
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        e[i] = lp[i] > 0.f ? __expf(mp[i] - mx) * lp[i] : 0.f;
        l += e[i];
      }
      const float inv = 1.f / wave_sum(l);
#pragma unroll
      for (int i = 0; i < NW; ++i) e[i] *= inv;
    }

    // 3. merged row m, dims 8 lane .. 8 lane + 7, in slot order.  The first
    //    chunk consumes slot u as soon as its load is complete; slots past ns
    //    read zeros and have weight zero, so they add nothing.
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    static_assert(UVC_CHUNK <= 64, "first chunk weights in e[0]");
    merge_chunk0<0, UVC_CHUNK, 0>(v, x, e[0]);
    for (int p0 = UVC_CHUNK; p0 < ns; p0 += UVC_CHUNK) {
#pragma unroll
      for (int u = 0; u < UVC_CHUNK; ++u)
        x[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(orow, ol, (p0 + u) * a.r * 2, 0));
#pragma unroll
      for (int u = 0; u < UVC_CHUNK; ++u) {
        const int p = p0 + u;
        if (p >= ns) break;
        const int i = p >> 6;
        const float ei = i == 0 ? e[0] : i == 1 ? e[1] : i == 2 ? e[2] : e[3];
        static_assert(UVC_MAX_SLOTS == 256, "four weight registers");
        const float wt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ei), p & 63));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] += wt * fp16_bits_to_f32(x[u][q] & 0xFFFFu);
          v[2 * q + 1] += wt * fp16_bits_to_f32(x[u][q] >> 16);
        }
      }
    }
    // A fragments: local row w hi at lane q*16 + w, lo at q*16 + 8 + w
    if (lane < NLANE) {
      u32x4 hi, lo;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hi[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
        lo[q] = pack_bf16x2(v[2 * q] - bf16_bits_to_f32(hi[q] & 0xFFFFu), v[2 * q + 1] - bf16_bits_to_f32(hi[q] >> 16));
      }
      const int kb = lane >> 2, q = lane & 3;
      afr[afr_pos(kb, q * 16 + wave)] = __builtin_bit_cast(bf16x8, hi);
      afr[afr_pos(kb, q * 16 + 8 + wave)] = __builtin_bit_cast(bf16x8, lo);
    }
  } else if (wave < UVC_RPW) {
    // no row for this wave: its fragment rows are zero
    if (lane < NLANE) {
      const int kb = lane >> 2, q = lane & 3;
      const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      afr[afr_pos(kb, q * 16 + wave)] = z;
      afr[afr_pos(kb, q * 16 + 8 + wave)] = z;
    }
  } else {
    // the head's W_UV tiles into LDS; fragment rows UVC_RPW..7 are zero.
    // Every copy is issued: chunks past the head's tiles repeat its last
    // chunk (into unused space, or onto the copy of that same chunk).
    if (lane < NLANE) {
      const int kb = lane >> 2, q = lane & 3;
      const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      afr[afr_pos(kb, q * 16 + wave)] = z;
      afr[afr_pos(kb, q * 16 + 8 + wave)] = z;
    }
    const unsigned char* wsrc = g.w.codes + (long long)h * TG * KB * 1024;
    const int nch = TG * KB;
#pragma unroll
    for (int i = 0; i < NCOPY; ++i) {
      const int ch = min(wave - UVC_RPW + NCOPYW * i, NCH - 1);
      __builtin_amdgcn_global_load_lds(wsrc + min(ch, nch - 1) * 1024 + lane * 16, wlds + ch * 1024, 16, 0, 0);
    }
  }
  vm_wait<0>();
  __syncthreads();  // fragments written, every wave's W_UV copies complete

  // 4. wave w: W_UV tile w (16 outputs of the head), all K
  if (wave < TG) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 A = afr[afr_pos(kb, lane)];
      const bf16x8 B = *(const bf16x8*)(wlds + ((wave * KB + kb) * 64 + lane) * 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc, 0, 0, 0);
    }
    // D row 4 (lane >> 4) + r (hi rows 0..7, lo rows 8..15), column lane & 15
#pragma unroll
    for (int r = 0; r < 4; ++r) olds[4 * (lane >> 4) + r][wave * 16 + (lane & 15)] = acc[r];
  }
  __syncthreads();

  // 5. o_proj input fragments: thread (w, kb, q) writes columns 32 kb + 8 q ..
  //    + 7 of local row w (hi + lo sum); for int8 fragments the quad of a
  //    32-block shares its maximum
  const int t = threadIdx.x;
  if (t < 128) {
    const int q = t & 3, kb = (t >> 2) & 3, mr = t >> 4;
    const int c0 = kb * 32 + q * 8;
    const bool ok = mr < nrows && c0 < TG * 16;
    float y[8];
    float bm = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y[i] = ok ? olds[mr][c0 + i] + olds[8 + mr][c0 + i] : 0.f;
      bm = fmaxf(bm, fabsf(y[i]));
    }
    bm = fmaxf(bm, dpp_mov<DPP_XOR1>(bm));
    bm = fmaxf(bm, dpp_mov<DPP_XOR2>(bm));
    if (ok) {
      if (g.fd.i8) {
        frag_put_i8_x8(g.fd, 0, row0 + mr, h * g.w.G + c0, y, frag_i8_exp(bm));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) frag_put(g.fd, 0, row0 + mr, h * g.w.G + c0 + i, y[i]);
      }
    }
  }
}

template <int KB>
__global__ __launch_bounds__(512) void k_uv_combine(UvCombineArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char wlds[UVC_TILES * KB * 1024];  // W_UV tiles of the head
  __shared__ __attribute__((aligned(16))) bf16x8 afr[KB * UVC_AKB];                    // A fragments (afr_pos)
  __shared__ float olds[16][UVC_OLD];                                                  // GEMM outputs
  uv_combine<KB>(a, wlds, afr, olds);
}

}  // namespace

bool uv_combine_supported(const GemvArgs& g, int n_seq, int slots) {
  return n_seq == 1 && g.M >= 1 && g.M <= 8 && g.hilo && g.w.fmt == DT_BF16 && (g.w.KB == 16 || g.w.KB == 2) &&
         g.w.K == 32 * g.w.KB && g.w.TG <= UVC_TILES && g.w.TG % 2 == 0 && g.w.G == 16 * g.w.TG &&
         g.w.G % 32 == 0 && slots <= UVC_MAX_SLOTS && !g.rs.ssq && !g.fd.rows;
}

hipError_t launch_uv_combine(const UvCombineArgs& a, hipStream_t st) {
  if (!uv_combine_supported(a.g, 1, a.slots) || a.r != 32 * a.g.w.KB || a.len1 < 0) return hipErrorInvalidValue;
  const int parts = (a.g.M + UVC_RPW - 1) / UVC_RPW;
  const dim3 grid(a.g.w.ngroups * parts);
  if (a.g.w.KB == 16)
    hipLaunchKernelGGL(k_uv_combine<16>, grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL(k_uv_combine<2>, grid, dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
