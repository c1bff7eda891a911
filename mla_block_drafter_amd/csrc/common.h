// Shared device-side definitions of the DSpark draft-pass library (gfx950).
//
// Data layouts in HBM (all owned by the caller; see include/dspark.h):
//
//  Packed weight matrix [N][K] (logical rows n, reduction index k), padded to
//  16-row tiles and Kp = round_up(K, 64):
//   * BF16:   one 1 KiB chunk per (tile t, 32-wide k block kb), chunk index
//             t*KB + kb; lane l of a wave owns 16 bytes = 8 bf16 of row
//             16t + (l & 15), columns 32kb + 8(l >> 4) .. +7.  This is the B
//             operand of v_mfma_f32_16x16x32_bf16, so one dwordx4 load per lane
//             per MFMA, and a wave streams contiguous 1 KiB chunks.
//   * Q8_0 / FP8: one 1 KiB chunk per (tile, pair of k blocks), index
//             t*(KB/2) + p; lane l owns 16 bytes: 8 codes of block 2p then 8
//             codes of block 2p+1, same row / column rule as BF16.
//             Q8_0 scales: one dword per (tile, pair, row): [tiles][KB/2][16]
//             holding the fp16 scales of blocks 2p (low half) and 2p+1, so a
//             wave reads 64 contiguous bytes of scales per 1 KiB of codes.
//             FP8 scales: fp32 [tiles*16].
//   * MXFP4:  one 1 KiB chunk per (tile, quad of k blocks), index
//             t*(KB/4) + p; lane l owns 16 bytes: dword j holds the 8 E2M1
//             codes (element i in nibble i) of block 4p + j, same row /
//             column rule as BF16.  Scales: one dword per (tile, quad, row):
//             [tiles][KB/4][16], byte j = E8M0 code of block 4p + j.
//             Needs KB % 4 == 0.
//   * F32:    one 1 KiB chunk per (tile, 16-wide k group g); lane l owns 4
//             floats of row 16t + (l & 15), columns 16g + 4(l >> 4) .. +3,
//             fed to four v_mfma_f32_16x16x4_f32 in turn.
//  Grouped matrices (per-head W_UK^T and W_UV) pad every group of G rows to
//  TG = ceil(G/16) tiles, so no tile spans two heads.
//
//  Activation fragments ("A" operand, written by the elementwise kernels):
//   * bf16 family, hi/lo (M <= 8): per group [KB][64 lanes][8] bf16; lane l
//     holds row m = l & 15 for m < 8 as the bf16 rounding hi = bf16(v) and
//     for m >= 8 the residual lo = bf16(v - hi) of row m - 8, columns
//     32kb + 8(l >> 4) .. +7.  Summing MFMA output rows m and m + 8 gives the
//     product with ~16 significant bits of the fp32 activation at no extra
//     MFMA cost (rows 8..15 would otherwise be padding).
//   * bf16 family, plain (M > 8): per group [MT][KB][64][8], row 16mt + (l & 15).
//   * f32 family: per group [MT][Kp/16][64][4] fp32, row 16mt + (l & 15),
//     columns 16g + 4(l >> 4) .. +3.
//   * int8 hi/lo (Q8_0 consumers, M <= 8): per group [KB][64 lanes][8] int8
//     codes then [KB][8 rows] int8 exponents (see frag_put_i8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

enum { DT_F32 = 0, DT_BF16 = 1, DT_Q8_0 = 2, DT_FP8 = 3, DT_MXFP4 = 4 };

// ------------------------------------------------------------------ scalars --
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 to packed bf16 (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Two fp32 to packed fp16 (low half = a), round to nearest even.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
}

__device__ __forceinline__ float fp16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}


// ------------------------------------------------------------ weight decode --
// Two int8 codes (bytes sh/8 and sh/8 + 1 of w) -> two bf16 in one dword.  Codes
// are integers of magnitude <= 127, exact in bf16; the fp32 conversion is exact
// and its upper half is the bf16 pattern.
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int sh) {
  float f0 = (float)(int8_t)(w >> sh);
  float f1 = (float)(int8_t)(w >> (sh + 8));
  return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r[0] = i8x2_to_bf16x2(lo, 0);
  r[1] = i8x2_to_bf16x2(lo, 16);
  r[2] = i8x2_to_bf16x2(hi, 0);
  r[3] = i8x2_to_bf16x2(hi, 16);
  return __builtin_bit_cast(bf16x8, r);
}

// Eight FP8 E4M3FN codes -> eight bf16 (every E4M3 value is exact in bf16),
// using the gfx950 scaled conversion with scale 1.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return __builtin_bit_cast(bf16x8, r);
}

// E8M0 scale code j (byte j of w) -> fp32 2^(code - 127), formed as the
// exponent field alone (code 0 gives 0, code 255 gives +inf).
template <int J>
__device__ __forceinline__ float e8m0_f32(uint32_t w) {
  return __uint_as_float((J < 3 ? w << (23 - 8 * J) : w >> 1) & 0x7F800000u);
}

// Eight E2M1 codes (nibble i = element i) times a power-of-two scale -> eight
// bf16, exact (two significant bits), by the gfx950 scaled conversion.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// ---------------------------------------------------------------- matrices --
// Device view of one packed weight matrix (see the layout notes above).
struct PackedMat {
  const unsigned char* codes;  // code plane
  const void* scales;          // Q8_0: u32 [tiles][KB/2][16]; FP8: f32 [tiles*16];
                               // MXFP4: u32 [tiles][KB/4][16]; else null
  int fmt;                     // DT_*
  int ngroups;                 // >= 1
  int G;                       // logical rows per group
  int TG;                      // 16-row tiles per group
  int K;                       // logical reduction length
  int Kp;                      // padded to a multiple of 64
  int KB;                      // Kp / 32
};

// Input buffer descriptor of one GEMM: either plain fp32 rows [group][M][ld]
// (rows = 1: the GEMM builds its MFMA fragments in LDS) or prepared fragments.
struct FragDesc {
  void* ptr;
  int rows;         // 1: fp32 rows, row stride ld, group stride gstride
  int ld;
  int f32;          // fragments: 1 f32 family, 0 bf16 family
  int hilo;         // bf16 family with M <= 8
  int i8;           // int8 hi/lo codes (M <= 8, Q8_0 consumers): gstride in bytes
  int KB;           // Kp / 32 (bf16 family, int8)
  int KG;           // Kp / 16 (f32 family)
  int MT;           // m-tiles of 16 rows
  long long gstride;  // elements per group
};

// Write activation element (row m, column k) of group g into a GEMM input.
__device__ __forceinline__ void frag_put(const FragDesc& fd, int g, int m, int k, float v) {
  if (fd.rows) {
    ((float*)fd.ptr)[(long long)g * fd.gstride + (long long)m * fd.ld + k] = v;
    return;
  }
  if (fd.f32) {
    const int grp = k >> 4, q = (k >> 2) & 3, i = k & 3;
    const int mt = m >> 4, lane = q * 16 + (m & 15);
    float* p = (float*)fd.ptr + (long long)g * fd.gstride;
    p[((long long)(mt * fd.KG + grp) * 64 + lane) * 4 + i] = v;
    return;
  }
  const int kb = k >> 5, q = (k >> 3) & 3, i = k & 7;
  uint16_t* p = (uint16_t*)fd.ptr + (long long)g * fd.gstride;
  const uint32_t hb = f32_to_bf16_bits(v);
  if (fd.hilo) {
    const float lo = v - bf16_bits_to_f32(hb);
    p[((long long)kb * 64 + q * 16 + m) * 8 + i] = (uint16_t)hb;
    p[((long long)kb * 64 + q * 16 + 8 + m) * 8 + i] = (uint16_t)f32_to_bf16_bits(lo);
  } else {
    const int mt = m >> 4, lane = q * 16 + (m & 15);
    p[((long long)(mt * fd.KB + kb) * 64 + lane) * 8 + i] = (uint16_t)hb;
  }
}

// Eight consecutive columns k0 .. k0 + 7 (k0 a multiple of 8) of row m of
// group g: bf16 fragments keep them together (one 16-byte store per code
// row); other layouts element by element.
__device__ __forceinline__ void frag_put8(const FragDesc& fd, int g, int m, int k0, const float (&v)[8]) {
  if (fd.rows || fd.f32 || fd.i8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) frag_put(fd, g, m, k0 + i, v[i]);
    return;
  }
  const int kb = k0 >> 5, q = (k0 >> 3) & 3;
  uint16_t* p = (uint16_t*)fd.ptr + (long long)g * fd.gstride;
  u32x4 hw, lw;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t h0 = f32_to_bf16_bits(v[2 * u]), h1 = f32_to_bf16_bits(v[2 * u + 1]);
    hw[u] = h0 | (h1 << 16);
    lw[u] = f32_to_bf16_bits(v[2 * u] - bf16_bits_to_f32(h0)) | (f32_to_bf16_bits(v[2 * u + 1] - bf16_bits_to_f32(h1)) << 16);
  }
  if (fd.hilo) {
    *(u32x4*)(p + ((long long)kb * 64 + q * 16 + m) * 8) = hw;
    *(u32x4*)(p + ((long long)kb * 64 + q * 16 + 8 + m) * 8) = lw;
  } else {
    *(u32x4*)(p + ((long long)((m >> 4) * fd.KB + kb) * 64 + q * 16 + (m & 15)) * 8) = hw;
  }
}

// int8 activation fragments (the A operand of v_mfma_i32_16x16x32_i8 for
// M <= 8 rows): per group, codes [KB][64 lanes][8 bytes] then exponents
// [KB][8 rows] (int8).  Row m of 32-block kb is v ~ (hi + lo / 256) * 2^e with
// hi, lo in [-127, 127] and e the smallest exponent with max |v| <= 127 * 2^e
// over the block; lane q * 16 + m holds the hi codes of k = 8 q .. 8 q + 7,
// lane q * 16 + 8 + m the lo codes.  bm = max |v| over the block.
__device__ __forceinline__ int frag_i8_exp(float bm) {
  int e = 0;
  if (bm > 0.f) frexpf(bm * (1.f / 127.f), &e);
  return e;
}
__device__ __forceinline__ void frag_i8_codes(float v, int e, int& hi, int& lo) {
  const float qh = fminf(fmaxf(rintf(ldexpf(v, -e)), -127.f), 127.f);
  const float ql = fminf(fmaxf(rintf(ldexpf(v - ldexpf(qh, e), 8 - e)), -127.f), 127.f);
  hi = (int)qh;
  lo = (int)ql;
}
__device__ __forceinline__ void frag_put_i8(const FragDesc& fd, int g, int m, int k, float v, float bm) {
  const int e = frag_i8_exp(bm);
  int qh, ql;
  frag_i8_codes(v, e, qh, ql);
  const int kb = k >> 5, q = (k >> 3) & 3, i = k & 7;
  unsigned char* p = (unsigned char*)fd.ptr + (long long)g * fd.gstride;
  p[((long long)kb * 64 + q * 16 + m) * 8 + i] = (unsigned char)qh;
  p[((long long)kb * 64 + q * 16 + 8 + m) * 8 + i] = (unsigned char)ql;
  if ((k & 31) == 0) p[(long long)fd.KB * 512 + kb * 8 + m] = (unsigned char)(signed char)e;
}
// The same codes for eight consecutive columns k0 .. k0 + 7 of row m (k0 a
// multiple of 8), written as one 8-byte word per code row; e is the block's
// exponent, written by the thread that holds the block's first column.
__device__ __forceinline__ void frag_put_i8_x8(const FragDesc& fd, int g, int m, int k0, const float (&v)[8], int e) {
  uint32_t hw[2] = {0u, 0u}, lw[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int qh, ql;
    frag_i8_codes(v[i], e, qh, ql);
    hw[i >> 2] |= ((uint32_t)qh & 0xFFu) << (8 * (i & 3));
    lw[i >> 2] |= ((uint32_t)ql & 0xFFu) << (8 * (i & 3));
  }
  const int kb = k0 >> 5, q = (k0 >> 3) & 3;
  unsigned char* p = (unsigned char*)fd.ptr + (long long)g * fd.gstride;
  *(u32x2*)(p + ((long long)kb * 64 + q * 16 + m) * 8) = u32x2{hw[0], hw[1]};
  *(u32x2*)(p + ((long long)kb * 64 + q * 16 + 8 + m) * 8) = u32x2{lw[0], lw[1]};
  if (q == 0) p[(long long)fd.KB * 512 + kb * 8 + m] = (unsigned char)(signed char)e;
}

// ------------------------------------------------------------- reductions --
// Cross-lane reductions without the LDS crossbar (a ds_bpermute per step,
// each followed by a wait on its result).  Inside each 16-lane DPP row, four
// DPP moves pair lane i with i ^ 1, i ^ 2 (quad permutes), 7 - i (half-row
// mirror) and 15 - i (row mirror); each step combines a lane with a partner
// that holds the other half of the lanes reduced so far, so after the four
// steps every lane holds the row total, bit-identical across the row (the
// operations are commutative).  Row totals are then read with v_readlane
// from lanes 0, 16, 32 and 48.  Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<DPP_XOR1>(v);
  v += dpp_mov<DPP_XOR2>(v);
  v += dpp_mov<DPP_HALF_MIRROR>(v);
  return v + dpp_mov<DPP_MIRROR>(v);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<DPP_XOR1>(v));
  v = fmaxf(v, dpp_mov<DPP_XOR2>(v));
  v = fmaxf(v, dpp_mov<DPP_HALF_MIRROR>(v));
  return fmaxf(v, dpp_mov<DPP_MIRROR>(v));
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
// Maximum over each 32-lane half of the wave.
__device__ __forceinline__ float half_wave_max(float v) {
  v = row16_max(v);
  const float h0 = fmaxf(lane_value(v, 0), lane_value(v, 16)), h1 = fmaxf(lane_value(v, 32), lane_value(v, 48));
  return (threadIdx.x & 32) ? h1 : h0;
}

// Wave-cooperative write: every lane of the wave calls it, lane L holding
// column k0 + L of row m with k0 a multiple of 64 (so each half wave covers
// one 32-block); `valid` masks columns outside the matrix.
__device__ __forceinline__ void frag_put_wave(const FragDesc& fd, int g, int m, int k, float v, bool valid) {
  if (fd.i8) {
    const float bm = half_wave_max(valid ? fabsf(v) : 0.f);
    if (valid) frag_put_i8(fd, g, m, k, v, bm);
  } else if (valid) {
    frag_put(fd, g, m, k, v);
  }
}

// Sum over a 256-thread block; `red` is __shared__ float[4].
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
__device__ __forceinline__ float block_max256(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Order-preserving 64-bit key of (value, index): larger value wins, and on
// equal values the lower index wins.  -0 is folded into +0 first.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ int key_index(unsigned long long k) {
  return (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
}

constexpr int KEY_SLOTS = 16;  // argmax partial slots per (sequence, position)

}  // namespace dspark
