// Markov rollout of a whole block in one persistent launch (huggingface.co
// "Kimi-K3-DSpark-NVFP4", original card, "Model Overview": a low-rank
// sequential Markov head supplies the intra-block dependency after the
// parallel backbone pass).
//
// Position i needs the argmax of position i - 1, so the W2 product is
// sequential over the block, but W2 itself is the same matrix every step.
// This kernel loads each wave's share of W2 (MK_TPW 16-row tiles) into
// registers once and keeps it there for all positions: 1024 waves (one per
// SIMD) x 10 tiles x 8 KiB hold the full 163,840 x 256 bf16 W2 (84 MB) in the
// register files of the 256 CUs, so positions 1..6 read no weights from
// memory at all.
//
// Exchange between workgroups: for every (position, sequence) each workgroup
// stores its local argmax key (64-bit, never zero) into its own slot; a
// workgroup that needs the predecessor polls all slots of the previous
// position until none is zero, and their maximum is the argmax.  The poll is
// the barrier and the data at once.  Slots are written and read with
// device-scope atomic operations, which are coherent across the XCDs' L2
// caches without release/acquire (that would write back and invalidate the
// whole L2 at every step).  With forced predecessors (teacher forcing) the
// positions are independent and nothing is polled.
//
// Every workgroup must be resident at once.  The host checks that the grid
// (one 4-wave workgroup per CU) fits the device at this kernel's occupancy;
// stream order leaves every CU free when the kernel starts.  (A cooperative
// launch would guarantee the same, at ~25 us of extra gaps per call.)  The
// poll is bounded: should residency ever fail, it expires, the kernel
// records an error flag and finishes, and k_markov_final reports tokens of
// -1, so a failure is loud and never a hang.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace dspark {

namespace {

constexpr int MK_TPW = 10;              // W2 tiles per wave, held in registers (VGPRs and AGPRs)
constexpr int MK_WAVES = 4;             // waves per workgroup (one per SIMD)
constexpr int MK_THREADS = 64 * MK_WAVES;
constexpr unsigned MK_SPIN_LIMIT = 1u << 22;

__device__ __forceinline__ u32x4 mk_ntload(const u32x4* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ unsigned long long mk_max(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

// Maximum of 64-bit keys over each 16-lane DPP row (every lane of the row
// gets it): the DPP moves of common.h's row reductions, applied to both
// halves of the key.  Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ unsigned long long mk_dpp_u64(unsigned long long v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ unsigned long long mk_row16_max(unsigned long long v) {
  v = mk_max(v, mk_dpp_u64<DPP_XOR1>(v));
  v = mk_max(v, mk_dpp_u64<DPP_XOR2>(v));
  v = mk_max(v, mk_dpp_u64<DPP_HALF_MIRROR>(v));
  return mk_max(v, mk_dpp_u64<DPP_MIRROR>(v));
}
__device__ __forceinline__ unsigned long long mk_lane_u64(unsigned long long v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long mk_wave_max(unsigned long long v) {
  v = mk_row16_max(v);
  return mk_max(mk_max(mk_lane_u64(v, 0), mk_lane_u64(v, 16)), mk_max(mk_lane_u64(v, 32), mk_lane_u64(v, 48)));
}

// Argmax keys of position `pos` for every sequence (into tok[m]), polling the
// slots of all workgroups until each is written.  All threads take part; wave
// w reduces sequences w, w + MK_WAVES, ...  The wait is bounded (spin_limit
// polls, default MK_SPIN_LIMIT): on expiry the error flag is raised and the
// predecessors become -1, and the workgroup carries on, so every workgroup
// still publishes every position and the grid drains.
__device__ void mk_poll(const MarkovArgs& a, int pos, int nwg, unsigned long long* red, int* tok) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (a.spin_limit < 0) {  // host-forced expiry: no wait at all
    if (threadIdx.x == 0) __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x < 16) tok[threadIdx.x] = -1;
    __syncthreads();
    return;
  }
  const unsigned limit = a.spin_limit > 0 ? (unsigned)a.spin_limit : MK_SPIN_LIMIT;
  unsigned spins = 0;
  for (;;) {
    int missing = 0;
    for (int q = wave; q < a.M; q += MK_WAVES) {
      const unsigned long long* sl = a.slots + ((long long)pos * a.M + q) * nwg;
      unsigned long long v = 0;
      for (int w = lane; w < nwg; w += 64) {
        const unsigned long long x = __hip_atomic_load(sl + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        missing |= x == 0;
        v = mk_max(v, x);
      }
      v = mk_wave_max(v);
      if (lane == 0) red[q] = v;
    }
    if (!__syncthreads_or(missing)) {
      if ((int)threadIdx.x < a.M) tok[threadIdx.x] = key_index(red[threadIdx.x]);
      __syncthreads();
      return;
    }
    __builtin_amdgcn_s_sleep(1);
    if (++spins >= limit) {
      if (threadIdx.x == 0) __hip_atomic_fetch_or(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (threadIdx.x < 16) tok[threadIdx.x] = -1;
      __syncthreads();
      return;
    }
  }
}

// This step's lm_head logits of the wave's MK_TPW * 16 columns, straight to
// LDS as [sequence][column] (they do not depend on the predecessor, so they
// arrive while it is resolved): one 16-byte copy per lane and sequence.
constexpr int MK_ZCOLS = MK_TPW * 16;
static_assert(MK_ZCOLS % 4 == 0 && MK_ZCOLS / 4 <= 64, "one copy per sequence");
__device__ __forceinline__ void mk_fetch_z(const MarkovArgs& a, int step, int t0, int lane, float* dst) {
  const int c = t0 * 16 + 4 * lane;  // first of this lane's four columns
  const bool ok = 4 * lane < MK_ZCOLS && c + 4 <= a.vocab;
  for (int mm = 0; mm < a.M; ++mm)
    if (ok)
      __builtin_amdgcn_global_load_lds(a.z + ((long long)mm * a.block + step) * a.vocab + c, dst + mm * MK_ZCOLS, 16, 0, 0);
}

template <int KB>
__global__ __launch_bounds__(MK_THREADS, 1) void k_markov_rollout(MarkovArgs a) {
  if (a.fallback && *a.fallback == 0) return;  // the candidate rollout drafted the block
  __shared__ unsigned long long red[MK_WAVES * 16];
  __shared__ __attribute__((aligned(16))) float zl[MK_WAVES][16][MK_ZCOLS];  // lm_head logits [sequence][column], current step
  __shared__ int tok[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.tiles;
  const int nwg = gridDim.x;
  const int t0 = (blockIdx.x * MK_WAVES + wave) * MK_TPW;

  mk_fetch_z(a, 0, t0, lane, &zl[wave][0][0]);
  // this wave's W2 tiles, resident for the whole block
  u32x4 w[MK_TPW][KB];
  {
    const u32x4* wp = (const u32x4*)a.w2 + lane;
#pragma unroll
    for (int j = 0; j < MK_TPW; ++j)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        w[j][kb] = t0 + j < T ? mk_ntload(wp + ((long long)(t0 + j) * KB + kb) * 64) : u32x4{0u, 0u, 0u, 0u};
  }

  const int m = lane & 15;  // sequence of this lane's A-operand row
  for (int step = 0; step < a.block; ++step) {
    // predecessor of every sequence
    if (step == 0) {
      if (threadIdx.x < 16) tok[threadIdx.x] = (int)threadIdx.x < a.M ? a.prev_token[threadIdx.x] : -1;
      __syncthreads();
    } else if (a.forced) {
      if (threadIdx.x < 16) tok[threadIdx.x] = (int)threadIdx.x < a.M ? a.forced[threadIdx.x * a.block + step - 1] : -1;
      __syncthreads();
    } else {
      mk_poll(a, step - 1, nwg, red, tok);
    }
    // A operand: row m = W1[t_prev(m)], k = 32 kb + 8 (lane >> 4) .. + 7
    bf16x8 A[KB];
    {
      const int tp = m < a.M ? tok[m] : -1;
      const bool ok = tp >= 0 && tp < a.vocab;
      const uint16_t* src = (const uint16_t*)a.w1 + (ok ? (long long)tp * a.w1_ld : 0) + 8 * (lane >> 4);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) A[kb] = ok ? *(const bf16x8*)(src + 32 * kb) : bf16x8{};
    }
    unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
    for (int j = 0; j < MK_TPW; ++j) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[kb], __builtin_bit_cast(bf16x8, w[j][kb]), acc, 0, 0, 0);
      const int col = (t0 + j) * 16 + (lane & 15);
      if (t0 + j < T && col < a.vocab) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mm = (lane >> 4) * 4 + r;  // sequence of output row r
          if (mm >= a.M) continue;
          const long long row = (long long)mm * a.block + step;
          const float v = acc[r] + zl[wave][mm][j * 16 + (lane & 15)];
          if (a.logits) a.logits[row * a.vocab + col] = v;
          // probabilistic drafting: argmax of v / T plus a Gumbel variate
          const float sel = a.sample_u ? v * a.inv_temp - logf(-logf(a.sample_u[row * a.vocab + col])) : v;
          best[r] = mk_max(best[r], argmax_key(sel, (uint32_t)col));
        }
      }
    }
    // argmax per sequence over the workgroup: the 16 columns of each lane
    // group (rows r >= M hold no sequence in any group), then the waves;
    // then this workgroup's slot
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r >= a.M) break;
      best[r] = mk_row16_max(best[r]);
    }
    if ((lane & 15) == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave * 16 + (lane >> 4) * 4 + r] = best[r];
    }
    __syncthreads();  // also: every wave is done with zl of this step
    if (step + 1 < a.block) mk_fetch_z(a, step + 1, t0, lane, &zl[wave][0][0]);
    if (threadIdx.x < 16 && (int)threadIdx.x < a.M) {
      unsigned long long k = red[threadIdx.x];
#pragma unroll
      for (int q = 1; q < MK_WAVES; ++q) k = mk_max(k, red[q * 16 + threadIdx.x]);
      // a workgroup without valid columns still publishes (a key that loses to any real one)
      if (!k) k = 1;
      __hip_atomic_store(a.slots + ((long long)step * a.M + threadIdx.x) * nwg + blockIdx.x, k, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // red is reused by the poll
  }
}

template <int KB>
hipError_t launch_rollout(const MarkovArgs& a, hipStream_t st) {
  const int waves = (a.tiles + MK_TPW - 1) / MK_TPW;
  const int wgs = (waves + MK_WAVES - 1) / MK_WAVES;
  if (wgs > a.max_wgs) return hipErrorInvalidValue;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_markov_rollout<KB>, MK_THREADS, 0)) != hipSuccess)
    return e;
  if ((long long)per_cu * cus < wgs) return hipErrorCooperativeLaunchTooLarge;
  hipLaunchKernelGGL(k_markov_rollout<KB>, dim3(wgs), dim3(MK_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int markov_rollout_wgs(int tiles) { return ((tiles + MK_TPW - 1) / MK_TPW + MK_WAVES - 1) / MK_WAVES; }

bool markov_rollout_supported(int KB, int M, int vocab) {
  return (KB == 8 || KB == 2) && M >= 1 && M <= 16 && vocab % 4 == 0;  // logits copied four columns at a time
}

hipError_t launch_markov_rollout(const MarkovArgs& a, int KB, hipStream_t st) {
  if (!markov_rollout_supported(KB, a.M, a.vocab)) return hipErrorInvalidValue;
  if (KB == 8) return launch_rollout<8>(a, st);
  if (KB == 2) return launch_rollout<2>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace dspark
