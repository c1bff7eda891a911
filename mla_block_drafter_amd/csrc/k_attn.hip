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
// row-major, four buffers deep.  S^T = K Q^T takes the key rows as the A operand (16-byte LDS
// reads), so the probabilities land with one query row per lane column,
// which is already the B-operand layout of P^T for O^T = V^T P^T: the
// probabilities never leave registers (the 32 keys' order inside the MFMA
// reduction is permuted identically on both operands).  The V^T operand is
// gathered from the same row-major tile with 2-byte LDS reads (the value is
// c_kv, the first kv_lora columns of the key row), so no transposed copy is
// staged.  Online softmax state (m, l) is per lane column.  Partials per slot
// are merged by k_attn_combine in a fixed order.
#include <type_traits>

#include "kernels.h"

namespace dspark {

namespace {

constexpr int KT = 32;  // keys per LDS tile
constexpr int NBUF = 4;  // key tile buffers: three tiles in flight while one computes
constexpr float REDO_SLACK = 60.f;  // natural-log units: e^60 * 2048 keys stays far below fp32 max
constexpr int MAX_COMBINE_SLOTS = 4096;

__device__ __forceinline__ void slot_lookup(const AttnArgs& a, int slot, int& s, int& p, int& len,
                                            int& off, int& J) {
  if (a.len1 >= 0) {  // one sequence: no memory round trip
    s = 0;
    p = slot;
    off = 0;
    len = a.len1;
    J = len + a.block;
    if (slot >= (J + a.C - 1) / a.C) s = -1;
    return;
  }
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

// ---------------------------------------------------------------- tiles --
// A key tile (KT = 32 keys) is fetched with gfx950's direct-to-LDS loads
// (global_load_lds_dwordx4: a wave writes 64 consecutive 16-byte LDS chunks,
// no registers involved).  Two regions per tile buffer:
//   A: the value part (first R = 8 CA elements of the key row), one key per
//      load, rows CA + 2 chunks apart: with 1056-byte rows both the 16-byte
//      reads of S^T (16 keys per 16 lanes) and the transposing reads of V
//      (8 keys per 32 lanes) hit each of the 64 LDS banks at most once per
//      phase (with one pad chunk, 1040-byte rows, both were two-way
//      conflicts);
//   B: the rope part (CB chunks per key), 64 / CB keys per load, chunk p of
//      key r holding source chunk p ^ bswz(r).  Rows are 128 bytes, so keys
//      of equal parity use the same half of the banks; bswz gives the 8 such
//      keys of a 16-lane read 8 different chunk orders.
// Loads that fall past the slot read a valid dummy row (the sequence's first
// block key); their scores are masked and their probabilities are zero.  So do
// the rope-region chunks past the stored row when the query width is padded
// beyond the latent (their query dims are zero).
// NBUF tile buffers: tiles t+1 .. t+NBUF-1 stream in while tile t computes.
//
// Inside each 16-key half of a tile, MFMA row m holds key pi(m) =
// (g & 1) + 8 (g >> 1) + 2 j for m = 4 g + j.  The score fragment of lane
// group g then covers keys {a, a+2, a+4, a+6}, whose padded rows fall on
// disjoint banks when the transposing LDS read gathers V for the same keys.
__device__ __forceinline__ int key_perm(int m) { return (m >> 2 & 1) + 8 * (m >> 3) + 2 * (m & 3); }

// Chunk order of region-B row r (depends on r mod 16 only, so key r of a
// tile and key r - 16 of its second half agree).
template <int CB>
__device__ __forceinline__ int bswz(int r) { return (r >> 1) % CB; }

template <int CA, int CB>
struct TileGeom {
  static constexpr int ROW_A = (CA + 2) * 8;      // elements between region-A rows
  static constexpr int SIZE_A = KT * ROW_A;       // elements
  static constexpr int KPB = 64 / CB;             // region-B keys per load
  static constexpr int NB_A = KT;                 // loads for region A
  static constexpr int NB_B = KT / KPB;           // loads for region B
  static constexpr int NBLK = NB_A + NB_B;
  static constexpr int BUF = SIZE_A + KT * CB * 8;  // elements per tile buffer
  static_assert(64 % CB == 0 && KT % KPB == 0 && CA <= 64, "tile geometry");
};

// This wave's share of one key tile: region-A keys wave, wave + 4, ... and
// region-B load number wave.  Everything but the lane offsets is uniform, so
// the address selection stays on the scalar unit.
// trow: the cache row of key kt0 (a tile never crosses a page, so key kt0 + i
// of the tile is row trow + i in both layouts; PAGED only keeps the two
// kernels' specializations apart).
//
// Paged caches: the cache row of key kt0 (kt0 < len, wave-uniform) of a slot
// whose first page is pfirst, lane i of pgv holding the slot's page i.
__device__ __forceinline__ int paged_row(const AttnArgs& a, int kt0, int pfirst, int pgv) {
  const int i = __builtin_amdgcn_readfirstlane((kt0 >> a.page_log2) - pfirst);  // 0 .. 63
  const int page = __builtin_amdgcn_readlane(pgv, i);
  return (page << a.page_log2) + (kt0 & ((1 << a.page_log2) - 1));
}

template <int CA, int CB, bool PAGED>
__device__ __forceinline__ void issue_tile(const AttnArgs& a, int lane, int wave, int kt0, int k_end, int s,
                                           int len, int trow, const uint16_t* cache, const uint16_t* bk,
                                           const uint16_t* dummy, uint16_t* dst) {
  using G = TileGeom<CA, CB>;
  static_assert(G::NB_A % 4 == 0 && G::NB_B <= 4, "load split over four waves");
  if (kt0 + KT <= min(len, k_end)) {
    // common case: the whole tile is valid cache rows (uniform row pointer)
    const long long ld = a.latent;
    const uint16_t* src = cache + (trow + wave) * ld + 8 * lane;
#pragma unroll
    for (int i = 0; i < G::NB_A / 4; ++i, src += 4 * ld)
      if (CA == 64 || lane < CA) __builtin_amdgcn_global_load_lds(src, dst + (wave + 4 * i) * G::ROW_A, 16, 0, 0);
    if (wave < G::NB_B) {
      const int r = wave * G::KPB + lane / CB, c = CA + ((lane % CB) ^ bswz<CB>(r));
      // chunks past the stored row (query padding, zero) read the dummy row
      const uint16_t* sb = 8 * c < a.latent ? cache + (trow + r) * ld + 8 * c : dummy;
      __builtin_amdgcn_global_load_lds(sb, dst + G::SIZE_A + wave * 512, 16, 0, 0);
    }
    return;
  }
  auto row_ptr = [&](int j) {
    const uint16_t* c = cache + (long long)(trow + j - kt0) * a.latent;
    const uint16_t* k = bk + (long long)(s * a.block + (j - len)) * a.latent;
    const uint16_t* r = j < len ? c : k;
    return j < k_end ? r : dummy;
  };
#pragma unroll
  for (int i = 0; i < G::NB_A / 4; ++i) {
    const int b = wave + 4 * i;
    const uint16_t* src = row_ptr(kt0 + b) + 8 * lane;
    if (CA == 64 || lane < CA) __builtin_amdgcn_global_load_lds(src, dst + b * G::ROW_A, 16, 0, 0);
  }
  if (wave < G::NB_B) {
    const int r = wave * G::KPB + lane / CB, c = CA + ((lane % CB) ^ bswz<CB>(r));
    // chunks past the stored row (query padding, zero) read the dummy row
    const uint16_t* src = 8 * c < a.latent ? row_ptr(kt0 + r) + 8 * c : dummy;
    __builtin_amdgcn_global_load_lds(src, dst + G::SIZE_A + wave * 512, 16, 0, 0);
  }
}

// Workgroups go to the 8 XCDs round-robin (linear id L to XCD L % 8), and
// each XCD has its own L2.  Each XCD gets a contiguous run of (slot, row
// group) pairs, so the row groups of a slot, which read the same key tiles,
// mostly share one L2 and the tiles come from HBM once per slot instead of
// once per row group.  Placement only: any mapping would be correct.
__device__ __forceinline__ int xcd_pair(int L, int ntot) {
  const int x = L % 8, j = L / 8;
  return x * (ntot / 8) + min(x, ntot % 8) + j;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int QK_AHEAD = 6;  // K fragments in flight ahead of the MFMA using them
constexpr int PV_AHEAD = 4;  // V fragment pairs in flight ahead of the MFMA using them

template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t*)p;
}

// LDS reads of the tile loop are issued from inline assembly with explicit,
// register-tied waits.  Two reasons: the compiler makes a transposing LDS read
// wait for every outstanding direct-to-LDS load (including the prefetch of the
// next tile), and under this register pressure it keeps only two ordinary LDS
// reads in flight.  LDS operations complete in issue order, so "at most n
// outstanding" covers every read issued n or more reads earlier.  Scalar
// memory loads, which share the counter but complete out of order, are never
// issued inside the tile loop.
template <int OFF>
__device__ __forceinline__ void lds_read_b128(uint32_t addr, u32x4& v) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
}

template <int OFF_LO, int OFF_HI>
__device__ __forceinline__ void tr_read_pair(uint32_t addr, u32x2& lo, u32x2& hi) {
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
               : "=v"(lo), "=v"(hi)
               : "v"(addr), "i"(OFF_LO), "i"(OFF_HI));
}

template <int N>
__device__ __forceinline__ void lds_wait(u32x4& v) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait_pair(u32x2& lo, u32x2& hi) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(lo), "+v"(hi) : "n"(N));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int NKB, int NDT, bool PAGED>
__global__ __launch_bounds__(256, 1) void k_attn_bf16(AttnArgs a) {
  constexpr int DQ = NKB * 32;
  constexpr int R = NDT * 16;
  constexpr int CA = R / 8, CB = (DQ - R) / 8;
  using G = TileGeom<CA, CB>;
  static_assert(CA % 4 == 0, "each k-step reads one region");
  static_assert(NBUF == 4, "tile buffers");
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[NBUF * G::BUF];

  const int ngrp = a.rows_pad / 64;
  const int pair = xcd_pair(blockIdx.x, gridDim.x);
  const int slot = pair / ngrp, rgrp = pair % ngrp;
  int s, p, len, off, J;
  slot_lookup(a, slot, s, p, len, off, J);
  if (s < 0) return;  // uniform over the workgroup
  const int k_begin = p * a.C;
  const int k_end = min(J, k_begin + a.C);
  const int ntiles = (k_end - k_begin + KT - 1) / KT;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps tile loads scalar
  const int row0 = rgrp * 64 + wave * 16;
  const int myrow = row0 + (lane & 15);
  const int grp = lane >> 4;

  const uint16_t* cache = (const uint16_t*)a.cache;
  const uint16_t* bk = (const uint16_t*)a.bkeys;
  const uint16_t* dummy = bk + (long long)s * a.block * a.latent;
  // paged caches: the page indices of this slot's keys (at most C / 32 = 64),
  // one per lane of a VGPR, read once here: no memory load may enter the tile
  // loop, whose LDS waits count on the shared counter (and more scalar
  // registers would spill under this register pressure)
  const int pfirst = PAGED ? k_begin >> a.page_log2 : 0;
  int pgv = 0;
  if (PAGED) {
    const int32_t* tb = a.table + (long long)s * a.max_pages;
    pgv = tb[min(pfirst + lane, a.max_pages - 1)];
  }

  // Q fragments (B operand of S^T = K Q^T): row myrow, dims 32kb + 8 grp.
  bf16x8 qf[NKB];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((long long)s * a.rows_pad + myrow) * DQ + 8 * grp;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) qf[kb] = *(const bf16x8*)(qrow + 32 * kb);
  }
  // LDS element offsets inside a tile buffer
  const int kA = key_perm(lane & 15);                 // key of this lane's A-operand row
  const int offA = kA * G::ROW_A + 8 * grp;           // + 16 h ROW_A + 32 kb
  const int offB = G::SIZE_A + kA * CB * 8;           // + 16 h CB 8 + chunk
  // byte offsets of chunks 4 k + grp (k < CB / 4) of region B for this lane's key
  uint32_t bx[CB / 4];
#pragma unroll
  for (int k = 0; k < CB / 4; ++k) bx[k] = 16 * ((4 * k + grp) ^ bswz<CB>(kA));
  const int kV = key_perm(4 * grp + ((lane & 15) >> 2));  // key this lane addresses for V
  const int offV = kV * G::ROW_A + 4 * (lane & 3);    // + 16 h ROW_A + 16 d
  int keyS[4];                                        // keys of this lane's score entries
#pragma unroll
  for (int j = 0; j < 4; ++j) keyS[j] = key_perm(4 * grp + j);

  // Softmax reference: the first tile's row maximum (pass 0).  The tile loop
  // never rescales the accumulators (they stay in AGPRs untouched by the
  // VALU); if a later score exceeds the reference by more than REDO_SLACK,
  // where exp() could approach the fp32 range, the workgroup redoes the slot
  // once with the exact row maximum as the reference (pass 1).
  // The running maximum and sum stay per lane inside the tile loop (no
  // cross-lane traffic there); the four lanes of a row are combined after it.
  __shared__ int redo_flag;
  const float c2 = a.tau * 1.4426950408889634f;  // base-2 score scale
  f32x4 acc[NDT];
  float m_run = -INFINITY, l_run = 0.f, m_all = -INFINITY;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
  for (int d = 0; d < NDT; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  l_run = 0.f;
  if (pass == 1) m_run = m_all;
  // prologue: tiles 0 .. NBUF - 2 in flight
#pragma unroll 1
  for (int i = 0; i < NBUF - 1; ++i)
    if (i < ntiles)
      issue_tile<CA, CB, PAGED>(a, lane, wave, k_begin + i * KT, k_end, s, len, PAGED ? paged_row(a, k_begin + i * KT, pfirst, pgv) : off + k_begin + i * KT, cache, bk, dummy,
                         k_lds + i * G::BUF);

  // One barrier per tile.  Direct-to-LDS copies complete in no fixed order
  // with respect to each other, so a partial count does not prove that tile
  // t has landed (waiting for "at most the later tiles' copies outstanding"
  // let a late copy of tile t be read, now and then, as a slightly different
  // result): each wave waits for all of its copies, then the barrier covers
  // every wave's.  Tiles t + 1 and t + 2 are then in LDS early; tile
  // t + NBUF - 1 goes out after the barrier (every wave has finished tile
  // t - 1, whose buffer it takes) and streams in during this tile's compute.
  for (int t = 0; t < ntiles; ++t) {
    const int kt0 = k_begin + t * KT;
    const int buf = t % NBUF;
    wait_vmcnt<0>();
    // the barrier intrinsic has no memory semantics of its own, so the
    // compiler fences keep LDS accesses on their side of it (a __syncthreads
    // would also drain the prefetch of the next tiles)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + NBUF - 1 < ntiles)
      issue_tile<CA, CB, PAGED>(a, lane, wave, kt0 + (NBUF - 1) * KT, k_end, s, len, PAGED ? paged_row(a, kt0 + (NBUF - 1) * KT, pfirst, pgv) : off + kt0 + (NBUF - 1) * KT, cache,
                         bk, dummy,
                         k_lds + ((t + NBUF - 1) % NBUF) * G::BUF);
    const uint16_t* tb = k_lds + buf * G::BUF;

    // ---- S^T for 32 keys x 16 rows: two 16-key MFMA tiles, read n = 2 kb + h
    //      feeding accumulator h; the two chains alternate ----
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
      constexpr int NR = 2 * NKB;
      const uint32_t abase = lds_addr(tb + offA), bbase = lds_addr(tb + offB);
      u32x4 kf[QK_AHEAD + 1];
      auto issue = [&](auto NI) {
        constexpr int n = decltype(NI)::value, kb = n / 2, h = n % 2;
        if constexpr (4 * kb < CA)
          lds_read_b128<2 * (16 * h * G::ROW_A + 32 * kb)>(abase, kf[n % (QK_AHEAD + 1)]);
        else
          lds_read_b128<2 * 16 * h * CB * 8>(bbase + bx[kb - CA / 4], kf[n % (QK_AHEAD + 1)]);
      };
      static_for<QK_AHEAD < NR ? QK_AHEAD : NR>(issue);
      static_for<NR>([&](auto NI) {
        constexpr int n = decltype(NI)::value;
        if constexpr (n + QK_AHEAD < NR) issue(std::integral_constant<int, n + QK_AHEAD>{});
        constexpr int ahead = NR - 1 - n < QK_AHEAD ? NR - 1 - n : QK_AHEAD;
        u32x4& f = kf[n % (QK_AHEAD + 1)];
        lds_wait<ahead>(f);
        st[n % 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f), qf[n / 2], st[n % 2], 0, 0, 0);
      });
    }
    // the first V fragments do not depend on P: their reads go out now and
    // arrive while the probabilities are computed
    const uint32_t vaddr = lds_addr(tb + offV);
    u32x2 vlo[PV_AHEAD + 1], vhi[PV_AHEAD + 1];
    auto issue_v = [&](auto DI) {
      constexpr int d = decltype(DI)::value;
      tr_read_pair<32 * d, 32 * d + 2 * 16 * G::ROW_A>(vaddr, vlo[d % (PV_AHEAD + 1)], vhi[d % (PV_AHEAD + 1)]);
    };
    static_for<PV_AHEAD < NDT ? PV_AHEAD : NDT>(issue_v);

    // lane holds keys kt0 + 16 h + keyS[r] for query row myrow.  Scores are
    // kept in base-2 units x = s * tau * log2(e) (tau > 0, so the maximum of
    // the raw products gives the maximum of x); keys past the slot (last
    // tile only) get -inf.
    if (kt0 + KT > k_end) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kt0 + 16 * h + keyS[r] >= k_end) st[h][r] = -INFINITY;
    }
    float tmax = fmaxf(fmaxf(fmaxf(st[0][0], st[0][1]), fmaxf(st[0][2], st[0][3])),
                       fmaxf(fmaxf(st[1][0], st[1][1]), fmaxf(st[1][2], st[1][3]))) * c2;
    m_all = fmaxf(m_all, tmax);  // this lane's keys only
    if (pass == 0 && t == 0) {
      // the reference: the row maximum over tile 0 (finite: tile 0 holds a
      // valid key).  These shuffles are LDS operations issued after the V
      // reads above; the compiler waits for them (and so for the V reads)
      // before m_run is used.
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      m_run = tmax;
    }
    u32x4 pw;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[h][r], c2, -m_run));
        l_run += pr[r];  // this lane's keys only
      }
      pw[2 * h] = pack_bf16x2(pr[0], pr[1]);
      pw[2 * h + 1] = pack_bf16x2(pr[2], pr[3]);
    }
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);

    // ---- O^T += V^T P^T.  k slots 0..3 of lane group g are keys keyS[] of
    //      the first half, slots 4..7 those of the second half, matching P.
    //      The transposing read hands lane 4a + e of each 16-lane group
    //      element e of the rows addressed by lanes a, a+4, a+8, a+12: lane
    //      (lane & 15) = 4 j + a addresses key keyS[j], dims 16 d + 4 a, so
    //      lane 4a + e receives dim 16 d + 4a + e of keys keyS[0..3] ----
    {
      static_for<NDT>([&](auto DI) {
        constexpr int d = decltype(DI)::value;
        if constexpr (d + PV_AHEAD < NDT) issue_v(std::integral_constant<int, d + PV_AHEAD>{});
        constexpr int ahead = NDT - 1 - d < PV_AHEAD ? NDT - 1 - d : PV_AHEAD;
        u32x2& lo = vlo[d % (PV_AHEAD + 1)];
        u32x2& hi = vhi[d % (PV_AHEAD + 1)];
        lds_wait_pair<2 * ahead>(lo, hi);
        const u32x4 v4 = {lo[0], lo[1], hi[0], hi[1]};
        acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v4), pf, acc[d], 0, 0, 0);
      });
    }
  }
    // combine the four lanes of each row (fixed butterfly: same bits in all)
    m_all = fmaxf(m_all, __shfl_xor(m_all, 16, 64));
    m_all = fmaxf(m_all, __shfl_xor(m_all, 32, 64));
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (pass == 1) break;
    // every wave has finished its tile reads; decide the redo together (the
    // barriers also keep the redo's tile loads off buffers still being read)
    if (threadIdx.x == 0) redo_flag = 0;
    __syncthreads();
    if (__any(m_all > m_run + REDO_SLACK * 1.4426950408889634f) && lane == 0) atomicOr(&redo_flag, 1);
    __syncthreads();
    if (!redo_flag) break;
  }

  // ---- partials: O^T[dim = 16d + 4(lane>>4) + r][row = myrow] divided by
  //      l, a convex combination of value rows, stored as fp16 (half the
  //      bytes of fp32; 11-bit significand, finer than the bf16 operands).
  //      Layout [row][slot][dim] so the combine of one row reads contiguous
  //      memory.  l >= 1: the reference key of the slot contributes exp(0). ----
  //      Each wave stages its 16 rows in LDS and stores them as whole rows
  //      (one 1 KiB row per store instead of 16 scattered 32-byte pieces).
  const long long prow = (long long)myrow * a.slots + slot;
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  __syncthreads();  // every wave is done with the tile buffers
  constexpr int RB = R * 2 + 16;  // bytes per staged row (the pad spreads the banks)
  unsigned char* stage = (unsigned char*)k_lds + wave * 16 * RB;
#pragma unroll
  for (int d = 0; d < NDT; ++d) {
    u32x2 h;
    h[0] = pack_f16x2(acc[d][0] * inv_l, acc[d][1] * inv_l);
    h[1] = pack_f16x2(acc[d][2] * inv_l, acc[d][3] * inv_l);
    *(u32x2*)(stage + (lane & 15) * RB + (16 * d + 4 * grp) * 2) = h;
  }
  constexpr int LPR = R / 8;     // lanes per row, 16 bytes each
  constexpr int RPI = 64 / LPR;  // rows per store
  static_assert(64 % LPR == 0 && 16 % RPI == 0, "row staging");
#pragma unroll
  for (int it = 0; it < 16 / RPI; ++it) {
    const int rr = it * RPI + lane / LPR, cb = (lane % LPR) * 16;
    const u32x4 v = *(const u32x4*)(stage + rr * RB + cb);
    *(u32x4*)((unsigned char*)(a.o_part + ((long long)(row0 + rr) * a.slots + slot) * a.r) + cb) = v;
  }
  if (grp == 0) {
    a.ml_part[prow * 2] = m_run * 0.6931471805599453f;  // back to natural-log units
    a.ml_part[prow * 2 + 1] = l_run;
  }
}

// Merge the slots of each (sequence, row) in slot order and write the
// un-absorb fragments: with w_p = exp(m_p - M) l_p and the stored
// Ohat_p = O_p / l_p, O = sum_p w_p Ohat_p / sum_p w_p.  Each lane owns eight
// adjacent dims (one 16-byte load of the fp16 row per slot); wave g sums the
// slots p = g mod 4 in slot order, the four waves' sums are added in a fixed
// order, and each wave writes a quarter of the dims.
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
  const int J = (a.len1 >= 0 ? a.len1 : a.offs[s + 1] - a.offs[s]) + a.block;
  const int ns = (J + a.C - 1) / a.C;
  const float* ml = a.ml_part + ((long long)row * a.slots + base) * 2;
  float mx = -INFINITY;
  for (int p = threadIdx.x; p < ns; p += 256) mx = fmaxf(mx, ml[2 * p]);
  mx = block_max256(mx, red);
  float l = 0.f;
  for (int p = threadIdx.x; p < ns; p += 256) {
    const float w = __expf(ml[2 * p] - mx) * ml[2 * p + 1];
    wgt[p] = w;
    l += w;
  }
  l = block_sum256(l, red);  // also orders the wgt writes before the reads below
  const float invL = 1.f / l;
  const int i = row / a.nh, h = row % a.nh;
  const int m = s * a.block + i;
  // lane ln of wave g holds dims 8 ln .. 8 ln + 7 (one 16-byte load per
  // slot) over slots g, g + 4, ...; four slots per lane in flight; the four
  // waves' sums are added in a fixed order
  const int g = threadIdx.x >> 6, ln = threadIdx.x & 63;
  const int nl = a.r / 8;  // lanes holding data (kv_lora % 16 == 0)
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (ln < nl) {
    const u32x4* op = (const u32x4*)(a.o_part + ((long long)row * a.slots + base) * a.r) + ln;
    for (int p0 = g; p0 < ns; p0 += 16) {
      u32x4 v[4];
      float w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + 4 * u;
        v[u] = p < ns ? op[(long long)p * nl] : u32x4{0u, 0u, 0u, 0u};
        w[u] = p < ns ? wgt[p] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += w[u] * fp16_bits_to_f32(v[u][e] & 0xFFFFu);
          acc[2 * e + 1] += w[u] * fp16_bits_to_f32(v[u][e] >> 16);
        }
    }
  }
  // every wave stores its sums, then wave g writes dims 8 ln + 2g, 8 ln + 2g + 1
  __shared__ float gsum[4][8][64];
  if (ln < nl) {
#pragma unroll
    for (int e = 0; e < 8; ++e) gsum[g][e][ln] = acc[e];
  }
  __syncthreads();
  if (ln < nl) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = 2 * g + k;
      frag_put(a.fd_uv, h, m, 8 * ln + e,
               ((gsum[0][e][ln] + gsum[1][e][ln]) + (gsum[2][e][ln] + gsum[3][e][ln])) * invL);
    }
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
  if (a.rows_pad % 64 || (long long)(a.rows_pad / 64) * a.slots > INT32_MAX) return hipErrorInvalidValue;
  // slots of whole key tiles, at most 2048 keys; pages of at least one key
  // tile, so a slot's keys span at most 64 pages (one per lane)
  if (a.C < KT || a.C % KT || a.C > 2048) return hipErrorInvalidValue;
  if (a.page_log2 >= 0 && (a.page_log2 < 5 || a.page_log2 > 24 || !a.table || a.max_pages < 1))
    return hipErrorInvalidValue;
  dim3 grid((a.rows_pad / 64) * a.slots), block(256);
  const bool paged = a.page_log2 >= 0;
  if (a.DQ == 576 && a.r == 512) {
    if (paged) hipLaunchKernelGGL((k_attn_bf16<18, 32, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attn_bf16<18, 32, false>), grid, block, 0, st, a);
  } else if (a.DQ == 96 && a.r == 64) {
    if (paged) hipLaunchKernelGGL((k_attn_bf16<3, 4, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_attn_bf16<3, 4, false>), grid, block, 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t st) {
  if (a.slots > MAX_COMBINE_SLOTS || a.r % 8 || a.r > 512) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_combine, dim3(a.rows, a.n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st) {
  if (a.latent > 1024 || a.r > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_f32, dim3(a.rows, a.n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
