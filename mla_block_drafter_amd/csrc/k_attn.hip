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
// row-major, four buffers deep, by direct-to-LDS copies.  S^T = K Q^T takes
// the key rows as the A operand (16-byte LDS reads), so the probabilities
// land with one query row per lane column, which is already the B-operand
// layout of P^T for O^T = V^T P^T (the 32 keys' order inside the MFMA
// reduction is permuted identically on both operands).  The V^T operand is
// gathered from the same row-major tile with transposing LDS reads (the
// value is c_kv, the first kv_lora columns of the key row), so no transposed
// copy is staged.  Two waves share 32 query rows and split the work so that
// every fragment read from LDS feeds two matrix instructions (see the
// kernel).  Partials per slot are merged in a fixed order by k_attn_combine
// or k_uv_combine.
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
  // a slot's last tile, or one that reaches the block's own keys: each row
  // chosen on its own (a runtime loop: this path runs once or twice per slot)
  auto row_ptr = [&](int j) {
    const uint16_t* c = cache + (long long)(trow + j - kt0) * a.latent;
    const uint16_t* k = bk + (long long)(s * a.block + (j - len)) * a.latent;
    const uint16_t* r = j < len ? c : k;
    return j < k_end ? r : dummy;
  };
#pragma unroll 1
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

// One wave-wide 16-byte-per-lane direct-to-LDS copy.  (Called from the
// kernel's lambdas through this device function: a lambda that names the
// builtin itself makes the host compilation drop the kernel's launch stub.)
__device__ __forceinline__ void copy_lds16(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
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

template <int N>
__device__ __forceinline__ void lds_wait_pair_x(u32x2& lo, u32x2& hi, u32x4& x) {
  asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(lo), "+v"(hi), "+v"(x) : "n"(N));
}

// Items of a tile step.  With the next-but-one tile's scores to compute
// (KEYS), value-fragment pairs and key fragments alternate (V0 K0 V1 K1 ...,
// then the rest of the longer list), so that the LDS-bound value reads and
// the matrix-core-bound score products overlap; otherwise only value pairs.
template <int ND, int NKB, bool KEYS>
struct StepItems {
  static constexpr int NP = KEYS ? (ND < NKB ? ND : NKB) : 0;  // alternating pairs
  static constexpr int N = ND + (KEYS ? NKB : 0);
  static constexpr bool is_v(int i) { return i < 2 * NP ? i % 2 == 0 : (KEYS ? ND > NKB : true); }
  static constexpr int idx(int i) { return i < 2 * NP ? i / 2 : i - NP; }
  static constexpr int ops(int i) { return is_v(i) ? 2 : 1; }  // LDS reads per item
  // LDS reads issued after item i when items up to i + W are issued
  template <int W>
  static constexpr int after(int i) {
    int n = 0;
    const int last = i + W < N - 1 ? i + W : N - 1;
    for (int j = i + 1; j <= last; ++j) n += ops(j);
    return n;
  }
};

// Waves 2p and 2p + 1 form pair p and share the query rows 32p .. 32p + 31
// of the workgroup's 64 (two 16-row MFMA blocks rb).  For S^T = K Q^T member
// h of the pair takes the keys of tile half h (16 keys) over every query
// dim, so each key fragment read from LDS feeds both row blocks; for
// O^T = V^T P^T it takes value dims h * R/2 .. (h + 1) * R/2 - 1 over all 32
// keys, so each value fragment also feeds both row blocks.  The members
// swap their bf16 probabilities through LDS (1 KiB per wave and tile).
// Per wave and tile this reads half the LDS bytes of one wave per 16 rows
// for the same matrix-core work.
//
// Software pipeline, one barrier per tile: step t multiplies P(t) by tile
// t's values, computes the scores of tile t + 2, and between those matrix
// instructions turns the scores of tile t + 1 (computed by the previous
// step) into probabilities, which the next barrier makes visible to the
// partner.  One wave per SIMD then keeps its matrix core busy while its LDS
// reads and exponentials are in flight.
template <int NKB, int NDT, bool PAGED>
__global__ __launch_bounds__(256, 1) void k_attn_bf16(AttnArgs a) {
  constexpr int DQ = NKB * 32;
  constexpr int R = NDT * 16;
  constexpr int CA = R / 8, CB = (DQ - R) / 8;
  constexpr int ND = NDT / 2;  // value dim tiles per wave
  using G = TileGeom<CA, CB>;
  static_assert(CA % 4 == 0 && NDT % 2 == 0, "each k-step reads one region; value dims split in two");
  static_assert(NBUF == 4, "tile buffers");
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[NBUF * G::BUF];
  __shared__ __attribute__((aligned(16))) u32x4 xp[2][4][64];  // own probabilities, by tile parity and wave
  __shared__ float xm[4][2][16];                              // row maxima of a wave's keys
  __shared__ float xl[4][2][16];                              // row sums of a wave's keys
  __shared__ int xv[4];                                       // redo votes

  const int ngrp = a.rows_pad / 64;
  const int pair_id = xcd_pair(blockIdx.x, gridDim.x);
  const int slot = pair_id / ngrp, rgrp = pair_id % ngrp;
  int s, p, len, off, J;
  slot_lookup(a, slot, s, p, len, off, J);
  if (s < 0) return;  // uniform over the workgroup
  const int k_begin = p * a.C;
  const int k_end = min(J, k_begin + a.C);
  const int ntiles = (k_end - k_begin + KT - 1) / KT;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps tile loads scalar
  const int mem = wave & 1;                                          // key half (S), value half (O)
  const int prow0 = rgrp * 64 + (wave >> 1) * 32;                    // the pair's first row
  const int grp = lane >> 4;

  const uint16_t* cache = (const uint16_t*)a.cache;
  const uint16_t* bk = (const uint16_t*)a.bkeys;
  const uint16_t* dummy = bk + (long long)s * a.block * a.latent;
  // paged caches: the page indices of this slot's keys (at most C / 32 = 64),
  // one per lane of a VGPR, read once here: no memory load may enter the tile
  // loop, whose LDS waits count on the shared counter
  const int pfirst = PAGED ? k_begin >> a.page_log2 : 0;
  int pgv = 0;
  if (PAGED) {
    const int32_t* tb = a.table + (long long)s * a.max_pages;
    pgv = tb[min(pfirst + lane, a.max_pages - 1)];
  }
  auto tile_row = [&](int kt0) { return PAGED ? paged_row(a, kt0, pfirst, pgv) : off + kt0; };
  auto issue = [&](int i) {  // key tile i of the slot into buffer i % NBUF
    const int kt0 = k_begin + i * KT;
    issue_tile<CA, CB, PAGED>(a, lane, wave, kt0, k_end, s, len, tile_row(kt0), cache, bk, dummy,
                              k_lds + (i % NBUF) * G::BUF);
  };

  // Q fragments (B operand of S^T = K Q^T): rows prow0 + 16 rb + (lane & 15),
  // dims 32 kb + 8 grp; read from LDS after the workgroup's copy (pass 0)
  bf16x8 qf[2][NKB];
  // The workgroup's 64 query rows into tile buffers 2 and 3 (rows 32 h ..
  // 32 h + 31 into buffer 2 + h) in the key tiles' layout, so that they are
  // read back like key fragments: one copy per workgroup instead of one load
  // per wave.
  auto issue_q = [&]() {
    const uint16_t* q = (const uint16_t*)a.q + ((long long)s * a.rows_pad + rgrp * 64) * DQ;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint16_t* dst = k_lds + (2 + h) * G::BUF;
      const uint16_t* src = q + (long long)(32 * h + wave) * DQ + 8 * lane;
#pragma unroll
      for (int i = 0; i < G::NB_A / 4; ++i, src += 4 * DQ)
        if (CA == 64 || lane < CA) copy_lds16(src, dst + (wave + 4 * i) * G::ROW_A);
      if (wave < G::NB_B) {
        const int r = wave * G::KPB + lane / CB, c = CA + ((lane % CB) ^ bswz<CB>(r));
        copy_lds16(q + (long long)(32 * h + r) * DQ + 8 * c, dst + G::SIZE_A + wave * 512);
      }
    }
  };
  // LDS element offsets inside a tile buffer
  const int kA = key_perm(lane & 15);                                 // key of this lane's A-operand row
  const int offA = (16 * mem + kA) * G::ROW_A + 8 * grp;              // + 32 kb
  const int offB = G::SIZE_A + (16 * mem + kA) * CB * 8;              // + chunk
  uint32_t bx[CB / 4];  // byte offsets of chunks 4 k + grp of region B for this lane's key
#pragma unroll
  for (int k = 0; k < CB / 4; ++k) bx[k] = 16 * ((4 * k + grp) ^ bswz<CB>(kA));
  const int kV = key_perm(4 * grp + ((lane & 15) >> 2));              // key this lane addresses for V
  const int offV = kV * G::ROW_A + 4 * (lane & 3) + 16 * ND * mem;   // + 16 h ROW_A + 16 d
  int keyS[4];                                                        // keys of this lane's score entries
#pragma unroll
  for (int j = 0; j < 4; ++j) keyS[j] = 16 * mem + key_perm(4 * grp + j);
  const uint32_t xp_par = lds_addr((const uint16_t*)&xp[0][wave ^ 1][lane]);
  constexpr uint32_t XP_PARITY = 4 * 64 * 16;  // bytes between the two tile parities

  const float c2 = a.tau * 1.4426950408889634f;  // base-2 score scale
  f32x4 acc[2][ND];
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f}, m_all[2] = {-INFINITY, -INFINITY};
  u32x4 pown;          // this wave's bf16 probabilities of a tile: row block rb in dwords 2 rb, 2 rb + 1
  f32x4 scn[2];        // scores of the tile after the current one (row block rb)
  float pr[2][4];      // probabilities being formed

  // Key-fragment read kb of the tile buffer at ab (region A) / bb (region B).
  auto read_k = [&](auto KI, uint32_t ab, uint32_t bb, u32x4& dst) {
    constexpr int kb = decltype(KI)::value;
    if constexpr (4 * kb < CA)
      lds_read_b128<2 * 32 * kb>(ab, dst);
    else
      lds_read_b128<0>(bb + bx[kb - CA / 4], dst);
  };
  // Softmax of one tile's scores sc[rb][r] (key kt0 + keyS[r], row 16 rb +
  // (lane & 15)) in pieces: 0 masks and takes the maxima, 1 + 4 rb + r forms
  // one probability, 9 packs them into pown.  Base-2 units
  // x = s tau log2(e): tau > 0, so the maximum of the raw products gives the
  // maximum of x.  Keys past the slot (last tile only) get -inf.
  auto sm_piece = [&](auto PI, f32x4 (&sc)[2], int kt0) {
    constexpr int pc = decltype(PI)::value;
    if constexpr (pc == 0) {
      if (kt0 + KT > k_end) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kt0 + keyS[r] >= k_end) sc[rb][r] = -INFINITY;
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        m_all[rb] = fmaxf(m_all[rb], fmaxf(fmaxf(sc[rb][0], sc[rb][1]), fmaxf(sc[rb][2], sc[rb][3])) * c2);
    } else if constexpr (pc <= 8) {
      constexpr int rb = (pc - 1) / 4, r = (pc - 1) % 4;
      pr[rb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[rb][r], c2, -m_run[rb]));
      l_run[rb] += pr[rb][r];  // this lane's keys only
    } else {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        pown[2 * rb] = pack_bf16x2(pr[rb][0], pr[rb][1]);
        pown[2 * rb + 1] = pack_bf16x2(pr[rb][2], pr[rb][3]);
      }
    }
  };
  constexpr int NPIECE = 10;
  // Scores of the tile in buffer tb (both row blocks).
  auto scores = [&](const uint16_t* tb, f32x4 (&sc)[2]) {
    sc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    sc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t ab = lds_addr(tb + offA), bb = lds_addr(tb + offB);
    constexpr int W0 = 6;
    u32x4 kf[NKB];
    static_for<W0 < NKB ? W0 : NKB>([&](auto KI) { read_k(KI, ab, bb, kf[decltype(KI)::value]); });
    static_for<NKB>([&](auto KI) {
      constexpr int kb = decltype(KI)::value;
      if constexpr (kb + W0 < NKB) read_k(std::integral_constant<int, kb + W0>{}, ab, bb, kf[kb + W0]);
      constexpr int ahead = NKB - 1 - kb < W0 ? NKB - 1 - kb : W0;
      lds_wait<ahead>(kf[kb]);
      const bf16x8 kfb = __builtin_bit_cast(bf16x8, kf[kb]);
      sc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfb, qf[0][kb], sc[0], 0, 0, 0);
      sc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfb, qf[1][kb], sc[1], 0, 0, 0);
    });
  };

  // The query rows into buffers 2 and 3 (free until tile 2, issued after
  // the reference exchange, once every wave has read its query fragments)
  // and tiles 0 and 1, then the wait: direct-to-LDS copies complete in no
  // fixed order with respect to each other, so only a full count proves
  // that a tile has landed; each wave waits for all of its copies and the
  // barrier covers every wave's.
  issue_q();
#pragma unroll 1
  for (int i = 0; i < min(2, ntiles); ++i) issue(i);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  {
    const uint16_t* qb = k_lds + (2 + (wave >> 1)) * G::BUF;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int rr = 16 * rb + (lane & 15);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        qf[rb][kb] = 4 * kb < CA ? *(const bf16x8*)(qb + rr * G::ROW_A + 32 * kb + 8 * grp)
                                 : *(const bf16x8*)(qb + G::SIZE_A + rr * CB * 8 +
                                                    8 * ((4 * (kb - CA / 4) + grp) ^ bswz<CB>(rr)));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }

  // Softmax reference: the first tile's row maximum (pass 0).  The tile loop
  // never rescales the accumulators; if a later score exceeds the reference
  // by more than REDO_SLACK, the workgroup redoes the slot once with the
  // exact row maximum (pass 1).
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[rb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
      l_run[rb] = 0.f;
      if (pass == 1) m_run[rb] = m_all[rb];
    }
    // Pass 1 fetches tiles 0 and 1 again (pass 0 did so with the query rows,
    // before this loop) and streams tile 2 in during the prologue.
    if (pass == 1) {
#pragma unroll 1
      for (int i = 0; i < min(2, ntiles); ++i) issue(i);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    {  // S and P of tile 0 (pass 0: the reference is its row maximum over both halves)
      f32x4 sc[2];
      scores(k_lds, sc);
      sm_piece(std::integral_constant<int, 0>{}, sc, k_begin);
      if (pass == 0) {
        float tm[2];  // row maxima of this wave's keys of tile 0
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          tm[rb] = fmaxf(m_all[rb], __shfl_xor(m_all[rb], 16, 64));
          tm[rb] = fmaxf(tm[rb], __shfl_xor(tm[rb], 32, 64));
          if (grp == 0) xm[wave][rb][lane] = tm[rb];
        }
        __syncthreads();
        // both members take the same reference (max is commutative)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) m_run[rb] = fmaxf(tm[rb], xm[wave ^ 1][rb][lane & 15]);
      }
      // tile 2 into buffer 2: in pass 0 every wave has read its query
      // fragments (the exchange's barrier above), in pass 1 the prologue's
      // barrier ended the previous pass
      if (2 < ntiles) issue(2);
      static_for<NPIECE - 1>([&](auto PI) { sm_piece(std::integral_constant<int, decltype(PI)::value + 1>{}, sc, k_begin); });
      *(u32x4*)&xp[0][wave][lane] = pown;
    }
    if (1 < ntiles) scores(k_lds + G::BUF, scn);

    // Step t: barrier (P(t) of both members written, tile t + 2 landed,
    // every wave done with step t - 1, whose value tile t - 1 the refill of
    // tile t + 3 overwrites), then P(t) V(t), S(t + 2) and P(t + 1).
    auto step = [&](auto K2, auto K1, int t) {
      constexpr bool KEYS = decltype(K2)::value;  // tile t + 2 exists
      constexpr bool NEXT = decltype(K1)::value;  // tile t + 1 exists
      using IT = StepItems<ND, NKB, KEYS>;
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if constexpr (KEYS)  // (a step without tile t + 2 has no tile t + 3 either)
        if (t + NBUF - 1 < ntiles) issue(t + NBUF - 1);
      const uint32_t vaddr = lds_addr(k_lds + (t % NBUF) * G::BUF + offV);
      const uint16_t* t2 = k_lds + ((t + 2) % NBUF) * G::BUF;
      const uint32_t ab = lds_addr(t2 + offA), bb = lds_addr(t2 + offB);
      const int kt1 = k_begin + (t + 1) * KT;
      u32x4 par;
      lds_read_b128<0>(xp_par + (t & 1) * XP_PARITY, par);

      constexpr int W = 6;
      u32x2 vlo[ND], vhi[ND];
      u32x4 kf[KEYS ? NKB : 1];
      f32x4 sn[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      auto issue_item = [&](auto II) {
        constexpr int i = decltype(II)::value;
        constexpr int j = IT::idx(i);
        if constexpr (IT::is_v(i))
          tr_read_pair<32 * j, 32 * j + 2 * 16 * G::ROW_A>(vaddr, vlo[j], vhi[j]);
        else
          read_k(std::integral_constant<int, j>{}, ab, bb, kf[j]);
      };
      static_for<W < IT::N ? W : IT::N>(issue_item);
      bf16x8 pf[2];
      static_for<IT::N>([&](auto II) {
        constexpr int i = decltype(II)::value;
        constexpr int j = IT::idx(i);
        if constexpr (i + W < IT::N) issue_item(std::integral_constant<int, i + W>{});
        constexpr int after = IT::template after<W>(i);
        if constexpr (IT::is_v(i)) {
          if constexpr (j == 0) {
            lds_wait_pair_x<after>(vlo[0], vhi[0], par);
            // k slots 0..3: keys of tile half 0, 4..7: half 1
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              const u32x4 lo_first = {pown[2 * rb], pown[2 * rb + 1], par[2 * rb], par[2 * rb + 1]};
              const u32x4 hi_first = {par[2 * rb], par[2 * rb + 1], pown[2 * rb], pown[2 * rb + 1]};
              pf[rb] = __builtin_bit_cast(bf16x8, mem ? hi_first : lo_first);
            }
          } else {
            lds_wait_pair<after>(vlo[j], vhi[j]);
          }
          const bf16x8 v8 = __builtin_bit_cast(bf16x8, u32x4{vlo[j][0], vlo[j][1], vhi[j][0], vhi[j][1]});
          acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, pf[0], acc[0][j], 0, 0, 0);
          acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, pf[1], acc[1][j], 0, 0, 0);
        } else {
          lds_wait<after>(kf[j]);
          const bf16x8 kfb = __builtin_bit_cast(bf16x8, kf[j]);
          sn[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfb, qf[0][j], sn[0], 0, 0, 0);
          sn[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfb, qf[1][j], sn[1], 0, 0, 0);
        }
        // probabilities of tile t + 1 between the matrix instructions (after
        // item 0, whose operands already hold this step's P(t))
        if constexpr (NEXT && i < NPIECE) sm_piece(std::integral_constant<int, i>{}, scn, kt1);
      });
      if constexpr (NEXT) {
        static_for<(IT::N < NPIECE ? NPIECE - IT::N : 0)>(
            [&](auto PI) { sm_piece(std::integral_constant<int, IT::N + decltype(PI)::value>{}, scn, kt1); });
        *(u32x4*)&xp[(t + 1) & 1][wave][lane] = pown;
      }
      if constexpr (KEYS) {
        scn[0] = sn[0];
        scn[1] = sn[1];
      }
    };
    int t = 0;
#pragma unroll 1
    for (; t + 2 < ntiles; ++t) step(std::true_type{}, std::true_type{}, t);
    if (t + 1 < ntiles) step(std::false_type{}, std::true_type{}, t++);
    step(std::false_type{}, std::false_type{}, t);

    // combine the four lanes of each row (fixed butterfly: same bits in all)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      m_all[rb] = fmaxf(m_all[rb], __shfl_xor(m_all[rb], 16, 64));
      m_all[rb] = fmaxf(m_all[rb], __shfl_xor(m_all[rb], 32, 64));
      l_run[rb] += __shfl_xor(l_run[rb], 16, 64);
      l_run[rb] += __shfl_xor(l_run[rb], 32, 64);
      if (grp == 0) xl[wave][rb][lane] = l_run[rb];
    }
    // one barrier: every wave is done with the tile buffers, the row sums of
    // both halves and the redo votes are visible
    const float lim = REDO_SLACK * 1.4426950408889634f;
    const bool vote = pass == 0 && __any(m_all[0] > m_run[0] + lim || m_all[1] > m_run[1] + lim);
    if (lane == 0) xv[wave] = vote;
    __syncthreads();
    if (pass == 1 || !(xv[0] | xv[1] | xv[2] | xv[3])) break;
    // the exact row maximum over both halves is the redo's reference
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      if (grp == 0) xm[wave][rb][lane] = m_all[rb];
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) m_all[rb] = fmaxf(m_all[rb], xm[wave ^ 1][rb][lane & 15]);
  }

  // ---- partials: O^T[dim][row] / l, a convex combination of value rows,
  //      stored as fp16 (11-bit significand, finer than the bf16 operands);
  //      layout [row][slot][dim] so the merge of one row reads contiguous
  //      memory; l >= 1 (the reference key contributes exp(0)).  The pair's
  //      row sums add both key halves; the 64 rows are staged in LDS (the
  //      barrier above ended every wave's tile reads) and stored as whole
  //      rows. ----
  float inv_l[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    l_run[rb] += xl[wave ^ 1][rb][lane & 15];  // the same sum in both members
    inv_l[rb] = 1.f / l_run[rb];
  }
  constexpr int RB = R * 2 + 16;  // bytes per staged row (the pad spreads the banks)
  unsigned char* stage = (unsigned char*)k_lds;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      u32x2 h;
      h[0] = pack_f16x2(acc[rb][d][0] * inv_l[rb], acc[rb][d][1] * inv_l[rb]);
      h[1] = pack_f16x2(acc[rb][d][2] * inv_l[rb], acc[rb][d][3] * inv_l[rb]);
      const int lrow = (wave >> 1) * 32 + 16 * rb + (lane & 15);
      *(u32x2*)(stage + lrow * RB + (16 * ND * mem + 16 * d + 4 * grp) * 2) = h;
    }
  __syncthreads();
  constexpr int LPR = R / 8;     // lanes per row, 16 bytes each
  constexpr int RPI = 64 / LPR;  // rows per store
  static_assert(64 % LPR == 0 && 16 % RPI == 0, "row staging");
#pragma unroll
  for (int it = 0; it < 16 / RPI; ++it) {
    const int rr = wave * 16 + it * RPI + lane / LPR, cb = (lane % LPR) * 16;
    const u32x4 v = *(const u32x4*)(stage + rr * RB + cb);
    *(u32x4*)((unsigned char*)(a.o_part + ((long long)(rgrp * 64 + rr) * a.slots + slot) * a.r) + cb) = v;
  }
  if (mem == 0 && grp == 0) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const long long prow = (long long)(prow0 + 16 * rb + lane) * a.slots + slot;
      a.ml_part[prow * 2] = m_run[rb] * 0.6931471805599453f;  // back to natural-log units
      a.ml_part[prow * 2 + 1] = l_run[rb];
    }
  }
}

// Merge the slots of each (sequence, row) in slot order and write the
// un-absorb fragments: with w_p = exp(m_p - M) l_p and the stored
// Ohat_p = O_p / l_p, O = sum_p w_p Ohat_p / sum_p w_p.  One wave per
// (sequence, row), four per workgroup: lane p holds slot p's weight (64
// slots per round), lane l owns dims 8 l .. 8 l + 7 (one 16-byte load of the
// fp16 row per slot), eight slots' loads are in flight at a time, and the
// slots are added in order with each weight read from its lane.
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);  // s * rows + row
  const int s = item / a.rows, row = item % a.rows;       // row = i * nh + h
  if (s >= a.n_seq) return;                               // the whole wave
  int base = 0;
  for (int t = 0; t < s; ++t) base += (a.offs[t + 1] - a.offs[t] + a.block + a.C - 1) / a.C;
  const int J = (a.len1 >= 0 ? a.len1 : a.offs[s + 1] - a.offs[s]) + a.block;
  const int ns = (J + a.C - 1) / a.C;
  const float* ml = a.ml_part + ((long long)row * a.slots + base) * 2;
  float mx = -INFINITY;
  for (int p = lane; p < ns; p += 64) mx = fmaxf(mx, ml[2 * p]);
  mx = wave_max(mx);
  const int nl = a.r / 8;  // lanes holding data (kv_lora % 8 == 0, <= 512)
  const u32x4* op = (const u32x4*)(a.o_part + ((long long)row * a.slots + base) * a.r) + (lane < nl ? lane : 0);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int c0 = 0; c0 < ns; c0 += 64) {
    const int pl = c0 + lane;
    const float wl = pl < ns ? __expf(ml[2 * pl] - mx) * ml[2 * pl + 1] : 0.f;
    L += wave_sum(wl);
    const int n = min(64, ns - c0);
    for (int u0 = 0; u0 < n; u0 += 8) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = u0 + u < n && lane < nl ? op[(long long)(c0 + u0 + u) * nl] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = u0 + u < n ? lane_value(wl, u0 + u) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += w * fp16_bits_to_f32(v[u][e] & 0xFFFFu);
          acc[2 * e + 1] += w * fp16_bits_to_f32(v[u][e] >> 16);
        }
      }
    }
  }
  if (lane < nl) {
    const float invL = 1.f / L;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= invL;
    const int i = row / a.nh, h = row % a.nh;
    frag_put8(a.fd_uv, h, s * a.block + i, 8 * lane, acc);
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
  hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)(((long long)a.rows * a.n_seq + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st) {
  if (a.latent > 1024 || a.r > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_f32, dim3(a.rows, a.n_seq), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dspark
