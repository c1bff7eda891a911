// Launch interfaces of the DSpark HIP kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dspark {

// ------------------------------------------------------------- skinny GEMM --
// out[split][m][col] = sum over the split's k range of act[m][k] * W[col][k]
// for the M activation rows (M = 7 per sequence), W streamed once from HBM.
enum { GEMV_STORE = 0, GEMV_MARKOV = 1, GEMV_QLAT = 2, GEMV_FRAG = 3, GEMV_OWN = 4 };

// Column-owning GEMM (GEMV_OWN): one workgroup owns 32 output columns (two
// 16-row tiles; for the fused gate/up matrix the two gate tiles and the two
// up tiles of those columns), its waves split the reduction and add their
// partial sums in LDS in a fixed order, and one wave runs a fused epilogue:
//   OWN_STORE:  x_out = W a (rows of the residual-stream layout) + chunk sums of x^2;
//   OWN_RESID:  x_out = x_in + W a, chunk sums of x^2, fragments of g1 * x_out
//               for the next GEMM, optional chunk sums of g1 * x_out * dotw;
//   OWN_SWIGLU: fragments of silu(W_g a) * (W_u a) for the next GEMM.
// Chunks are the workgroup's 32 columns (chunk index = workgroup index).
enum { OWN_STORE = 1, OWN_RESID = 2, OWN_SWIGLU = 3 };
constexpr int OWN_COLS = 32;

// Partial sums of squares per (row, column chunk), row stride SSQ_LD: chunks
// of 256 columns from the column-parallel kernels, of OWN_COLS columns from
// the column-owning GEMMs.
constexpr int SSQ_LD = 256;

// Per-row RMSNorm scale rs[m] = 1/sqrt(sum_c ssq[m][c] * invn + eps); ssq = null: 1.
struct RowScale {
  const float* ssq;
  int nch;
  float invn, eps;
};

// Sum of the nch <= SSQ_LD chunk values of one row, by a whole wave (all 64
// lanes call it with the same arguments): every chunk is loaded at once and
// added in a fixed order (per lane, then a butterfly), so the cost is one
// memory round trip and every lane returns the same bits.
__device__ __forceinline__ float chunk_lane_sum(const float* row, int nch, int lane) {
  float t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = lane + 64 * i < nch ? row[lane + 64 * i] : 0.f;
  return (t[0] + t[1]) + (t[2] + t[3]);
}
__device__ __forceinline__ float chunk_sum_wave(const float* row, int nch) {
  return wave_sum(chunk_lane_sum(row, nch, threadIdx.x & 63));
}

__device__ __forceinline__ float row_scale_wave(const RowScale& s, int m) {
  if (!s.ssq) return 1.f;
  return rsqrtf(chunk_sum_wave(s.ssq + (long long)m * SSQ_LD, s.nch) * s.invn + s.eps);
}

struct GemvArgs {
  PackedMat w;
  const void* act;        // input buffer (STORE/QLAT/FRAG) or plain gather table (MARKOV)
  long long act_gstride;  // elements per group of the input buffer
  int act_ld;             // fp32 rows: row stride (elements)
  int M;                  // valid activation rows
  int hilo;               // bf16 family with M <= 8
  int ksteps_per_split;   // in 32-wide blocks (bf16 family) or 16-wide groups (f32)
  int ksteps_lo;          // GEMV_OWN with 8 waves: k steps of waves 4..7 (waves 0..3 take ksteps_per_split)
  RowScale rs;            // optional output row scale (STORE, FRAG)
  // STORE
  float* out;             // [S][M][out_ld]
  long long out_ld;
  long long out_split_stride;
  // QLAT: output (m, head g, column j) -> query buffer row (m % block) * nh + g
  void* q; int q_f32, DQ, rows_pad, nh;
  // FRAG: output (m, col) -> fragments of the next GEMM
  FragDesc fd;
  // MARKOV: M = n_seq; activation row m = W1[t_prev(m)], t_prev resolved in-kernel
  int gather_ld;          // elements per table row (>= Kp)
  const int32_t* prev_token;
  const int32_t* forced;
  unsigned long long* keys;  // [n_seq][block][KEY_SLOTS]
  int step, block;
  const float* z;         // [n_seq*block][V]
  float* logits;          // optional [n_seq][block][V]
  // OWN (column-owning GEMM, see GEMV_OWN): fused epilogue
  int epi;                // OWN_STORE / OWN_RESID / OWN_SWIGLU
  int tile_jump;          // tiles j >= TPW/2 of a workgroup sit tile_jump tiles further (gate/up: up rows)
  const float* x_in;      // RESID: residual stream in [M][G]
  float* x_out;           // STORE / RESID: output [M][G] (may alias x_in)
  const float* g1;        // RESID: gain of the next GEMM's input (fragments of g1 * x_out); null: none
  float* ssq_out;         // STORE / RESID: [M][SSQ_LD] chunk sums of x_out^2
  const float* dotw;      // RESID: chunk sums of g1 * x_out * dotw -> dot_out (null: none)
  float* dot_out;
};

// Waves of a split-K workgroup whose activation chunks are shared through LDS
// (amode 5): every staged chunk feeds that many x TPW weight tiles.  FP8
// weights (1 byte per weight against 2 per activation element) read half as
// many activation bytes with eight waves; the BF16 lm_head measured faster
// with four.
constexpr int lds_bf_waves(int fmt) { return fmt == DT_FP8 ? 8 : 4; }
constexpr int LDS_BF_CK = 4;  // amode 5: k blocks per staged chunk

struct GemvPlan {
  int MT, TPW, S, ksteps_per_split, hilo;
  int ksteps_lo;          // GEMV_OWN with 8 waves: k steps of waves 4..7
  int nw;                 // GEMV_OWN: waves per workgroup splitting the reduction; 0: split-K over workgroups
  int grid_x;
  int amode;              // activation operand: 0 prepared global fragments,
                          // 1 fp32 rows -> bf16 fragments in LDS,
                          // 2 fp32 rows -> int8 hi/lo codes in LDS (Q8_0, M <= 8)
                          // 3 int8 hi/lo fragments from the producer (Q8_0, M <= 8)
                          // 5 bf16 fragments of several m-tiles shared through LDS (FP8 / BF16, M > 8)
};

// i8_in: the producer of the input can write int8 fragments (frag_put_wave /
// the int8 FRAG epilogue), which Q8_0 weights with M <= 8 then read directly.
GemvPlan plan_gemv(const PackedMat& w, int M, bool allow_split, bool gather = false, bool i8_in = false);
// Column-owning plan (M <= 8; 32 output columns per workgroup).  swiglu: the
// fused gate/up matrix (G = 2 inter rows, gate then up).  Returns a plan with
// nw == 0 when the shape or format is not covered (the caller then uses
// plan_gemv and separate reduction kernels).
GemvPlan plan_own(const PackedMat& w, int M, bool swiglu, bool i8_in);
hipError_t launch_gemv(const GemvArgs& a, const GemvPlan& p, int mode, hipStream_t st);

// --------------------------------------------------------------- attention --
struct AttnArgs {
  const void* q;          // [n_seq][rows_pad][DQ] (bf16 or f32)
  const void* cache;      // [total][latent]
  const void* bkeys;      // [n_seq*block][latent]
  const int32_t* offs;    // [n_seq + 1]
  int n_seq, block, nh, rows, rows_pad, latent, r, DQ;
  int C;                  // keys per split (multiple of 32)
  int slots;              // slot bound (grid.y)
  int len1;               // n_seq == 1: the cache length (== offs[1]), so no lookup; else -1
  // paged caches (page_log2 >= 0): cache = page pool [pages][1 << page_log2][latent];
  // token j of sequence s in page table[s * max_pages + (j >> page_log2)]
  const int32_t* table;
  int page_log2;          // -1: packed rows, sequence s from offs[s]
  int max_pages;
  float tau;
  uint16_t* o_part;       // [rows_pad][slots][r] fp16: each slot's O / l
  float* ml_part;         // [rows_pad][slots][2]: each slot's (m, l)
  FragDesc fd_uv;         // output fragments (un-absorb input, grouped by head)
};

// Attention combine fused with the un-absorb GEMM (one sequence, M <= 8,
// at most UVC_MAX_SLOTS slots).
constexpr int UVC_MAX_SLOTS = 256;
struct UvCombineArgs {
  GemvArgs g;               // W_UV grouped by head, M, fd = o_proj fragments, hilo
  const uint16_t* o_part;   // attention partials [rows_pad][slots][r] fp16 (O / l)
  const float* ml_part;     // [rows_pad][slots][2] (m, l)
  int slots, C, block, nh, r;
  int len1;                 // the sequence's cache length
};
bool uv_combine_supported(const GemvArgs& g, int n_seq, int slots);
hipError_t launch_uv_combine(const UvCombineArgs& a, hipStream_t st);

bool attn_bf16_supported(int DQ, int r);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st);
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t st);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st);

// ------------------------------------------------------------ elementwise --
struct InitArgs {
  void* zero_ptr;         // 16-byte aligned
  long long zero_bytes;   // multiple of 16
  // fc input fragments (optional: captured == nullptr to skip)
  const void* captured;   // [n_seq][ncap][block][H]
  int cap_f32;
  int n_seq, ncap, block, H;
  FragDesc fd_fc;
  // RoPE table (optional: rope == nullptr to skip): rope[m][p] = (cos, sin) of
  // pos(m) * freqs[p] for row m = s * block + i at position kv_len(s) + i
  float* rope;            // [n_seq * block][npairs][2]
  const int32_t* offs;    // [n_seq + 1] cache offsets
  const int32_t* positions;  // optional [n_seq * block]: position of row m (instead of the offsets)
  const double* freqs;    // [npairs]
  int npairs;
};
hipError_t launch_init(const InitArgs& a, hipStream_t st);

// Streaming-read probe (measurement): READ_PROBE_WGS workgroups, one XOR word each.
constexpr int READ_PROBE_WGS = 2048;
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t st);

// Split-K partial sums [S][M][ld] of one GEMM.
struct PartIn {
  const float* part;
  int S;
  long long ld, ss;
};

enum { RP_COPY = 0, RP_SUM = 1, RP_ADD = 2, RP_NORM = 3 };
struct ResidPost {
  PartIn p;
  int mode;               // COPY: x = x_in; SUM: x = sum p; ADD: x = x_in + sum p;
                          // NORM: x = g0 * x_in * rs_in
  const float* x_in; float* x_out;
  RowScale rs_in; const float* g0;
  int M, H;
  const float* g1;        // fragments of g1 * x for the next GEMM (null: none)
  FragDesc fd;
  float* ssq_out;         // [M][SSQ_LD] chunk sums of x^2 (null: none)
  const float* dotw;      // chunk sums of g1 * x * dotw -> dot_out (null: none)
  float* dot_out;
};
hipError_t launch_post_resid(const ResidPost& a, hipStream_t st);

struct QkvaPost {
  PartIn p; RowScale rs_in;
  int M, q_lora, r, dr, latent, block;
  const float* g_qa; const float* g_kva; float eps;
  FragDesc fd_qb; float* ssq_cq;
  void* bkeys; int kv_f32;   // [M][latent]
  const float* rope;          // [M][dr/2][2] (cos, sin), written by k_init
};
hipError_t launch_post_qkva(const QkvaPost& a, hipStream_t st);

// Cache append: the latent row of each new row m (kv_a partials, columns
// 0 .. latent - 1) written to cache row slot[m].
struct KvRowPost {
  PartIn p; RowScale rs_in;
  int M, r, dr, latent;
  const float* g_kva; float eps;
  const float* rope;          // [M][dr/2][2] (cos, sin), written by k_init
  void* dst; int dst_f32;     // cache [rows][latent]
  const int64_t* slot;        // [M] destination rows
};
hipError_t launch_post_kv_rows(const KvRowPost& a, hipStream_t st);

struct QbPost {
  PartIn p; RowScale rs;
  int M, nh, dn, dr, r, block, DQ, rows_pad;
  FragDesc fd_uk;             // absorb input, groups = heads
  void* q; int q_f32;         // [n_seq][rows_pad][DQ]
  const float* rope;          // [M][dr/2][2] (cos, sin), written by k_init
};
hipError_t launch_post_qb(const QbPost& a, hipStream_t st);

// q_b post fused with the W_UK absorb GEMM (M <= 8, bf16 W_UK, qk_nope 128):
// g is the absorb GEMM (query-buffer output), qb the post (fd_uk unused).
struct QbAbsorbArgs {
  GemvArgs g;
  QbPost qb;
};
bool qb_absorb_supported(const GemvArgs& g, const QbPost& p);
hipError_t launch_qb_absorb(const QbAbsorbArgs& a, hipStream_t st);

struct SwigluPost {
  PartIn p; RowScale rs;
  int M, inter;
  FragDesc fd;
};
hipError_t launch_post_swiglu(const SwigluPost& a, hipStream_t st);

// Persistent Markov rollout (k_markov.hip): W2 held in registers across the
// block's positions; one launch for all of them.
struct MarkovArgs {
  const void* w2;             // packed bf16 W2, tiles of 16 vocabulary rows, KB k blocks each
  int tiles;                  // ceil(vocab / 16)
  const void* w1; int w1_ld;  // bf16 W1 rows (gather table)
  int vocab, M, block;        // M = n_seq <= 16
  const int32_t* prev_token; const int32_t* forced;
  const float* z;             // lm_head logits [n_seq * block][vocab]
  float* logits;              // optional [n_seq][block][vocab]
  unsigned long long* slots;  // [block][M][workgroups] argmax keys, zeroed
  int max_wgs;                // workgroups the slot array was sized for
  unsigned* err;              // error flag, zeroed
  const float* sample_u;      // optional [n_seq][block][vocab] uniforms: Gumbel-max draws
  float inv_temp;             // 1 / temperature (with sample_u)
  int spin_limit;             // polls per position before expiry: 0 default, < 0 expire at once
  const int* fallback;        // candidate pruning ran: nothing to do unless *fallback (null: always run)
};
int markov_rollout_wgs(int tiles);

// Markov rollout by exact candidate pruning (k_markov_prune.hip).
constexpr int MK_CHUNK = 8192;    // vocabulary rows per candidate workgroup (1024 threads)
constexpr int MK_CAPC = 8;        // list entries kept per (position, chunk)
constexpr int MK_MAXCH = 32;      // chunks per position: vocab <= MK_MAXCH * MK_CHUNK
constexpr int MK_CAPG = 16;       // candidates kept per position after the global threshold
constexpr int MK_MAX_BLOCK = 8;   // positions per block
inline int markov_prune_chunks(int vocab) { return (vocab + MK_CHUNK - 1) / MK_CHUNK; }
struct MarkovPruneArgs {
  const float* z;             // lm_head logits [n_seq * block][vocab]
  const float* n2;            // [vocab] upper bounds of W2's row norms
  const unsigned* w1max;      // upper bound of W1's largest row norm (float bits)
  int vocab, n_seq, block, R, KB, nch;
  const void* w2;             // packed bf16 W2 (16-row tiles, KB k blocks)
  const void* w1; int w1_f32, w1_ld;
  const int32_t* prev_token; const int32_t* forced;
  float* lch;                 // [M][nch] largest lower end of each chunk
  int* ccnt;                  // [M][nch] rows of the chunk whose upper end reaches it
  u32x4* list;                // [M][nch][MK_CAPC] the first of them: (row, z bits, bound bits, 0)
  int* fallback;              // zeroed; 1 = too many candidates: the full rollout runs
  RowScale rs_final; const float* dot; int nch_dot;
  const float* conf_wm; const float* conf_b;
  int32_t* tokens; float* conf; int32_t* status;
};
bool markov_prune_supported(int R, int block, int vocab);
hipError_t launch_markov_prune(const MarkovPruneArgs& a, hipStream_t st);
// Upper bounds of the row L2 norms of rows [V][R] (row stride ld, bf16 or
// f32): nrm[v] (optional) and their maximum into *maxbits (optional, zeroed).
hipError_t launch_row_norms(const void* rows, int f32, long long ld, int R, int V, float* nrm, unsigned* maxbits,
                            hipStream_t st);
bool markov_rollout_supported(int KB, int M, int vocab);
hipError_t launch_markov_rollout(const MarkovArgs& a, int KB, hipStream_t st);

// Verification of a sampled draft block (token rule or block rule).
constexpr int DSPARK_VERIFY_TOKEN_C = 0, DSPARK_VERIFY_BLOCK_C = 1;
struct VerifyArgs {
  int n_seq, block, vocab, method;
  float inv_temp;
  const int32_t* draft;       // [n_seq][block]
  const float* dlog;          // [n_seq][block][vocab] draft logits
  const float* tlog;          // [n_seq][block + 1][vocab] target logits
  const float* u;             // [n_seq][block + 1] uniforms: acceptance, then the draw
  float* stats;               // [n_seq][block + 1][verify_nch()][4]
  float* resid;               // [n_seq][block][verify_nch()][2]
  float* probs;               // [n_seq][block + 1][8] row normalisers, p(x), q(x), prefix weight
  int32_t* out_len; int32_t* out_token;
};
int verify_nch();
hipError_t launch_verify(const VerifyArgs& a, hipStream_t st);

struct MarkovFinalArgs {
  const unsigned long long* keys;
  const int32_t* prev_token; const int32_t* forced;
  const void* w1; int w1_f32; int w1_ld; int R;
  const float* conf_wm; const float* conf_b;
  const float* dot; int nch;  // chunk sums of (g_final * x) . w_h, row stride SSQ_LD
  RowScale rs_final;
  const float* x; const float* g_final; int H;
  float* hidden;              // optional [M][H] = rs * g_final * x
  int32_t* tokens; float* conf;
  int n_seq, block, vocab;
  // rollout mode: argmax keys come from the rollout's slots [block][n_seq][nwg]
  // instead of keys; nonzero *rollout_err (an expired poll) gives tokens of -1
  const unsigned long long* slots; int nwg;
  const unsigned* rollout_err;
  int32_t* status;            // optional [1]: 1 if the rollout expired, else 0
  const int* fallback;        // candidate pruning ran: nothing to do unless *fallback (null: always run)
};
hipError_t launch_markov_final(const MarkovFinalArgs& a, hipStream_t st);

hipError_t launch_accept_len(const int32_t* d, const int32_t* v, int n_seq, int block, int32_t* out,
                             hipStream_t st);

// -------------------------------------------------------- static scratch --
// Address and size of this device's copy of the library's static scratch
// (dspark_static.hip); the address is looked up once per device.
hipError_t static_scratch(void** ptr, size_t* bytes);

// ---------------------------------------------------------------- repack --
enum { XF_NORMAL = 0, XF_UK = 1, XF_UV = 2 };
struct RepackArgs {
  const void* src; int src_fmt; const float* src_scales;
  long long src_rows, src_cols;   // source tensor geometry
  int xf;                         // transform
  int dn, dv, r;                  // kv_b geometry (XF_UK / XF_UV)
  unsigned char* codes; void* scales;  // destination planes
  PackedMat dst;
  int row0;                       // destination logical row of source row 0 (XF_NORMAL)
  int nrows;                      // destination logical rows written
};
hipError_t launch_repack(const RepackArgs& a, hipStream_t st);
hipError_t launch_dequant(const PackedMat& w, float* out, hipStream_t st);

}  // namespace dspark
