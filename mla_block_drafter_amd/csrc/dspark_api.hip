// Host side of the C ABI declared in include/dspark.h: validation, the packed
// weight plan and repack, the per-call workspace plan, and the launch sequence
// of one draft pass (all launches asynchronous on the caller's stream).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/dspark.h"
#include "kernels.h"

using namespace dspark;

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIPCHK(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(DSPARK_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

inline long long rup(long long a, long long b) { return (a + b - 1) / b * b; }
inline long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

// ----------------------------------------------------------- packed plan --
struct Mat {
  PackedMat pm{};
  long long codes_off = -1, scales_off = -1, codes_bytes = 0, scales_bytes = 0;
  bool present = false;
};

// Bytes of one packed row of n reduction elements.
long long code_bytes(int fmt, long long n) {
  return fmt == DT_F32 ? 4 * n : fmt == DT_BF16 ? 2 * n : fmt == DT_MXFP4 ? n / 2 : n;
}

// Bytes of the scale plane per 16-row tile.
long long scale_tile_bytes(const PackedMat& p) {
  return p.fmt == DT_Q8_0 ? (p.KB / 2) * 16 * 4 : p.fmt == DT_FP8 ? 16 * 4 : p.fmt == DT_MXFP4 ? (p.KB / 4) * 16 * 4 : 0;
}

void mat_geom(Mat& m, int fmt, int ngroups, int G, int K) {
  PackedMat& p = m.pm;
  p.fmt = fmt;
  p.ngroups = ngroups;
  p.G = G;
  p.TG = (int)cdiv(G, 16);
  p.K = K;
  p.Kp = (int)rup(K, 64);
  p.KB = p.Kp / 32;
  const long long T = (long long)ngroups * p.TG;
  m.codes_bytes = T * 16 * code_bytes(fmt, p.Kp);
  m.scales_bytes = fmt == DT_Q8_0 ? T * (p.KB / 2) * 16 * 4
                   : fmt == DT_FP8 ? T * 16 * 4
                   : fmt == DT_MXFP4 ? T * (p.KB / 4) * 16 * 4 : 0;
  m.present = true;
}

struct Layer {
  Mat qkva, qb, uk, uv, o, gu, down;
  long long in_norm = -1, q_a_norm = -1, kv_a_norm = -1, post_norm = -1;
};

}  // namespace

struct dspark_model {
  dspark_config c{};
  unsigned char* base = nullptr;
  long long bytes = 0;
  bool layers_only = false;
  bool plan_only = false;  // DSPARK_CFG_PLAN_ONLY: validated and planned, no packed weights
  Mat fc, lm, w2;
  long long fc_norm = -1, final_norm = -1, conf_w = -1, conf_b = -1, w1 = -1, freqs = -1;
  long long w2n = -1, w1max = -1;  // row-norm bounds of W2 and the largest of W1 (candidate pruning)
  int w1_fmt = DT_BF16, w1_ld = 0;
  std::vector<Layer> L;
  float tau = 1.f;
  bool has_mlp = true;
};

namespace {

const dspark_weight* find_w(const dspark_weight* w, int n, int id) {
  for (int i = 0; i < n; ++i)
    if (w[i].id == id) return &w[i];
  return nullptr;
}

int32_t check_cfg(const dspark_config* c) {
  if (!c) return fail(DSPARK_EINVAL, "config is NULL");
  if (c->flags & ~(DSPARK_CFG_LAYERS_ONLY | DSPARK_CFG_PLAN_ONLY)) return fail(DSPARK_EINVAL, "unknown config flags");
  if (c->hidden <= 0 || c->n_layers <= 0 || c->n_heads <= 0 || c->q_lora <= 0 || c->kv_lora <= 0 ||
      c->qk_nope <= 0 || c->qk_rope <= 0 || c->v_head <= 0 || c->block <= 0)
    return fail(DSPARK_EINVAL, "config has a non-positive dimension");
  if (!(c->flags & DSPARK_CFG_LAYERS_ONLY) &&
      (c->vocab <= 0 || c->markov_rank <= 0 || c->n_captured <= 0 || c->inter <= 0))
    return fail(DSPARK_EINVAL, "config has a non-positive head / fc dimension");
  if (c->qk_rope % 2) return fail(DSPARK_EUNSUPPORTED, "qk_rope must be even");
  if ((c->kv_lora + c->qk_rope) % 8) return fail(DSPARK_EUNSUPPORTED, "kv_lora + qk_rope must be a multiple of 8");
  if (c->kv_lora % 16) return fail(DSPARK_EUNSUPPORTED, "kv_lora must be a multiple of 16");
  if (c->block > 64) return fail(DSPARK_EUNSUPPORTED, "block > 64");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f) || !(c->yarn_factor >= 1.f))
    return fail(DSPARK_EINVAL, "rms_eps / rope_theta / yarn_factor out of range");
  return DSPARK_OK;
}

// Look up one matrix source: id, allowed dtypes, exact shape.
int32_t get_mat(const dspark_weight* w, int n, int id, long long rows, long long cols, const dspark_weight** out,
                bool required = true) {
  const dspark_weight* x = find_w(w, n, id);
  *out = x;
  if (!x) return required ? fail(DSPARK_EINVAL, "weight id %d missing", id) : DSPARK_OK;
  if (x->rows != rows || x->cols != cols)
    return fail(DSPARK_EINVAL, "weight id %d: shape [%lld][%lld], expected [%lld][%lld]", id, (long long)x->rows,
                (long long)x->cols, rows, cols);
  if (x->dtype < DSPARK_DT_F32 || x->dtype > DSPARK_DT_MXFP4)
    return fail(DSPARK_EUNSUPPORTED, "weight id %d: unknown dtype %d", id, x->dtype);
  if (!x->data) return fail(DSPARK_EINVAL, "weight id %d: data is NULL", id);
  if (x->dtype == DSPARK_DT_Q8_0 && cols % 32) return fail(DSPARK_EUNSUPPORTED, "weight id %d: Q8_0 needs cols %% 32 == 0", id);
  if (x->dtype == DSPARK_DT_FP8_E4M3 && !x->scales) return fail(DSPARK_EINVAL, "weight id %d: FP8 scales NULL", id);
  if (x->dtype == DSPARK_DT_MXFP4 && (cols % 32 || rup(cols, 64) % 128))
    return fail(DSPARK_EUNSUPPORTED, "weight id %d: MXFP4 needs cols %% 32 == 0 and round_up(cols, 64) %% 128 == 0", id);
  return DSPARK_OK;
}

int32_t get_vec(const dspark_weight* w, int n, int id, long long len, const dspark_weight** out) {
  const dspark_weight* x = find_w(w, n, id);
  *out = x;
  if (!x) return fail(DSPARK_EINVAL, "weight id %d missing", id);
  if (x->dtype != DSPARK_DT_F32) return fail(DSPARK_EUNSUPPORTED, "weight id %d must be F32", id);
  if (x->rows * x->cols != len) return fail(DSPARK_EINVAL, "weight id %d: length %lld, expected %lld", id,
                                            (long long)(x->rows * x->cols), len);
  if (!x->data) return fail(DSPARK_EINVAL, "weight id %d: data is NULL", id);
  return DSPARK_OK;
}

// Build the plan (geometry + offsets) of every packed item; returns total bytes.
int32_t build_plan(const dspark_config* c, const dspark_weight* w, int n, dspark_model& m) {
  int32_t rc = check_cfg(c);
  if (rc) return rc;
  if (!w || n <= 0) return fail(DSPARK_EINVAL, "weight table empty");
  m.c = *c;
  m.layers_only = (c->flags & DSPARK_CFG_LAYERS_ONLY) != 0;
  m.plan_only = (c->flags & DSPARK_CFG_PLAN_ONLY) != 0;
  const long long H = c->hidden, nh = c->n_heads, r = c->kv_lora, dr = c->qk_rope, dn = c->qk_nope, dv = c->v_head;
  const long long latent = r + dr;
  long long off = 0;
  auto take = [&](long long bytes) {
    const long long o = off;
    off = rup(off + bytes, 256);
    return o;
  };
  auto place = [&](Mat& mt) {
    mt.codes_off = take(mt.codes_bytes);
    if (mt.scales_bytes) mt.scales_off = take(mt.scales_bytes);
  };
  const dspark_weight *a, *b;
  m.L.assign(c->n_layers, Layer());
  m.has_mlp = true;
  for (int l = 0; l < c->n_layers; ++l) {
    Layer& L = m.L[l];
    const dspark_weight* v;
    if ((rc = get_vec(w, n, DSPARK_LAYER_W(l, DSPARK_L_IN_NORM), H, &v))) return rc;
    L.in_norm = take(H * 4);
    if ((rc = get_vec(w, n, DSPARK_LAYER_W(l, DSPARK_L_Q_A_NORM), c->q_lora, &v))) return rc;
    L.q_a_norm = take(c->q_lora * 4);
    if ((rc = get_vec(w, n, DSPARK_LAYER_W(l, DSPARK_L_KV_A_NORM), r, &v))) return rc;
    L.kv_a_norm = take(r * 4);
    if ((rc = get_mat(w, n, DSPARK_LAYER_W(l, DSPARK_L_Q_A), c->q_lora, H, &a))) return rc;
    if ((rc = get_mat(w, n, DSPARK_LAYER_W(l, DSPARK_L_KV_A), latent, H, &b))) return rc;
    if (a->dtype != b->dtype) return fail(DSPARK_EUNSUPPORTED, "layer %d: q_a and kv_a dtypes differ", l);
    mat_geom(L.qkva, a->dtype, 1, (int)(c->q_lora + latent), (int)H);
    place(L.qkva);
    if ((rc = get_mat(w, n, DSPARK_LAYER_W(l, DSPARK_L_Q_B), nh * (dn + dr), c->q_lora, &a))) return rc;
    mat_geom(L.qb, a->dtype, 1, (int)(nh * (dn + dr)), c->q_lora);
    place(L.qb);
    if ((rc = get_mat(w, n, DSPARK_LAYER_W(l, DSPARK_L_KV_B), nh * (dn + dv), r, &a))) return rc;
    if (a->dtype != DSPARK_DT_BF16 && a->dtype != DSPARK_DT_F32)
      return fail(DSPARK_EUNSUPPORTED, "layer %d: kv_b must be BF16 or F32", l);
    mat_geom(L.uk, a->dtype, (int)nh, (int)r, (int)dn);
    place(L.uk);
    mat_geom(L.uv, a->dtype, (int)nh, (int)dv, (int)r);
    place(L.uv);
    if ((rc = get_mat(w, n, DSPARK_LAYER_W(l, DSPARK_L_O), H, nh * dv, &a))) return rc;
    mat_geom(L.o, a->dtype, 1, (int)H, (int)(nh * dv));
    place(L.o);
    const dspark_weight* g = find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_GATE));
    if (!g) {
      if (!m.layers_only) return fail(DSPARK_EINVAL, "layer %d: gate missing", l);
      m.has_mlp = false;
      continue;
    }
    if ((rc = get_vec(w, n, DSPARK_LAYER_W(l, DSPARK_L_POST_NORM), H, &v))) return rc;
    L.post_norm = take(H * 4);
    if ((rc = get_mat(w, n, DSPARK_LAYER_W(l, DSPARK_L_GATE), c->inter, H, &a))) return rc;
    if ((rc = get_mat(w, n, DSPARK_LAYER_W(l, DSPARK_L_UP), c->inter, H, &b))) return rc;
    if (a->dtype != b->dtype) return fail(DSPARK_EUNSUPPORTED, "layer %d: gate and up dtypes differ", l);
    mat_geom(L.gu, a->dtype, 1, 2 * c->inter, (int)H);
    place(L.gu);
    if ((rc = get_mat(w, n, DSPARK_LAYER_W(l, DSPARK_L_DOWN), H, c->inter, &a))) return rc;
    mat_geom(L.down, a->dtype, 1, (int)H, c->inter);
    place(L.down);
  }
  // one workspace plan serves every layer: all layers must share layer 0's formats
  for (int l = 1; l < c->n_layers; ++l) {
    const Layer &A = m.L[0], &B = m.L[l];
    if (A.qkva.pm.fmt != B.qkva.pm.fmt || A.qb.pm.fmt != B.qb.pm.fmt || A.uk.pm.fmt != B.uk.pm.fmt ||
        A.o.pm.fmt != B.o.pm.fmt || A.gu.pm.fmt != B.gu.pm.fmt || A.down.pm.fmt != B.down.pm.fmt ||
        A.gu.present != B.gu.present)
      return fail(DSPARK_EUNSUPPORTED, "layer %d formats differ from layer 0", l);
  }
  if (!m.layers_only) {
    const dspark_weight* v;
    if ((rc = get_mat(w, n, DSPARK_W_FC, H, (long long)c->n_captured * H, &a))) return rc;
    mat_geom(m.fc, a->dtype, 1, (int)H, (int)(c->n_captured * H));
    place(m.fc);
    if ((rc = get_vec(w, n, DSPARK_W_FC_NORM, H, &v))) return rc;
    m.fc_norm = take(H * 4);
    if ((rc = get_vec(w, n, DSPARK_W_FINAL_NORM, H, &v))) return rc;
    m.final_norm = take(H * 4);
    if ((rc = get_mat(w, n, DSPARK_W_LM_HEAD, c->vocab, H, &a))) return rc;
    mat_geom(m.lm, a->dtype, 1, c->vocab, (int)H);
    place(m.lm);
    if ((rc = get_mat(w, n, DSPARK_W_MARKOV_W1, c->vocab, c->markov_rank, &a))) return rc;
    if ((rc = get_mat(w, n, DSPARK_W_MARKOV_W2, c->vocab, c->markov_rank, &b))) return rc;
    if ((a->dtype != DSPARK_DT_BF16 && a->dtype != DSPARK_DT_F32) || a->dtype != b->dtype)
      return fail(DSPARK_EUNSUPPORTED, "Markov W1/W2 must both be BF16 or both F32");
    mat_geom(m.w2, b->dtype, 1, c->vocab, c->markov_rank);
    place(m.w2);
    m.w1_fmt = a->dtype;
    m.w1_ld = m.w2.pm.Kp;
    m.w1 = take((long long)c->vocab * m.w1_ld * (a->dtype == DSPARK_DT_F32 ? 4 : 2));
    m.w2n = take((long long)c->vocab * 4);
    m.w1max = take(4);
    if ((rc = get_vec(w, n, DSPARK_W_CONF_W, H + c->markov_rank, &v))) return rc;
    m.conf_w = take((H + c->markov_rank) * 4);
    if ((rc = get_vec(w, n, DSPARK_W_CONF_B, 1, &v))) return rc;
    m.conf_b = take(4);
  }
  m.freqs = take((dr / 2) * 8);
  m.bytes = off;
  // softmax scale: (0.1 ln s + 1)^2 / sqrt(qk_nope + qk_rope)
  const double s = c->yarn_factor;
  const double msc = s > 1.0 ? (0.1 * std::log(s) + 1.0) : 1.0;
  m.tau = (float)(msc * msc / std::sqrt((double)(dn + dr)));
  return DSPARK_OK;
}

// Rope angular frequencies (YaRN NTK-by-parts when yarn_factor > 1), fp64.
std::vector<double> rope_freqs(const dspark_config& c) {
  const int d = c.qk_rope;
  std::vector<double> f(d / 2);
  const double s = c.yarn_factor, L = c.yarn_orig_ctx;
  const double lo = c.yarn_beta_slow, hi = c.yarn_beta_fast;
  for (int k = 0; k < d / 2; ++k) {
    const double theta = std::pow((double)c.rope_theta, -2.0 * k / d);
    if (s == 1.0) {
      f[k] = theta;
      continue;
    }
    const double rot = L * theta / (2.0 * M_PI);  // rotations over the original window
    double gamma = (rot - lo) / (hi - lo);
    gamma = gamma < 0 ? 0 : gamma > 1 ? 1 : gamma;
    f[k] = (1.0 - gamma) * theta / s + gamma * theta;
  }
  return f;
}

void bind(dspark_model& m, Mat& mt) {
  if (!mt.present) return;
  mt.pm.codes = m.base + mt.codes_off;
  mt.pm.scales = mt.scales_off >= 0 ? (const void*)(m.base + mt.scales_off) : nullptr;
}

int32_t repack(dspark_model& m, Mat& mt, const dspark_weight* src, int xf, int row0, int nrows, hipStream_t st) {
  RepackArgs a{};
  a.src = src->data;
  a.src_fmt = src->dtype;
  a.src_scales = (const float*)src->scales;
  a.src_rows = src->rows;
  a.src_cols = src->cols;
  a.xf = xf;
  a.dn = m.c.qk_nope;
  a.dv = m.c.v_head;
  a.r = m.c.kv_lora;
  a.codes = m.base + mt.codes_off;
  a.scales = mt.scales_off >= 0 ? (void*)(m.base + mt.scales_off) : nullptr;
  a.dst = mt.pm;
  a.row0 = row0;
  a.nrows = nrows;
  HIPCHK(launch_repack(a, st));
  return DSPARK_OK;
}

int32_t copy_vec(dspark_model& m, long long off, const dspark_weight* w, hipStream_t st) {
  HIPCHK(hipMemcpyAsync(m.base + off, w->data, (size_t)(w->rows * w->cols * 4), hipMemcpyDeviceToDevice, st));
  return DSPARK_OK;
}

// ---------------------------------------------------------- workspace plan --
struct Frag {
  FragDesc fd{};
  long long off = 0, bytes = 0;
};

// Input buffer of one GEMM: int8 hi/lo codes (plan.amode 3), fp32 rows when
// the GEMM converts its activations in LDS (amode 1 and 2), else prepared
// fragments (amode 0).
void frag_geom(Frag& f, const PackedMat& w, int M, const GemvPlan& p) {
  f.fd = FragDesc{};
  if (p.amode == 3) {  // int8 codes [KB][64][8 B] + exponents [KB][8]
    f.fd.i8 = 1;
    f.fd.KB = w.KB;
    f.fd.gstride = (long long)w.KB * (512 + 8);
    f.bytes = f.fd.gstride * w.ngroups;
    return;
  }
  if (p.amode == 1 || p.amode == 2) {
    f.fd.rows = 1;
    f.fd.ld = w.K;
    f.fd.gstride = (long long)M * w.K;
    f.bytes = f.fd.gstride * 4 * w.ngroups;
    return;
  }
  f.fd.f32 = w.fmt == DT_F32;
  f.fd.hilo = p.hilo;
  f.fd.KB = w.KB;
  f.fd.KG = w.Kp / 16;
  f.fd.MT = f.fd.hilo ? 1 : (M + 15) / 16;
  const long long per = f.fd.f32 ? (long long)f.fd.MT * f.fd.KG * 64 * 4 : (long long)f.fd.MT * f.fd.KB * 64 * 8;
  f.fd.gstride = per;
  f.bytes = per * (f.fd.f32 ? 4 : 2) * w.ngroups;
}

struct Plan {
  int n_seq = 0, M = 0;
  long long total_ctx = 0;
  bool kv_f32 = false;
  long long x = 0, part = 0, q = 0, bkeys = 0, opart = 0, mlpart = 0, z = 0, keys = 0, mslots = 0, merr = 0, total = 0;
  long long mfall = 0, mlmax = 0, mlcnt = 0, mlist = 0;  // candidate pruning of the Markov rollout
  int nch_v = 0;
  int mwgs = 0;
  long long ssq_a = 0, ssq_b = 0, ssq_cq = 0, dot = 0, rope = 0;
  long long zero_begin = 0, zero_end = 0;
  Frag f_fc, f_qkva, f_qb, f_uk, f_uv, f_o, f_gu, f_down, f_lm;
  GemvPlan p_fc{}, p_qkva{}, p_qb{}, p_uk{}, p_uv{}, p_o{}, p_gu{}, p_down{}, p_lm{}, p_w2{};
  int rows = 0, rows_pad = 0, DQ = 0, C = 0, slots = 0;
};

void make_plan(const dspark_model& m, int n_seq, long long total_ctx, bool kv_f32, Plan& P) {
  const dspark_config& c = m.c;
  P.n_seq = n_seq;
  P.total_ctx = total_ctx;
  P.kv_f32 = kv_f32;
  const int M = n_seq * c.block;
  P.M = M;
  long long off = 0;
  auto take = [&](long long bytes) {
    const long long o = off;
    off = rup(off + bytes, 256);
    return o;
  };
  const Layer& L0 = m.L[0];
  P.x = take((long long)M * c.hidden * 4);
  long long part = 0;
  // i8: whether the producing kernel of the GEMM's input can write int8
  // fragments (column-per-lane producers always can; the W_UV epilogue can
  // when its 32-column blocks are pairs of its own 16-row tiles)
  auto gp = [&](GemvPlan& gpn, const Mat& mt, bool split, bool i8) {
    gpn = plan_gemv(mt.pm, M, split, false, i8);
    if (split) part = std::max(part, (long long)gpn.S * M * mt.pm.ngroups * mt.pm.G * 4);
  };
  gp(P.p_qkva, L0.qkva, true, true);
  gp(P.p_uk, L0.uk, false, false);  // epilogue writes the query buffer
  gp(P.p_uv, L0.uv, false, false);  // epilogue writes the o_proj fragments
  const bool uv_i8 = P.p_uv.MT == 1 && P.p_uv.TPW % 2 == 0 && L0.uv.pm.TG % 2 == 0 && L0.uv.pm.G % 32 == 0;
  // column-owning GEMMs (split inside the workgroup, fused epilogue) where
  // the shape and format are covered, else split-K plus a reduction kernel
  auto own = [&](GemvPlan& gpn, const Mat& mt, bool swiglu, bool i8) {
    gpn = plan_own(mt.pm, M, swiglu, i8);
    return gpn.nw > 0;
  };
  gp(P.p_qb, L0.qb, true, true);  // (a column-owning q_b measured slower than split-K + the fused absorb)
  if (!own(P.p_o, L0.o, false, uv_i8)) gp(P.p_o, L0.o, true, uv_i8);
  if (m.has_mlp) {
    if (!own(P.p_gu, L0.gu, true, true)) gp(P.p_gu, L0.gu, true, true);
    if (!own(P.p_down, L0.down, false, true)) gp(P.p_down, L0.down, true, true);
  }
  if (!m.layers_only) {
    if (!own(P.p_fc, m.fc, false, true)) gp(P.p_fc, m.fc, true, true);
    P.p_lm = plan_gemv(m.lm.pm, M, false, false, true);
    P.p_w2 = plan_gemv(m.w2.pm, n_seq, false, true);
  }
  frag_geom(P.f_qkva, L0.qkva.pm, M, P.p_qkva);
  frag_geom(P.f_qb, L0.qb.pm, M, P.p_qb);
  frag_geom(P.f_uk, L0.uk.pm, M, P.p_uk);
  frag_geom(P.f_uv, L0.uv.pm, M, P.p_uv);
  frag_geom(P.f_o, L0.o.pm, M, P.p_o);
  if (m.has_mlp) {
    frag_geom(P.f_gu, L0.gu.pm, M, P.p_gu);
    frag_geom(P.f_down, L0.down.pm, M, P.p_down);
  }
  if (!m.layers_only) {
    frag_geom(P.f_fc, m.fc.pm, M, P.p_fc);
    frag_geom(P.f_lm, m.lm.pm, M, P.p_lm);
    P.f_fc.off = take(P.f_fc.bytes);
  }
  // zeroed region: fragment buffers, argmax keys and the query buffer
  P.zero_begin = off;
  for (Frag* f : {&P.f_qkva, &P.f_qb, &P.f_uk, &P.f_uv, &P.f_o, &P.f_gu, &P.f_down, &P.f_lm})
    if (f->bytes) f->off = take(f->bytes);
  P.keys = take((long long)n_seq * c.block * KEY_SLOTS * 8);
  if (!m.layers_only) {  // Markov rollout argmax slots and error flag
    P.mwgs = markov_rollout_wgs(m.w2.pm.ngroups * m.w2.pm.TG);
    P.mslots = take((long long)c.block * n_seq * P.mwgs * 8);
    P.merr = take(16);
    P.mfall = take(16);
  }
  P.rows = c.block * c.n_heads;
  P.rows_pad = (int)rup(P.rows, 64);
  P.DQ = (int)rup(c.kv_lora + c.qk_rope, 32);
  P.q = take((long long)n_seq * P.rows_pad * P.DQ * (kv_f32 ? 4 : 2));
  P.zero_end = off;
  P.part = take(part);
  P.bkeys = take((long long)M * (c.kv_lora + c.qk_rope) * (kv_f32 ? 4 : 2));
  // Keys per attention slot: the multiple of 32 in [128, 2048] with the
  // smallest estimated attention time.  One workgroup runs per CU (256 on
  // MI355X), so the grid of (rows / 64) x slots workgroups runs in whole
  // rounds; a workgroup costs about seven key tiles' time in fixed work (query
  // and first-tile loads, partial stores) plus one per key tile, and its slot
  // partials are written and read back once more (at ~6 TB/s).  At context
  // 98,304 this picks 1376 keys (2 rounds of 72 slots) over 1024 (3 rounds);
  // context 8192 keeps 256 (one round), and context 4096 takes 160 (26
  // slots of 5 tiles per row group instead of 17 of 8).  The slot count uses the bound cdiv(keys, C) +
  // n_seq, which holds for any split of the context between sequences.
  {
    constexpr int kCUs = 256;
    const long long keys = total_ctx + (long long)n_seq * c.block;
    const long long part_row = (long long)c.kv_lora * 2 + 8;
    const double step_s = 1.05e-6;  // one key tile of a workgroup, measured
    double best = 0.0;
    for (int cc = 128; cc <= 2048; cc += 32) {
      const long long slots = cdiv(keys, cc) + n_seq;
      const long long rounds = cdiv((long long)(P.rows_pad / 64) * slots, kCUs);
      const double cost = (double)rounds * (7 + cc / 32) +
                          2.0 * (double)slots * P.rows_pad * part_row / 6e12 / step_s;
      if (cc == 128 || cost < best) {
        best = cost;
        P.C = cc;
      }
    }
  }
  P.slots = (int)(cdiv(total_ctx + (long long)n_seq * c.block, P.C) + n_seq);
  if (!kv_f32) {
    P.opart = take((long long)P.slots * P.rows_pad * c.kv_lora * 2);
    P.mlpart = take((long long)P.slots * P.rows_pad * 2 * 4);
  }
  const long long ssq = (long long)M * SSQ_LD * 4;
  P.ssq_a = take(ssq);
  P.ssq_b = take(ssq);
  P.ssq_cq = take(ssq);
  P.dot = take(ssq);
  P.rope = take((long long)M * (c.qk_rope / 2) * 8);
  if (!m.layers_only) {
    P.z = take((long long)M * c.vocab * 4);
    P.nch_v = markov_prune_chunks(c.vocab);
    P.mlmax = take((long long)M * P.nch_v * 4);
    P.mlcnt = take((long long)M * P.nch_v * 4);
    P.mlist = take((long long)M * P.nch_v * MK_CAPC * 16);
  }
  P.total = off;
}

void bind_frag(Frag& f, unsigned char* ws) {
  f.fd.ptr = f.bytes ? (void*)(ws + f.off) : nullptr;
}

GemvArgs gemv_base(const Mat& mt, const GemvPlan& p, const Frag& f, int M) {
  GemvArgs a{};
  a.w = mt.pm;
  a.act = f.fd.ptr;
  a.act_gstride = f.fd.gstride;
  a.act_ld = f.fd.ld;
  a.M = M;
  a.hilo = p.hilo;
  a.ksteps_per_split = p.ksteps_per_split;
  a.ksteps_lo = p.ksteps_lo;
  a.out_ld = (long long)mt.pm.ngroups * mt.pm.G;
  a.out_split_stride = (long long)M * a.out_ld;
  return a;
}

// One GEMV launch with the STORE epilogue into `out` (optionally row-scaled).
hipError_t run_gemv(const Mat& mt, const GemvPlan& p, const Frag& f, int M, float* out, hipStream_t st,
                    RowScale rs = RowScale{}) {
  GemvArgs a = gemv_base(mt, p, f, M);
  a.out = out;
  a.rs = rs;
  return launch_gemv(a, p, GEMV_STORE, st);
}

struct Ctx {
  const dspark_model* m;
  Plan P;
  unsigned char* ws;
  hipStream_t st;
  // paged caches (page_log2 >= 0), see dspark_block_in
  const int32_t* table = nullptr;
  int page_log2 = -1, max_pages = 0;
  float* part() const { return (float*)(ws + P.part); }
  float* x() const { return (float*)(ws + P.x); }
  float* ssq(long long off) const { return (float*)(ws + off); }
  // chunk counts of the sums of squares now in ssq_a / ssq_b: 256-column
  // chunks from the column-parallel kernels, OWN_COLS-column chunks from the
  // column-owning GEMM epilogues
  int nch_a = 0, nch_b = 0;
  int nch_of(long long off, int n) const {
    return off == P.ssq_a && nch_a ? nch_a : off == P.ssq_b && nch_b ? nch_b : (n + 255) / 256;
  }
  RowScale rs(long long off, int n) const {
    RowScale r{};
    r.ssq = (const float*)(ws + off);
    r.nch = nch_of(off, n);
    r.invn = 1.f / (float)n;
    r.eps = m->c.rms_eps;
    return r;
  }
  PartIn pin(const GemvPlan& p, const Mat& mt) const {
    PartIn q{};
    q.part = part();
    q.S = p.S;
    q.ld = (long long)mt.pm.ngroups * mt.pm.G;
    q.ss = (long long)P.M * q.ld;
    return q;
  }
};

// RoPE table of the pass (cos, sin per row and frequency), built by k_init.
void set_rope(const Ctx& C, InitArgs& a, const int32_t* offs) {
  a.rope = (float*)(C.ws + C.P.rope);
  a.offs = offs;
  a.freqs = (const double*)(C.m->base + C.m->freqs);
  a.npairs = C.m->c.qk_rope / 2;
}

// Attention half of layer l.  Input: fragments of in_norm * x in f_qkva and
// the chunk sums of x^2 at workspace offset `x_ssq`.  Leaves the o_proj partials.
int32_t attn_half(Ctx& C, int l, long long x_ssq, const void* kv, const int32_t* offs) {
  const dspark_model& m = *C.m;
  const dspark_config& c = m.c;
  const Layer& L = m.L[l];
  Plan& P = C.P;
  const int M = P.M;
  HIPCHK(run_gemv(L.qkva, P.p_qkva, P.f_qkva, M, C.part(), C.st));
  {
    QkvaPost a{};
    a.p = C.pin(P.p_qkva, L.qkva);
    a.rs_in = C.rs(x_ssq, c.hidden);
    a.M = M;
    a.q_lora = c.q_lora;
    a.r = c.kv_lora;
    a.dr = c.qk_rope;
    a.latent = c.kv_lora + c.qk_rope;
    a.block = c.block;
    a.g_qa = (const float*)(m.base + L.q_a_norm);
    a.g_kva = (const float*)(m.base + L.kv_a_norm);
    a.eps = c.rms_eps;
    a.fd_qb = P.f_qb.fd;
    a.ssq_cq = C.ssq(P.ssq_cq);
    a.bkeys = C.ws + P.bkeys;
    a.kv_f32 = P.kv_f32;
    a.rope = (const float*)(C.ws + P.rope);
    HIPCHK(launch_post_qkva(a, C.st));
  }
  HIPCHK(run_gemv(L.qb, P.p_qb, P.f_qb, M, C.part(), C.st));
  {
    QbPost a{};
    a.p = C.pin(P.p_qb, L.qb);
    a.rs = C.rs(P.ssq_cq, c.q_lora);
    a.M = M;
    a.nh = c.n_heads;
    a.dn = c.qk_nope;
    a.dr = c.qk_rope;
    a.r = c.kv_lora;
    a.block = c.block;
    a.DQ = P.DQ;
    a.rows_pad = P.rows_pad;
    a.fd_uk = P.f_uk.fd;
    a.q = C.ws + P.q;
    a.q_f32 = P.kv_f32;
    a.rope = (const float*)(C.ws + P.rope);
    GemvArgs u = gemv_base(L.uk, P.p_uk, P.f_uk, M);
    u.q = C.ws + P.q;
    u.q_f32 = P.kv_f32;
    u.DQ = P.DQ;
    u.rows_pad = P.rows_pad;
    u.nh = c.n_heads;
    u.block = c.block;
    if (qb_absorb_supported(u, a)) {
      HIPCHK(launch_qb_absorb(QbAbsorbArgs{u, a}, C.st));  // post fused with the absorb GEMM
    } else {
      HIPCHK(launch_post_qb(a, C.st));
      HIPCHK(launch_gemv(u, P.p_uk, GEMV_QLAT, C.st));
    }
  }
  {
    AttnArgs a{};
    a.q = C.ws + P.q;
    a.cache = kv;
    a.bkeys = C.ws + P.bkeys;
    a.offs = offs;
    a.n_seq = P.n_seq;
    a.block = c.block;
    a.nh = c.n_heads;
    a.rows = P.rows;
    a.rows_pad = P.rows_pad;
    a.latent = c.kv_lora + c.qk_rope;
    a.r = c.kv_lora;
    a.DQ = P.DQ;
    a.C = P.C;
    a.slots = P.slots;
    a.len1 = P.n_seq == 1 ? (int)P.total_ctx : -1;  // the contract: kv_offsets = {0, total_ctx}
    a.table = C.table;
    a.page_log2 = C.page_log2;
    a.max_pages = C.max_pages;
    a.tau = m.tau;
    a.fd_uv = P.f_uv.fd;
    GemvArgs g = gemv_base(L.uv, P.p_uv, P.f_uv, M);
    g.fd = P.f_o.fd;
    bool fused = false;
    if (P.kv_f32) {
      HIPCHK(launch_attn_f32(a, C.st));
    } else {
      a.o_part = (uint16_t*)(C.ws + P.opart);
      a.ml_part = (float*)(C.ws + P.mlpart);
      HIPCHK(launch_attn_bf16(a, C.st));
      if (a.len1 >= 0 && uv_combine_supported(g, P.n_seq, P.slots)) {
        UvCombineArgs u{};  // combine fused with the un-absorb GEMM
        u.g = g;
        u.o_part = a.o_part;
        u.ml_part = a.ml_part;
        u.slots = P.slots;
        u.C = P.C;
        u.block = c.block;
        u.nh = c.n_heads;
        u.r = c.kv_lora;
        u.len1 = a.len1;
        HIPCHK(launch_uv_combine(u, C.st));
        fused = true;
      } else {
        HIPCHK(launch_attn_combine(a, C.st));
      }
    }
    if (!fused) HIPCHK(launch_gemv(g, P.p_uv, GEMV_FRAG, C.st));
  }
  return DSPARK_OK;
}

// The residual update x_out = x_in + W a of o_proj or down, the chunk sums
// of x_out^2 into `ssq_out` and, with g1, the fragments of g1 * x_out for
// the next GEMM (`fd`; with dotw also the confidence dot chunks): one
// column-owning launch, or split-K plus the residual kernel.
int32_t resid_gemm(Ctx& C, const Mat& mt, const GemvPlan& p, const Frag& f, const float* x_in, float* x_out,
                   const float* g1, const FragDesc* fd, long long ssq_out, const float* dotw) {
  Plan& P = C.P;
  const int H = C.m->c.hidden;
  if (p.nw) {
    GemvArgs a = gemv_base(mt, p, f, P.M);
    a.epi = OWN_RESID;
    a.x_in = x_in;
    a.x_out = x_out;
    a.g1 = g1;
    if (fd) a.fd = *fd;
    a.ssq_out = ssq_out >= 0 ? C.ssq(ssq_out) : nullptr;
    a.dotw = dotw;
    a.dot_out = dotw ? C.ssq(P.dot) : nullptr;
    HIPCHK(launch_gemv(a, p, GEMV_OWN, C.st));
  } else {
    HIPCHK(run_gemv(mt, p, f, P.M, C.part(), C.st));
    ResidPost a{};
    a.p = C.pin(p, mt);
    a.mode = RP_ADD;
    a.x_in = x_in;
    a.x_out = x_out;
    a.M = P.M;
    a.H = H;
    a.g1 = g1;
    if (fd) a.fd = *fd;
    a.ssq_out = ssq_out >= 0 ? C.ssq(ssq_out) : nullptr;
    a.dotw = dotw;
    a.dot_out = dotw ? C.ssq(P.dot) : nullptr;
    HIPCHK(launch_post_resid(a, C.st));
  }
  const int nch = p.nw ? H / OWN_COLS : (H + 255) / 256;
  if (ssq_out == P.ssq_a) C.nch_a = nch;
  if (ssq_out == P.ssq_b) C.nch_b = nch;
  return DSPARK_OK;
}

// SwiGLU half of layer l.  Input: fragments of post_norm * x in f_gu and the
// chunk sums of x^2 at `x_ssq`.  Leaves the down partials.
int32_t mlp_half(Ctx& C, int l, long long x_ssq) {
  const dspark_model& m = *C.m;
  const Layer& L = m.L[l];
  Plan& P = C.P;
  const int M = P.M;
  if (P.p_gu.nw) {  // gate/up with the SwiGLU fused: workgroup gi owns gate and up columns 32 gi .. + 31
    GemvArgs a = gemv_base(L.gu, P.p_gu, P.f_gu, M);
    a.epi = OWN_SWIGLU;
    a.rs = C.rs(x_ssq, m.c.hidden);
    a.tile_jump = L.gu.pm.TG / 2 - 2;  // up tiles follow the gate tiles
    a.fd = P.f_down.fd;
    HIPCHK(launch_gemv(a, P.p_gu, GEMV_OWN, C.st));
    return DSPARK_OK;
  }
  HIPCHK(run_gemv(L.gu, P.p_gu, P.f_gu, M, C.part(), C.st));
  SwigluPost a{};
  a.p = C.pin(P.p_gu, L.gu);
  a.rs = C.rs(x_ssq, m.c.hidden);
  a.M = M;
  a.inter = m.c.inter;
  a.fd = P.f_down.fd;
  HIPCHK(launch_post_swiglu(a, C.st));
  return DSPARK_OK;
}

ResidPost resid_base(Ctx& C) {
  ResidPost a{};
  a.x_in = C.x();
  a.x_out = C.x();
  a.mode = RP_ADD;
  a.M = C.P.M;
  a.H = C.m->c.hidden;
  return a;
}

bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p) % a != 0; }

int32_t check_ws(const Plan& P, void* ws, size_t ws_bytes) {
  if (!ws) return fail(DSPARK_EINVAL, "workspace is NULL");
  if ((uintptr_t)ws % 256) return fail(DSPARK_EINVAL, "workspace must be 256-byte aligned");
  if ((long long)ws_bytes < P.total)
    return fail(DSPARK_EWORKSPACE, "workspace %zu bytes, need %lld", ws_bytes, P.total);
  return DSPARK_OK;
}

}  // namespace

// ============================================================== the C ABI ==
extern "C" {

const char* dspark_last_error(void) { return g_err.c_str(); }

size_t dspark_packed_bytes(const dspark_config* cfg, const dspark_weight* w, int32_t n) {
  dspark_model m;
  if (build_plan(cfg, w, n, m)) return 0;
  return (size_t)m.bytes;
}

int32_t dspark_model_create(const dspark_config* cfg, const dspark_weight* w, int32_t n, void* packed_buf,
                            size_t packed_bytes, void* stream, dspark_model** out) {
  g_err.clear();
  if (!out) return fail(DSPARK_EINVAL, "out is NULL");
  *out = nullptr;
  dspark_model* m = new dspark_model();
  int32_t rc = build_plan(cfg, w, n, *m);
  if (rc) {
    delete m;
    return rc;
  }
  if (m->plan_only) {  // no device, no packed buffer: sizes and validation only
    *out = m;
    return DSPARK_OK;
  }
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
    delete m;
    return fail(DSPARK_ENODEVICE, "no HIP device");
  }
  if (!packed_buf || (uintptr_t)packed_buf % 256) {
    delete m;
    return fail(DSPARK_EINVAL, "packed_buf NULL or not 256-byte aligned");
  }
  if ((long long)packed_bytes < m->bytes) {
    const long long need = m->bytes;
    delete m;
    return fail(DSPARK_EWORKSPACE, "packed buffer %zu bytes, need %lld", packed_bytes, need);
  }
  m->base = (unsigned char*)packed_buf;
  hipStream_t st = (hipStream_t)stream;
  auto body = [&]() -> int32_t {
    const dspark_config& c = m->c;
    HIPCHK(hipMemsetAsync(m->base, 0, (size_t)m->bytes, st));
    for (Mat* mt : {&m->fc, &m->lm, &m->w2}) bind(*m, *mt);
    for (int l = 0; l < c.n_layers; ++l) {
      Layer& L = m->L[l];
      for (Mat* mt : {&L.qkva, &L.qb, &L.uk, &L.uv, &L.o, &L.gu, &L.down}) bind(*m, *mt);
      const dspark_weight* x;
      int32_t r2;
      x = find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_Q_A));
      if ((r2 = repack(*m, L.qkva, x, XF_NORMAL, 0, c.q_lora, st))) return r2;
      x = find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_KV_A));
      if ((r2 = repack(*m, L.qkva, x, XF_NORMAL, c.q_lora, c.kv_lora + c.qk_rope, st))) return r2;
      x = find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_Q_B));
      if ((r2 = repack(*m, L.qb, x, XF_NORMAL, 0, L.qb.pm.G, st))) return r2;
      x = find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_KV_B));
      if ((r2 = repack(*m, L.uk, x, XF_UK, 0, c.n_heads * c.kv_lora, st))) return r2;
      if ((r2 = repack(*m, L.uv, x, XF_UV, 0, c.n_heads * c.v_head, st))) return r2;
      x = find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_O));
      if ((r2 = repack(*m, L.o, x, XF_NORMAL, 0, c.hidden, st))) return r2;
      if ((r2 = copy_vec(*m, L.in_norm, find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_IN_NORM)), st))) return r2;
      if ((r2 = copy_vec(*m, L.q_a_norm, find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_Q_A_NORM)), st))) return r2;
      if ((r2 = copy_vec(*m, L.kv_a_norm, find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_KV_A_NORM)), st))) return r2;
      if (L.gu.present) {
        x = find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_GATE));
        if ((r2 = repack(*m, L.gu, x, XF_NORMAL, 0, c.inter, st))) return r2;
        x = find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_UP));
        if ((r2 = repack(*m, L.gu, x, XF_NORMAL, c.inter, c.inter, st))) return r2;
        x = find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_DOWN));
        if ((r2 = repack(*m, L.down, x, XF_NORMAL, 0, c.hidden, st))) return r2;
        if ((r2 = copy_vec(*m, L.post_norm, find_w(w, n, DSPARK_LAYER_W(l, DSPARK_L_POST_NORM)), st))) return r2;
      }
    }
    if (!m->layers_only) {
      int32_t r2;
      if ((r2 = repack(*m, m->fc, find_w(w, n, DSPARK_W_FC), XF_NORMAL, 0, c.hidden, st))) return r2;
      if ((r2 = repack(*m, m->lm, find_w(w, n, DSPARK_W_LM_HEAD), XF_NORMAL, 0, c.vocab, st))) return r2;
      if ((r2 = repack(*m, m->w2, find_w(w, n, DSPARK_W_MARKOV_W2), XF_NORMAL, 0, c.vocab, st))) return r2;
      const dspark_weight* w1 = find_w(w, n, DSPARK_W_MARKOV_W1);
      const size_t esz = m->w1_fmt == DT_F32 ? 4 : 2;
      HIPCHK(hipMemcpy2DAsync(m->base + m->w1, (size_t)m->w1_ld * esz, w1->data, (size_t)c.markov_rank * esz,
                              (size_t)c.markov_rank * esz, (size_t)c.vocab, hipMemcpyDeviceToDevice, st));
      // row-norm bounds for the exact candidate pruning of the Markov rollout
      const dspark_weight* w2s = find_w(w, n, DSPARK_W_MARKOV_W2);
      HIPCHK(launch_row_norms(w2s->data, w2s->dtype == DSPARK_DT_F32, w2s->cols, c.markov_rank, c.vocab,
                              (float*)(m->base + m->w2n), nullptr, st));
      HIPCHK(launch_row_norms(w1->data, w1->dtype == DSPARK_DT_F32, w1->cols, c.markov_rank, c.vocab, nullptr,
                              (unsigned*)(m->base + m->w1max), st));
      if ((r2 = copy_vec(*m, m->fc_norm, find_w(w, n, DSPARK_W_FC_NORM), st))) return r2;
      if ((r2 = copy_vec(*m, m->final_norm, find_w(w, n, DSPARK_W_FINAL_NORM), st))) return r2;
      if ((r2 = copy_vec(*m, m->conf_w, find_w(w, n, DSPARK_W_CONF_W), st))) return r2;
      if ((r2 = copy_vec(*m, m->conf_b, find_w(w, n, DSPARK_W_CONF_B), st))) return r2;
    }
    const std::vector<double> f = rope_freqs(c);
    HIPCHK(hipMemcpyAsync(m->base + m->freqs, f.data(), f.size() * 8, hipMemcpyHostToDevice, st));
    HIPCHK(hipStreamSynchronize(st));
    return DSPARK_OK;
  };
  rc = body();
  if (rc) {
    delete m;
    return rc;
  }
  *out = m;
  return DSPARK_OK;
}

int32_t dspark_model_destroy(dspark_model* m) {
  delete m;
  return DSPARK_OK;
}

size_t dspark_workspace_bytes(const dspark_model* m, int32_t n_seq, int64_t total_ctx) {
  if (!m || n_seq < 1 || total_ctx < 0) {
    fail(DSPARK_EINVAL, "workspace query: bad model / n_seq / total_ctx");
    return 0;
  }
  // size for the larger of the two KV precisions
  Plan a, b;
  make_plan(*m, n_seq, total_ctx, false, a);
  make_plan(*m, n_seq, total_ctx, true, b);
  return (size_t)std::max(a.total, b.total);
}

int32_t dspark_draft_block(const dspark_model* m, const dspark_block_in* in, dspark_block_out* out, void* workspace,
                           size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!m || !in || !out) return fail(DSPARK_EINVAL, "model / in / out is NULL");
  if (m->layers_only) return fail(DSPARK_EINVAL, "model holds decoder layers only");
  const dspark_config& c = m->c;
  if (in->n_seq < 1) return fail(DSPARK_EINVAL, "n_seq < 1");
  if (in->n_seq > 16) return fail(DSPARK_EUNSUPPORTED, "n_seq > 16");
  if (in->total_ctx < 0 || in->total_ctx > (1ll << 30)) return fail(DSPARK_EINVAL, "total_ctx out of range");
  if (!in->captured || !in->kv || !in->kv_offsets || !in->prev_token || !out->tokens || !out->conf)
    return fail(DSPARK_EINVAL, "a required pointer is NULL");
  if (misaligned(in->captured, 4) || misaligned(in->kv_offsets, 4) || misaligned(in->prev_token, 4) ||
      misaligned(in->forced_prev, 4) || misaligned(in->sample_u, 4) || misaligned(in->block_table, 4) ||
      misaligned(out->tokens, 4) || misaligned(out->conf, 4) || misaligned(out->logits, 4) ||
      misaligned(out->hidden, 4) || misaligned(out->status, 4))
    return fail(DSPARK_EINVAL, "an input or output pointer is not 4-byte aligned");
  if (in->act_dtype != DSPARK_DT_F32 && in->act_dtype != DSPARK_DT_BF16)
    return fail(DSPARK_EINVAL, "act_dtype must be F32 or BF16");
  if (in->kv_dtype != DSPARK_DT_F32 && in->kv_dtype != DSPARK_DT_BF16)
    return fail(DSPARK_EINVAL, "kv_dtype must be F32 or BF16");
  for (int l = 0; l < c.n_layers; ++l) {
    if (!in->kv[l] && in->total_ctx > 0) return fail(DSPARK_EINVAL, "kv[%d] is NULL", l);
    if (misaligned(in->kv[l], 16)) return fail(DSPARK_EINVAL, "kv[%d] is not 16-byte aligned", l);
  }
  const bool kv_f32 = in->kv_dtype == DSPARK_DT_F32;
  int page_log2 = -1;
  if (in->page_size != 0) {
    const int ps = in->page_size;
    if (ps < 32 || (ps & (ps - 1))) return fail(DSPARK_EINVAL, "page_size %d: not a power of two >= 32", ps);
    if (!in->block_table || in->max_pages < 1) return fail(DSPARK_EINVAL, "paged caches need block_table and max_pages");
    if (kv_f32) return fail(DSPARK_EUNSUPPORTED, "paged caches are bf16 only");
    page_log2 = __builtin_ctz((unsigned)ps);
  }
  if (in->sample_u) {
    if (!(in->temperature > 0.f)) return fail(DSPARK_EINVAL, "temperature must be > 0 when sample_u is set");
    if (!(m->w2.pm.fmt == DT_BF16 && markov_rollout_supported(m->w2.pm.KB, in->n_seq, c.vocab)))
      return fail(DSPARK_EUNSUPPORTED, "probabilistic drafting needs the bf16 Markov rollout");
  }
  Ctx C;
  C.m = m;
  make_plan(*m, in->n_seq, in->total_ctx, kv_f32, C.P);
  if (!kv_f32 && !attn_bf16_supported(C.P.DQ, c.kv_lora))
    return fail(DSPARK_EUNSUPPORTED, "no bf16 attention kernel for latent %d / kv_lora %d", c.kv_lora + c.qk_rope,
                c.kv_lora);
  if (kv_f32 && (c.kv_lora + c.qk_rope > 1024)) return fail(DSPARK_EUNSUPPORTED, "f32 latent > 1024");
  int32_t rc = check_ws(C.P, workspace, ws_bytes);
  if (rc) return rc;
  if (m->plan_only) return fail(DSPARK_EPLANONLY, "plan-only model: arguments valid, nothing enqueued");
  C.ws = (unsigned char*)workspace;
  C.st = (hipStream_t)stream;
  C.table = in->block_table;
  C.page_log2 = page_log2;
  C.max_pages = in->max_pages;
  Plan& P = C.P;
  for (Frag* f : {&P.f_fc, &P.f_qkva, &P.f_qb, &P.f_uk, &P.f_uv, &P.f_o, &P.f_gu, &P.f_down, &P.f_lm}) bind_frag(*f, C.ws);
  const int M = P.M;
  hipEvent_t* ev = (hipEvent_t*)out->stage_events;
  auto mark = [&](int idx) -> hipError_t { return ev ? hipEventRecord(ev[idx], C.st) : hipSuccess; };
  HIPCHK(mark(2 * DSPARK_STAGE_FC));
  {
    InitArgs a{};
    a.zero_ptr = C.ws + P.zero_begin;
    a.zero_bytes = P.zero_end - P.zero_begin;
    a.captured = in->captured;
    a.cap_f32 = in->act_dtype == DSPARK_DT_F32;
    a.n_seq = in->n_seq;
    a.ncap = c.n_captured;
    a.block = c.block;
    a.H = c.hidden;
    a.fd_fc = P.f_fc.fd;
    set_rope(C, a, in->kv_offsets);
    HIPCHK(launch_init(a, C.st));
  }
  if (P.p_fc.nw) {                        // y = fc output, chunk sums of y^2 (one launch)
    GemvArgs a = gemv_base(m->fc, P.p_fc, P.f_fc, M);
    a.epi = OWN_STORE;
    a.x_out = C.x();
    a.ssq_out = C.ssq(P.ssq_a);
    HIPCHK(launch_gemv(a, P.p_fc, GEMV_OWN, C.st));
    C.nch_a = c.hidden / OWN_COLS;
  } else {
    HIPCHK(run_gemv(m->fc, P.p_fc, P.f_fc, M, C.part(), C.st));
    ResidPost a = resid_base(C);          // y = fc output, chunk sums of y^2
    a.mode = RP_SUM;
    a.p = C.pin(P.p_fc, m->fc);
    a.ssq_out = C.ssq(P.ssq_a);
    HIPCHK(launch_post_resid(a, C.st));
    C.nch_a = (c.hidden + 255) / 256;
  }
  {
    ResidPost a = resid_base(C);          // x = RMSNorm(y; g_fc), fragments of in_norm * x
    a.mode = RP_NORM;
    a.rs_in = C.rs(P.ssq_a, c.hidden);
    a.g0 = (const float*)(m->base + m->fc_norm);
    a.g1 = (const float*)(m->base + m->L[0].in_norm);
    a.fd = P.f_qkva.fd;
    a.ssq_out = C.ssq(P.ssq_b);
    HIPCHK(launch_post_resid(a, C.st));
    C.nch_b = (c.hidden + 255) / 256;
  }
  HIPCHK(mark(2 * DSPARK_STAGE_FC + 1));
  HIPCHK(mark(2 * DSPARK_STAGE_LAYERS));
  for (int l = 0; l < c.n_layers; ++l) {
    const Layer& L = m->L[l];
    if ((rc = attn_half(C, l, P.ssq_b, in->kv[l], in->kv_offsets))) return rc;
    // x += o_proj; fragments of post_norm * x
    if ((rc = resid_gemm(C, L.o, P.p_o, P.f_o, C.x(), C.x(), (const float*)(m->base + L.post_norm), &P.f_gu.fd,
                         P.ssq_a, nullptr)))
      return rc;
    if ((rc = mlp_half(C, l, P.ssq_a))) return rc;
    // x += down; fragments of the next norm * x (the last layer: final norm, confidence dot)
    const bool last = l + 1 == c.n_layers;
    const float* g1 = (const float*)(m->base + (last ? m->final_norm : m->L[l + 1].in_norm));
    if ((rc = resid_gemm(C, L.down, P.p_down, P.f_down, C.x(), C.x(), g1, last ? &P.f_lm.fd : &P.f_qkva.fd, P.ssq_b,
                         last ? (const float*)(m->base + m->conf_w) : nullptr)))
      return rc;
  }
  HIPCHK(mark(2 * DSPARK_STAGE_LAYERS + 1));
  float* z = (float*)(C.ws + P.z);
  HIPCHK(mark(2 * DSPARK_STAGE_LM_HEAD));
  HIPCHK(run_gemv(m->lm, P.p_lm, P.f_lm, M, z, C.st, C.rs(P.ssq_b, c.hidden)));
  HIPCHK(mark(2 * DSPARK_STAGE_LM_HEAD + 1));
  HIPCHK(mark(2 * DSPARK_STAGE_MARKOV));
  const bool rollout = m->w2.pm.fmt == DT_BF16 && markov_rollout_supported(m->w2.pm.KB, in->n_seq, c.vocab);
  // greedy passes that need neither the full logits nor the hidden state:
  // the candidate rollout first; the full rollout only if it falls back
  const bool prune = rollout && !in->sample_u && !out->logits && !out->hidden && in->poll_limit == 0 &&
                     m->w1_fmt == DT_BF16 && markov_prune_supported(c.markov_rank, c.block, c.vocab);
  const int* fallback = prune ? (const int*)(C.ws + P.mfall) : nullptr;
  if (prune) {
    MarkovPruneArgs a{};
    a.z = z;
    a.n2 = (const float*)(m->base + m->w2n);
    a.w1max = (const unsigned*)(m->base + m->w1max);
    a.vocab = c.vocab;
    a.n_seq = in->n_seq;
    a.block = c.block;
    a.R = c.markov_rank;
    a.KB = m->w2.pm.KB;
    a.nch = P.nch_v;
    a.w2 = m->w2.pm.codes;
    a.w1 = m->base + m->w1;
    a.w1_f32 = m->w1_fmt == DT_F32;
    a.w1_ld = m->w1_ld;
    a.prev_token = in->prev_token;
    a.forced = in->forced_prev;
    a.lch = (float*)(C.ws + P.mlmax);
    a.ccnt = (int*)(C.ws + P.mlcnt);
    a.list = (u32x4*)(C.ws + P.mlist);
    a.fallback = (int*)(C.ws + P.mfall);
    a.rs_final = C.rs(P.ssq_b, c.hidden);
    a.dot = C.ssq(P.dot);
    a.nch_dot = C.nch_of(P.ssq_b, c.hidden);
    a.conf_wm = (const float*)(m->base + m->conf_w) + c.hidden;
    a.conf_b = (const float*)(m->base + m->conf_b);
    a.tokens = out->tokens;
    a.conf = out->conf;
    a.status = out->status;
    HIPCHK(launch_markov_prune(a, C.st));
  }
  if (rollout) {
    MarkovArgs a{};
    a.w2 = m->w2.pm.codes;
    a.tiles = m->w2.pm.ngroups * m->w2.pm.TG;
    a.w1 = m->base + m->w1;
    a.w1_ld = m->w1_ld;
    a.vocab = c.vocab;
    a.M = in->n_seq;
    a.block = c.block;
    a.prev_token = in->prev_token;
    a.forced = in->forced_prev;
    a.z = z;
    a.logits = out->logits;
    a.slots = (unsigned long long*)(C.ws + P.mslots);
    a.max_wgs = P.mwgs;
    a.err = (unsigned*)(C.ws + P.merr);
    a.sample_u = in->sample_u;
    a.inv_temp = in->sample_u ? 1.f / in->temperature : 1.f;
    a.spin_limit = in->poll_limit;
    a.fallback = fallback;
    HIPCHK(launch_markov_rollout(a, m->w2.pm.KB, C.st));
  }
  for (int i = 0; !rollout && i < c.block; ++i) {
    GemvArgs a{};
    a.w = m->w2.pm;
    a.act = m->base + m->w1;
    a.M = in->n_seq;
    a.ksteps_per_split = P.p_w2.ksteps_per_split;
    a.gather_ld = m->w1_ld;
    a.prev_token = in->prev_token;
    a.forced = in->forced_prev;
    a.keys = (unsigned long long*)(C.ws + P.keys);
    a.step = i;
    a.block = c.block;
    a.z = z;
    a.logits = out->logits;
    HIPCHK(launch_gemv(a, P.p_w2, GEMV_MARKOV, C.st));
  }
  {
    MarkovFinalArgs a{};
    a.keys = (const unsigned long long*)(C.ws + P.keys);
    a.prev_token = in->prev_token;
    a.forced = in->forced_prev;
    a.w1 = m->base + m->w1;
    a.w1_f32 = m->w1_fmt == DT_F32;
    a.w1_ld = m->w1_ld;
    a.R = c.markov_rank;
    a.conf_wm = (const float*)(m->base + m->conf_w) + c.hidden;
    a.conf_b = (const float*)(m->base + m->conf_b);
    a.dot = C.ssq(P.dot);
    a.nch = C.nch_of(P.ssq_b, c.hidden);  // the dot chunks come with the last sums of squares
    a.rs_final = C.rs(P.ssq_b, c.hidden);
    a.x = C.x();
    a.g_final = (const float*)(m->base + m->final_norm);
    a.H = c.hidden;
    a.hidden = out->hidden;
    a.tokens = out->tokens;
    a.conf = out->conf;
    a.n_seq = in->n_seq;
    a.block = c.block;
    a.vocab = c.vocab;
    a.slots = rollout ? (const unsigned long long*)(C.ws + P.mslots) : nullptr;
    a.nwg = rollout ? markov_rollout_wgs(m->w2.pm.ngroups * m->w2.pm.TG) : 0;
    a.rollout_err = rollout ? (const unsigned*)(C.ws + P.merr) : nullptr;
    a.status = out->status;
    a.fallback = fallback;
    HIPCHK(launch_markov_final(a, C.st));
  }
  HIPCHK(mark(2 * DSPARK_STAGE_MARKOV + 1));
  return DSPARK_OK;
}

int32_t dspark_draft_block_static(const dspark_model* m, const dspark_block_in* in, dspark_block_out* out,
                                  void* stream) {
  g_err.clear();
  if (!m || !in || !out) return fail(DSPARK_EINVAL, "model / in / out is NULL");
  if (in->n_seq < 1) return fail(DSPARK_EINVAL, "n_seq < 1");
  if (in->total_ctx < 0 || in->total_ctx > (1ll << 30)) return fail(DSPARK_EINVAL, "total_ctx out of range");
  const size_t need = dspark_workspace_bytes(m, in->n_seq, in->total_ctx);
  if (need == 0) return DSPARK_EINVAL;  // message set by the query
  if (need > DSPARK_STATIC_SCRATCH_BYTES)
    return fail(DSPARK_EWORKSPACE,
                "this call needs %zu bytes of workspace; the static scratch holds %zu (use dspark_draft_block "
                "with a caller workspace)", need, (size_t)DSPARK_STATIC_SCRATCH_BYTES);
  if (m->plan_only) return dspark_draft_block(m, in, out, (void*)(uintptr_t)256, need, stream);
  void* ws = nullptr;
  size_t bytes = 0;
  HIPCHK(static_scratch(&ws, &bytes));
  return dspark_draft_block(m, in, out, ws, bytes, stream);
}

int32_t dspark_layer_forward(const dspark_model* m, int32_t layer, int32_t with_mlp, int32_t n_seq, const float* x_in,
                             float* x_out, const void* kv, int32_t kv_dtype, const int32_t* kv_offsets,
                             int64_t total_ctx, void* workspace, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!m) return fail(DSPARK_EINVAL, "model is NULL");
  const dspark_config& c = m->c;
  if (layer < 0 || layer >= c.n_layers) return fail(DSPARK_EINVAL, "layer %d out of range", layer);
  if (with_mlp && !m->L[layer].gu.present) return fail(DSPARK_EINVAL, "layer %d has no MLP weights", layer);
  if (n_seq < 1) return fail(DSPARK_EINVAL, "n_seq < 1");
  if (!x_in || !x_out || !kv_offsets || (!kv && total_ctx > 0)) return fail(DSPARK_EINVAL, "a required pointer is NULL");
  if (kv_dtype != DSPARK_DT_F32 && kv_dtype != DSPARK_DT_BF16) return fail(DSPARK_EINVAL, "bad kv_dtype");
  if (total_ctx < 0 || total_ctx > (1ll << 30)) return fail(DSPARK_EINVAL, "total_ctx out of range");
  const bool kv_f32 = kv_dtype == DSPARK_DT_F32;
  Ctx C;
  C.m = m;
  make_plan(*m, n_seq, total_ctx, kv_f32, C.P);
  if (!kv_f32 && !attn_bf16_supported(C.P.DQ, c.kv_lora))
    return fail(DSPARK_EUNSUPPORTED, "no bf16 attention kernel for this latent size");
  int32_t rc = check_ws(C.P, workspace, ws_bytes);
  if (rc) return rc;
  if (misaligned(x_in, 16) || misaligned(x_out, 16) || misaligned(kv, 16) || misaligned(kv_offsets, 4))
    return fail(DSPARK_EINVAL, "x_in / x_out / kv not 16-byte or kv_offsets not 4-byte aligned");
  if (m->plan_only) return fail(DSPARK_EPLANONLY, "plan-only model: arguments valid, nothing enqueued");
  C.ws = (unsigned char*)workspace;
  C.st = (hipStream_t)stream;
  Plan& P = C.P;
  for (Frag* f : {&P.f_qkva, &P.f_qb, &P.f_uk, &P.f_uv, &P.f_o, &P.f_gu, &P.f_down}) bind_frag(*f, C.ws);
  {
    InitArgs a{};
    a.zero_ptr = C.ws + P.zero_begin;
    a.zero_bytes = P.zero_end - P.zero_begin;
    a.n_seq = n_seq;
    a.block = c.block;
    set_rope(C, a, kv_offsets);
    HIPCHK(launch_init(a, C.st));
  }
  const Layer& L = m->L[layer];
  {
    ResidPost a = resid_base(C);          // x = x_in, fragments of in_norm * x
    a.mode = RP_COPY;
    a.x_in = x_in;
    a.g1 = (const float*)(m->base + L.in_norm);
    a.fd = P.f_qkva.fd;
    a.ssq_out = C.ssq(P.ssq_b);
    HIPCHK(launch_post_resid(a, C.st));
  }
  if ((rc = attn_half(C, layer, P.ssq_b, kv, kv_offsets))) return rc;
  if (!with_mlp) return resid_gemm(C, L.o, P.p_o, P.f_o, C.x(), x_out, nullptr, nullptr, -1, nullptr);
  if ((rc = resid_gemm(C, L.o, P.p_o, P.f_o, C.x(), C.x(), (const float*)(m->base + L.post_norm), &P.f_gu.fd,
                       P.ssq_a, nullptr)))
    return rc;
  if ((rc = mlp_half(C, layer, P.ssq_a))) return rc;
  return resid_gemm(C, L.down, P.p_down, P.f_down, C.x(), x_out, nullptr, nullptr, -1, nullptr);
}

// ---------------------------------------------------------- cache append --
namespace {

// Rows row0 .. row0 + nrows - 1 of a packed matrix as a matrix of its own
// (16-row tiles are stored one after another, codes and scales alike).
bool row_view(const Mat& mt, int row0, int nrows, PackedMat& out) {
  const PackedMat& p = mt.pm;
  if (!mt.present || p.ngroups != 1 || row0 % 16 || row0 + nrows > p.G) return false;
  const long long t0 = row0 / 16;
  out = p;
  // (a plan-only model has no packed buffer: its views stay null)
  if (p.codes) out.codes = p.codes + t0 * 16 * code_bytes(p.fmt, p.Kp);
  if (p.scales) out.scales = (const unsigned char*)p.scales + t0 * scale_tile_bytes(p);
  out.G = nrows;
  out.TG = (int)cdiv(nrows, 16);
  return true;
}

struct AppendPlan {
  int M = 0;
  Frag f_fc, f_kv;
  GemvPlan p_fc{}, p_kv{};
  PackedMat kv{};  // geometry of the kv_a rows (layer 0's view)
  long long x = 0, part = 0, ssq_a = 0, ssq_b = 0, rope = 0, zero_begin = 0, zero_end = 0, total = 0;
};

int32_t make_append_plan(const dspark_model& m, int n_new, AppendPlan& A) {
  const dspark_config& c = m.c;
  if (m.layers_only) return fail(DSPARK_EINVAL, "model holds decoder layers only");
  if (n_new < 1 || n_new > DSPARK_APPEND_MAX) return fail(DSPARK_EINVAL, "n_new %d out of range", n_new);
  const int latent = c.kv_lora + c.qk_rope;
  if (!row_view(m.L[0].qkva, c.q_lora, latent, A.kv))
    return fail(DSPARK_EUNSUPPORTED, "kv_a rows start at q_lora %d: not a multiple of 16", c.q_lora);
  A.M = n_new;
  long long off = 0;
  auto take = [&](long long bytes) {
    const long long o = off;
    off = rup(off + bytes, 256);
    return o;
  };
  A.p_fc = plan_gemv(m.fc.pm, n_new, true, false, true);
  A.p_kv = plan_gemv(A.kv, n_new, true, false, true);
  frag_geom(A.f_fc, m.fc.pm, n_new, A.p_fc);
  frag_geom(A.f_kv, A.kv, n_new, A.p_kv);
  A.f_fc.off = take(A.f_fc.bytes);  // written whole by k_init
  A.zero_begin = off;
  A.f_kv.off = take(A.f_kv.bytes);
  A.zero_end = off;
  A.x = take((long long)n_new * c.hidden * 4);
  A.part = take(std::max((long long)A.p_fc.S * n_new * m.fc.pm.G, (long long)A.p_kv.S * n_new * A.kv.G) * 4);
  A.ssq_a = take((long long)n_new * SSQ_LD * 4);
  A.ssq_b = take((long long)n_new * SSQ_LD * 4);
  A.rope = take((long long)n_new * (c.qk_rope / 2) * 8);
  A.total = off;
  return DSPARK_OK;
}

}  // namespace

size_t dspark_append_workspace_bytes(const dspark_model* m, int32_t n_new) {
  g_err.clear();
  if (!m) {
    fail(DSPARK_EINVAL, "model is NULL");
    return 0;
  }
  AppendPlan A;
  if (make_append_plan(*m, n_new, A)) return 0;
  return (size_t)A.total;
}

int32_t dspark_cache_append(const dspark_model* m, const dspark_append_in* in, void* workspace, size_t ws_bytes,
                            void* stream) {
  g_err.clear();
  if (!m || !in) return fail(DSPARK_EINVAL, "model / in is NULL");
  const dspark_config& c = m->c;
  AppendPlan A;
  int32_t rc = make_append_plan(*m, in->n_new, A);
  if (rc) return rc;
  if (!in->captured || !in->positions || !in->slot_mapping || !in->kv) return fail(DSPARK_EINVAL, "a required pointer is NULL");
  for (int l = 0; l < c.n_layers; ++l)
    if (!in->kv[l]) return fail(DSPARK_EINVAL, "kv[%d] is NULL", l);
  if (in->act_dtype != DSPARK_DT_F32 && in->act_dtype != DSPARK_DT_BF16) return fail(DSPARK_EINVAL, "bad act_dtype");
  if (in->kv_dtype != DSPARK_DT_F32 && in->kv_dtype != DSPARK_DT_BF16) return fail(DSPARK_EINVAL, "bad kv_dtype");
  if (!workspace || (uintptr_t)workspace % 256) return fail(DSPARK_EINVAL, "workspace NULL or not 256-byte aligned");
  if ((long long)ws_bytes < A.total) return fail(DSPARK_EWORKSPACE, "workspace %zu bytes, need %lld", ws_bytes, A.total);
  if (misaligned(in->captured, 4) || misaligned(in->positions, 4) || misaligned(in->slot_mapping, 8))
    return fail(DSPARK_EINVAL, "captured / positions not 4-byte or slot_mapping not 8-byte aligned");
  for (int l = 0; l < c.n_layers; ++l)
    if (misaligned(in->kv[l], 16)) return fail(DSPARK_EINVAL, "kv[%d] is not 16-byte aligned", l);
  if (m->plan_only) return fail(DSPARK_EPLANONLY, "plan-only model: arguments valid, nothing enqueued");
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  bind_frag(A.f_fc, ws);
  bind_frag(A.f_kv, ws);
  const int M = A.M, H = c.hidden;
  float* x = (float*)(ws + A.x);
  float* part = (float*)(ws + A.part);
  auto rs = [&](long long o, int n) {
    RowScale r{};
    r.ssq = (const float*)(ws + o);
    r.nch = (n + 255) / 256;
    r.invn = 1.f / (float)n;
    r.eps = c.rms_eps;
    return r;
  };
  {  // zeroed fragments, fc input fragments of each row, RoPE table at the given positions
    InitArgs a{};
    a.zero_ptr = ws + A.zero_begin;
    a.zero_bytes = A.zero_end - A.zero_begin;
    a.captured = in->captured;
    a.cap_f32 = in->act_dtype == DSPARK_DT_F32;
    a.n_seq = M;  // one row per "sequence": captured is [n_new][n_captured][1][hidden]
    a.ncap = c.n_captured;
    a.block = 1;
    a.H = H;
    a.fd_fc = A.f_fc.fd;
    a.rope = (float*)(ws + A.rope);
    a.positions = in->positions;
    a.freqs = (const double*)(m->base + m->freqs);
    a.npairs = c.qk_rope / 2;
    HIPCHK(launch_init(a, st));
  }
  {  // fc
    GemvArgs g{};
    g.w = m->fc.pm;
    g.act = A.f_fc.fd.ptr;
    g.act_gstride = A.f_fc.fd.gstride;
    g.act_ld = A.f_fc.fd.ld;
    g.M = M;
    g.hilo = A.p_fc.hilo;
    g.ksteps_per_split = A.p_fc.ksteps_per_split;
    g.out = part;
    g.out_ld = m->fc.pm.G;
    g.out_split_stride = (long long)M * g.out_ld;
    HIPCHK(launch_gemv(g, A.p_fc, GEMV_STORE, st));
  }
  auto resid = [&]() {
    ResidPost a{};
    a.x_in = x;
    a.x_out = x;
    a.M = M;
    a.H = H;
    return a;
  };
  {  // y = fc output (chunk sums of y^2)
    ResidPost a = resid();
    a.mode = RP_SUM;
    a.p = PartIn{part, A.p_fc.S, (long long)m->fc.pm.G, (long long)M * m->fc.pm.G};
    a.ssq_out = (float*)(ws + A.ssq_a);
    HIPCHK(launch_post_resid(a, st));
  }
  {  // x = RMSNorm(y; g_fc) (chunk sums of x^2), fragments of in_norm_0 * x
    ResidPost a = resid();
    a.mode = RP_NORM;
    a.rs_in = rs(A.ssq_a, H);
    a.g0 = (const float*)(m->base + m->fc_norm);
    a.g1 = (const float*)(m->base + m->L[0].in_norm);
    a.fd = A.f_kv.fd;
    a.ssq_out = (float*)(ws + A.ssq_b);
    HIPCHK(launch_post_resid(a, st));
  }
  const int latent = c.kv_lora + c.qk_rope;
  for (int l = 0; l < c.n_layers; ++l) {
    const Layer& L = m->L[l];
    if (l > 0) {  // fragments of in_norm_l * x
      ResidPost a = resid();
      a.mode = RP_COPY;
      a.g1 = (const float*)(m->base + L.in_norm);
      a.fd = A.f_kv.fd;
      HIPCHK(launch_post_resid(a, st));
    }
    PackedMat kv{};
    if (!row_view(L.qkva, c.q_lora, latent, kv)) return fail(DSPARK_EUNSUPPORTED, "kv_a view of layer %d", l);
    GemvArgs g{};
    g.w = kv;
    g.act = A.f_kv.fd.ptr;
    g.act_gstride = A.f_kv.fd.gstride;
    g.act_ld = A.f_kv.fd.ld;
    g.M = M;
    g.hilo = A.p_kv.hilo;
    g.ksteps_per_split = A.p_kv.ksteps_per_split;
    g.out = part;
    g.out_ld = kv.G;
    g.out_split_stride = (long long)M * kv.G;
    HIPCHK(launch_gemv(g, A.p_kv, GEMV_STORE, st));
    KvRowPost a{};
    a.p = PartIn{part, A.p_kv.S, (long long)kv.G, (long long)M * kv.G};
    a.rs_in = rs(A.ssq_b, H);
    a.M = M;
    a.r = c.kv_lora;
    a.dr = c.qk_rope;
    a.latent = latent;
    a.g_kva = (const float*)(m->base + L.kv_a_norm);
    a.eps = c.rms_eps;
    a.rope = (const float*)(ws + A.rope);
    a.dst = in->kv[l];
    a.dst_f32 = in->kv_dtype == DSPARK_DT_F32;
    a.slot = in->slot_mapping;
    HIPCHK(launch_post_kv_rows(a, st));
  }
  return DSPARK_OK;
}

// ------------------------------------------------------------ verification --
size_t dspark_verify_workspace_bytes(int32_t n_seq, int32_t block) {
  g_err.clear();
  if (n_seq < 1 || block < 1 || block > 63) {
    fail(DSPARK_EINVAL, "verify workspace: bad n_seq / block");
    return 0;
  }
  const long long nch = verify_nch();
  return (size_t)(rup((long long)n_seq * (block + 1) * nch * 4 * 4, 256) + rup((long long)n_seq * block * nch * 2 * 4, 256) +
                  (long long)n_seq * (block + 1) * 8 * 4);
}

int32_t dspark_verify(const dspark_verify_in* in, int32_t* out_len, int32_t* out_token, void* workspace,
                      size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!in || !out_len || !out_token) return fail(DSPARK_EINVAL, "in / out_len / out_token is NULL");
  if (in->n_seq < 1 || in->block < 1 || in->block > 63 || in->vocab < 1)
    return fail(DSPARK_EINVAL, "bad n_seq / block / vocab");
  if (in->method != DSPARK_VERIFY_TOKEN && in->method != DSPARK_VERIFY_BLOCK) return fail(DSPARK_EINVAL, "bad method");
  if (!(in->temperature > 0.f)) return fail(DSPARK_EINVAL, "temperature must be > 0");
  if (!in->draft || !in->draft_logits || !in->target_logits || !in->u) return fail(DSPARK_EINVAL, "a required pointer is NULL");
  const size_t need = dspark_verify_workspace_bytes(in->n_seq, in->block);
  if (!workspace || (uintptr_t)workspace % 256) return fail(DSPARK_EINVAL, "workspace NULL or not 256-byte aligned");
  if (ws_bytes < need) return fail(DSPARK_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  VerifyArgs a{};
  a.n_seq = in->n_seq;
  a.block = in->block;
  a.vocab = in->vocab;
  a.method = in->method == DSPARK_VERIFY_TOKEN ? DSPARK_VERIFY_TOKEN_C : DSPARK_VERIFY_BLOCK_C;
  a.inv_temp = 1.f / in->temperature;
  a.draft = in->draft;
  a.dlog = in->draft_logits;
  a.tlog = in->target_logits;
  a.u = in->u;
  a.stats = (float*)workspace;
  const long long stats_b = rup((long long)in->n_seq * (in->block + 1) * verify_nch() * 4 * 4, 256);
  a.resid = (float*)((unsigned char*)workspace + stats_b);
  a.probs = (float*)((unsigned char*)workspace + stats_b + rup((long long)in->n_seq * in->block * verify_nch() * 2 * 4, 256));
  a.out_len = out_len;
  a.out_token = out_token;
  HIPCHK(launch_verify(a, (hipStream_t)stream));
  return DSPARK_OK;
}

int32_t dspark_accept_len_host(const int32_t* draft, const int32_t* verifier, int32_t n_seq, int32_t block,
                               int32_t* out_len) {
  g_err.clear();
  if (!draft || !verifier || !out_len) return fail(DSPARK_EINVAL, "NULL pointer");
  if (n_seq < 0 || block < 0) return fail(DSPARK_EINVAL, "negative n_seq / block");
  for (int s = 0; s < n_seq; ++s) {
    int k = 0;
    while (k < block && draft[(long long)s * block + k] == verifier[(long long)s * block + k]) ++k;
    out_len[s] = k;
  }
  return DSPARK_OK;
}

int32_t dspark_accept_len(const int32_t* draft, const int32_t* verifier, int32_t n_seq, int32_t block,
                          int32_t* out_len, void* stream) {
  g_err.clear();
  if (!draft || !verifier || !out_len) return fail(DSPARK_EINVAL, "NULL pointer");
  if (n_seq < 0 || block < 0) return fail(DSPARK_EINVAL, "negative n_seq / block");
  if (n_seq == 0) return DSPARK_OK;
  HIPCHK(launch_accept_len(draft, verifier, n_seq, block, out_len, (hipStream_t)stream));
  return DSPARK_OK;
}

static_assert(READ_PROBE_WGS == 2048, "the header promises 2048 output words");

int32_t dspark_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  g_err.clear();
  if (!buf || !out) return fail(DSPARK_EINVAL, "NULL pointer");
  if (misaligned(buf, 16) || bytes % 16 || misaligned(out, 4))
    return fail(DSPARK_EINVAL, "buf must be 16-byte aligned, bytes a multiple of 16, out 4-byte aligned");
  HIPCHK(launch_read_probe(buf, bytes, out, (hipStream_t)stream));
  return DSPARK_OK;
}

int32_t dspark_dequant(const dspark_model* m, int32_t id, float* out, void* stream) {
  g_err.clear();
  if (!m || !out) return fail(DSPARK_EINVAL, "NULL pointer");
  const Mat* mt = nullptr;
  if (id == DSPARK_W_FC) mt = &m->fc;
  else if (id == DSPARK_W_LM_HEAD) mt = &m->lm;
  else if (id == DSPARK_W_MARKOV_W2) mt = &m->w2;
  else if (id >= DSPARK_W_LAYER_BASE) {
    const int l = (id - DSPARK_W_LAYER_BASE) / DSPARK_W_LAYER_STRIDE, k = (id - DSPARK_W_LAYER_BASE) % DSPARK_W_LAYER_STRIDE;
    if (l < m->c.n_layers) {
      const Layer& L = m->L[l];
      switch (k) {
        case DSPARK_L_Q_B: mt = &L.qb; break;
        case DSPARK_L_O: mt = &L.o; break;
        case DSPARK_L_DOWN: mt = &L.down; break;
        case DSPARK_L_GATE: mt = &L.gu; break;   // gate rows then up rows
        case DSPARK_L_Q_A: mt = &L.qkva; break;  // q_a rows then kv_a rows
        default: break;
      }
    }
  }
  if (!mt || !mt->present) return fail(DSPARK_EINVAL, "weight id %d has no packed matrix to decode", id);
  if (m->plan_only) return fail(DSPARK_EPLANONLY, "plan-only model: arguments valid, nothing enqueued");
  HIPCHK(launch_dequant(mt->pm, out, (hipStream_t)stream));
  return DSPARK_OK;
}

}  // extern "C"
