// Host-side checks of the C ABI (include/dspark.h) without a device: every
// pre-enqueue validation error of every call, on plan-only models
// (DSPARK_CFG_PLAN_ONLY), and the host acceptance length brute-forced over all
// (draft, verifier) pairs of small alphabets.  Built with AddressSanitizer
// and UndefinedBehaviorSanitizer against a host-only sanitized build of the
// library (tests/test_abi_host.py); prints "ok <n> checks" and exits 0, or
// names the first failing check and exits 1.
//
// Device pointers are fake, aligned addresses: plan-only models never read
// them and nothing is enqueued, so no device is touched.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../include/dspark.h"

namespace {

int g_checks = 0, g_fail = 0;

void expect(int32_t got, int32_t want, const char* what) {
  ++g_checks;
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: got %d want %d (%s)\n", what, got, want, dspark_last_error());
    ++g_fail;
    return;
  }
  if (want != DSPARK_OK && std::strlen(dspark_last_error()) == 0) {
    std::fprintf(stderr, "FAIL %s: no error text\n", what);
    ++g_fail;
  }
}

void expect_true(bool ok, const char* what) {
  ++g_checks;
  if (!ok) {
    std::fprintf(stderr, "FAIL %s\n", what);
    ++g_fail;
  }
}

const void* fake(uintptr_t k) { return (const void*)(uintptr_t)(0x10000000ull + k * 0x100000ull); }

// The ragged small geometry: hidden 352, 2 layers, 4 heads, q_lora 96,
// latent 64 + 16, nope 32, v 24, inter 480, vocab 1000, Markov rank 24.
dspark_config small_cfg() {
  dspark_config c{};
  c.hidden = 352; c.n_layers = 2; c.n_heads = 4; c.q_lora = 96; c.kv_lora = 64; c.qk_nope = 32;
  c.qk_rope = 16; c.v_head = 24; c.inter = 480; c.vocab = 1000; c.markov_rank = 24; c.block = 7;
  c.n_captured = 5; c.flags = DSPARK_CFG_PLAN_ONLY; c.rms_eps = 1e-6f; c.rope_theta = 10000.f;
  c.yarn_factor = 4.f; c.yarn_orig_ctx = 128; c.yarn_beta_fast = 32.f; c.yarn_beta_slow = 1.f;
  return c;
}

// Weight table: Q8_0 fc / q_b / o / MLP, BF16 q_a / kv_a / kv_b / lm_head /
// Markov, F32 norms and confidence head.
std::vector<dspark_weight> table(const dspark_config& c) {
  std::vector<dspark_weight> w;
  uintptr_t k = 0;
  auto add = [&](int id, int dt, long long r, long long cols) {
    dspark_weight x{};
    x.id = id; x.dtype = dt; x.data = fake(k++); x.scales = dt == DSPARK_DT_FP8_E4M3 ? fake(k++) : nullptr;
    x.rows = r; x.cols = cols;
    w.push_back(x);
  };
  const long long H = c.hidden, nh = c.n_heads, lat = c.kv_lora + c.qk_rope;
  add(DSPARK_W_FC, DSPARK_DT_Q8_0, H, c.n_captured * H);
  add(DSPARK_W_FC_NORM, DSPARK_DT_F32, H, 1);
  add(DSPARK_W_FINAL_NORM, DSPARK_DT_F32, H, 1);
  add(DSPARK_W_LM_HEAD, DSPARK_DT_BF16, c.vocab, H);
  add(DSPARK_W_MARKOV_W1, DSPARK_DT_BF16, c.vocab, c.markov_rank);
  add(DSPARK_W_MARKOV_W2, DSPARK_DT_BF16, c.vocab, c.markov_rank);
  add(DSPARK_W_CONF_W, DSPARK_DT_F32, H + c.markov_rank, 1);
  add(DSPARK_W_CONF_B, DSPARK_DT_F32, 1, 1);
  for (int l = 0; l < c.n_layers; ++l) {
    add(DSPARK_LAYER_W(l, DSPARK_L_IN_NORM), DSPARK_DT_F32, H, 1);
    add(DSPARK_LAYER_W(l, DSPARK_L_Q_A), DSPARK_DT_BF16, c.q_lora, H);
    add(DSPARK_LAYER_W(l, DSPARK_L_Q_A_NORM), DSPARK_DT_F32, c.q_lora, 1);
    add(DSPARK_LAYER_W(l, DSPARK_L_KV_A), DSPARK_DT_BF16, lat, H);
    add(DSPARK_LAYER_W(l, DSPARK_L_KV_A_NORM), DSPARK_DT_F32, c.kv_lora, 1);
    add(DSPARK_LAYER_W(l, DSPARK_L_Q_B), DSPARK_DT_Q8_0, nh * (c.qk_nope + c.qk_rope), c.q_lora);
    add(DSPARK_LAYER_W(l, DSPARK_L_KV_B), DSPARK_DT_BF16, nh * (c.qk_nope + c.v_head), c.kv_lora);
    add(DSPARK_LAYER_W(l, DSPARK_L_O), DSPARK_DT_Q8_0, H, nh * c.v_head);
    add(DSPARK_LAYER_W(l, DSPARK_L_POST_NORM), DSPARK_DT_F32, H, 1);
    add(DSPARK_LAYER_W(l, DSPARK_L_GATE), DSPARK_DT_Q8_0, c.inter, H);
    add(DSPARK_LAYER_W(l, DSPARK_L_UP), DSPARK_DT_Q8_0, c.inter, H);
    add(DSPARK_LAYER_W(l, DSPARK_L_DOWN), DSPARK_DT_Q8_0, H, c.inter);
  }
  return w;
}

dspark_weight* find(std::vector<dspark_weight>& w, int id) {
  for (auto& x : w)
    if (x.id == id) return &x;
  return nullptr;
}

int32_t create(const dspark_config& c, const std::vector<dspark_weight>& w, dspark_model** m) {
  return dspark_model_create(&c, w.data(), (int32_t)w.size(), nullptr, 0, nullptr, m);
}

void config_and_table_checks(bool no_device) {
  dspark_model* m = nullptr;
  dspark_config c = small_cfg();
  std::vector<dspark_weight> w = table(c);
  expect(create(c, w, &m), DSPARK_OK, "plan-only create");
  expect_true(m != nullptr, "plan-only handle");
  dspark_model_destroy(m);
  expect(dspark_model_create(nullptr, w.data(), (int32_t)w.size(), nullptr, 0, nullptr, &m), DSPARK_EINVAL, "cfg NULL");
  expect(dspark_model_create(&c, w.data(), (int32_t)w.size(), nullptr, 0, nullptr, nullptr), DSPARK_EINVAL, "out NULL");
  expect(dspark_model_create(&c, nullptr, 0, nullptr, 0, nullptr, &m), DSPARK_EINVAL, "empty table");
  auto bad_cfg = [&](void (*mut)(dspark_config&), int32_t want, const char* what) {
    dspark_config d = small_cfg();
    mut(d);
    dspark_model* mm = nullptr;
    expect(create(d, w, &mm), want, what);
    expect_true(mm == nullptr, "no handle after an error");
    expect_true(dspark_packed_bytes(&d, w.data(), (int32_t)w.size()) == 0, what);
  };
  bad_cfg([](dspark_config& d) { d.hidden = 0; }, DSPARK_EINVAL, "hidden 0");
  bad_cfg([](dspark_config& d) { d.n_heads = -4; }, DSPARK_EINVAL, "negative heads");
  bad_cfg([](dspark_config& d) { d.vocab = 0; }, DSPARK_EINVAL, "vocab 0");
  bad_cfg([](dspark_config& d) { d.qk_rope = 15; }, DSPARK_EUNSUPPORTED, "odd rope");
  bad_cfg([](dspark_config& d) { d.kv_lora = 56; }, DSPARK_EUNSUPPORTED, "kv_lora not a multiple of 16");
  bad_cfg([](dspark_config& d) { d.block = 65; }, DSPARK_EUNSUPPORTED, "block > 64");
  bad_cfg([](dspark_config& d) { d.flags |= 4; }, DSPARK_EINVAL, "unknown flag");
  bad_cfg([](dspark_config& d) { d.yarn_factor = 0.5f; }, DSPARK_EINVAL, "yarn factor < 1");
  bad_cfg([](dspark_config& d) { d.rms_eps = -1.f; }, DSPARK_EINVAL, "negative eps");
  bad_cfg([](dspark_config& d) { d.rope_theta = NAN; }, DSPARK_EINVAL, "NaN rope base");

  auto bad_table = [&](int id, void (*mut)(dspark_weight&), int32_t want, const char* what) {
    std::vector<dspark_weight> v = table(c);
    mut(*find(v, id));
    dspark_model* mm = nullptr;
    expect(create(c, v, &mm), want, what);
    expect_true(dspark_packed_bytes(&c, v.data(), (int32_t)v.size()) == 0, what);
  };
  bad_table(DSPARK_W_FC, [](dspark_weight& x) { x.rows += 1; }, DSPARK_EINVAL, "fc shape");
  bad_table(DSPARK_LAYER_W(1, DSPARK_L_DOWN), [](dspark_weight& x) { x.id = 999; }, DSPARK_EINVAL, "down missing");
  bad_table(DSPARK_W_LM_HEAD, [](dspark_weight& x) { x.dtype = 9; }, DSPARK_EUNSUPPORTED, "unknown dtype");
  bad_table(DSPARK_W_LM_HEAD, [](dspark_weight& x) { x.data = nullptr; }, DSPARK_EINVAL, "data NULL");
  bad_table(DSPARK_LAYER_W(0, DSPARK_L_O), [](dspark_weight& x) { x.dtype = DSPARK_DT_FP8_E4M3; x.scales = nullptr; },
            DSPARK_EINVAL, "FP8 without scales");
  bad_table(DSPARK_LAYER_W(0, DSPARK_L_KV_A), [](dspark_weight& x) { x.dtype = DSPARK_DT_F32; }, DSPARK_EUNSUPPORTED,
            "q_a / kv_a dtypes differ");
  bad_table(DSPARK_LAYER_W(0, DSPARK_L_KV_B), [](dspark_weight& x) { x.dtype = DSPARK_DT_Q8_0; }, DSPARK_EUNSUPPORTED,
            "kv_b Q8_0");
  bad_table(DSPARK_LAYER_W(0, DSPARK_L_UP), [](dspark_weight& x) { x.dtype = DSPARK_DT_BF16; }, DSPARK_EUNSUPPORTED,
            "gate / up dtypes differ");
  bad_table(DSPARK_W_MARKOV_W1, [](dspark_weight& x) { x.dtype = DSPARK_DT_F32; }, DSPARK_EUNSUPPORTED,
            "W1 / W2 dtypes differ");
  bad_table(DSPARK_W_CONF_W, [](dspark_weight& x) { x.rows -= 1; }, DSPARK_EINVAL, "conf_w length");
  bad_table(DSPARK_W_FC_NORM, [](dspark_weight& x) { x.dtype = DSPARK_DT_BF16; }, DSPARK_EUNSUPPORTED, "norm not F32");
  bad_table(DSPARK_LAYER_W(1, DSPARK_L_GATE), [](dspark_weight& x) { x.dtype = DSPARK_DT_FP8_E4M3; x.scales = x.data; },
            DSPARK_EUNSUPPORTED, "gate FP8 / up Q8_0");
  {
    // Q8_0 with a reduction length that is not a multiple of 32 (q_lora 88 -> q_b K 88)
    dspark_config d = small_cfg();
    d.q_lora = 88;
    std::vector<dspark_weight> v = table(d);
    dspark_model* mm = nullptr;
    expect(create(d, v, &mm), DSPARK_EUNSUPPORTED, "Q8_0 K % 32");
  }
  {
    // MXFP4 needs round_up(K, 64) % 128 == 0: K = 352 -> 384 is fine, 96 -> 128 fine, 480 -> 512 fine;
    // fc K = 1760 -> 1792 = 14 * 128 fine; o K = 96 fine.  A K of 160 (-> 192) is not.
    dspark_config d = small_cfg();
    d.q_lora = 160;
    std::vector<dspark_weight> v = table(d);
    for (auto& x : v)
      if (x.dtype == DSPARK_DT_Q8_0) x.dtype = DSPARK_DT_MXFP4;
    dspark_model* mm = nullptr;
    expect(create(d, v, &mm), DSPARK_EUNSUPPORTED, "MXFP4 K rounding");
  }
  if (no_device) {
    // the whole validation runs before the device query
    dspark_config d = small_cfg();
    d.flags = 0;
    dspark_model* mm = nullptr;
    expect(create(d, w, &mm), DSPARK_ENODEVICE, "create without a device");
    d.hidden = 0;
    expect(create(d, w, &mm), DSPARK_EINVAL, "validation precedes the device query");
  }
  expect_true(dspark_packed_bytes(&c, w.data(), (int32_t)w.size()) > 0, "packed bytes");
}

struct DraftCall {
  dspark_block_in in{};
  dspark_block_out out{};
  const void* kv[2];
  void* ws = nullptr;
  size_t ws_bytes = 0;
};

DraftCall valid_draft(const dspark_model* m) {
  DraftCall d;
  d.kv[0] = fake(200);
  d.kv[1] = fake(201);
  d.in.n_seq = 3;
  d.in.act_dtype = DSPARK_DT_BF16;
  d.in.kv_dtype = DSPARK_DT_BF16;
  d.in.total_ctx = 337;
  d.in.captured = fake(202);
  d.in.kv = d.kv;
  d.in.kv_offsets = (const int32_t*)fake(203);
  d.in.prev_token = (const int32_t*)fake(204);
  d.out.tokens = (int32_t*)fake(205);
  d.out.conf = (float*)fake(206);
  d.ws_bytes = dspark_workspace_bytes(m, 3, 337);
  d.ws = (void*)fake(300);
  return d;
}

int32_t run(const dspark_model* m, DraftCall& d) {
  return dspark_draft_block(m, &d.in, &d.out, d.ws, d.ws_bytes, nullptr);
}

void draft_checks(const dspark_model* m, const dspark_model* layers_only) {
  {
    DraftCall d = valid_draft(m);
    expect_true(d.ws_bytes > 0, "workspace bytes");
    expect(run(m, d), DSPARK_EPLANONLY, "valid draft");
    d.out.logits = (float*)fake(207);
    d.out.hidden = (float*)fake(208);
    d.out.status = (int32_t*)fake(209);
    d.in.forced_prev = (const int32_t*)fake(210);
    expect(run(m, d), DSPARK_EPLANONLY, "valid draft, optional outputs");
    d.in.page_size = 64; d.in.max_pages = 8; d.in.block_table = (const int32_t*)fake(211);
    expect(run(m, d), DSPARK_EPLANONLY, "valid paged draft");
    d.in.sample_u = (const float*)fake(212); d.in.temperature = 0.7f;
    expect(run(m, d), DSPARK_EPLANONLY, "valid sampled draft");
    d.in.poll_limit = -1;
    expect(run(m, d), DSPARK_EPLANONLY, "poll limit");
  }
  struct Mut {
    void (*f)(DraftCall&);
    int32_t want;
    const char* what;
  };
  const Mut muts[] = {
      {[](DraftCall& d) { d.in.n_seq = 0; }, DSPARK_EINVAL, "n_seq 0"},
      {[](DraftCall& d) { d.in.n_seq = 17; }, DSPARK_EUNSUPPORTED, "n_seq 17"},
      {[](DraftCall& d) { d.in.total_ctx = -1; }, DSPARK_EINVAL, "total_ctx < 0"},
      {[](DraftCall& d) { d.in.total_ctx = (1ll << 31); }, DSPARK_EINVAL, "total_ctx too large"},
      {[](DraftCall& d) { d.in.captured = nullptr; }, DSPARK_EINVAL, "captured NULL"},
      {[](DraftCall& d) { d.in.captured = (const char*)d.in.captured + 2; }, DSPARK_EINVAL, "captured misaligned"},
      {[](DraftCall& d) { d.in.kv = nullptr; }, DSPARK_EINVAL, "kv array NULL"},
      {[](DraftCall& d) { d.kv[1] = nullptr; }, DSPARK_EINVAL, "kv[1] NULL"},
      {[](DraftCall& d) { d.kv[0] = (const char*)d.kv[0] + 8; }, DSPARK_EINVAL, "kv[0] misaligned"},
      {[](DraftCall& d) { d.in.kv_offsets = nullptr; }, DSPARK_EINVAL, "offsets NULL"},
      {[](DraftCall& d) { d.in.prev_token = (const int32_t*)((const char*)d.in.prev_token + 1); }, DSPARK_EINVAL,
       "prev_token misaligned"},
      {[](DraftCall& d) { d.out.tokens = nullptr; }, DSPARK_EINVAL, "tokens NULL"},
      {[](DraftCall& d) { d.out.conf = (float*)((char*)d.out.conf + 2); }, DSPARK_EINVAL, "conf misaligned"},
      {[](DraftCall& d) { d.out.logits = (float*)((char*)fake(207) + 1); }, DSPARK_EINVAL, "logits misaligned"},
      {[](DraftCall& d) { d.in.act_dtype = DSPARK_DT_Q8_0; }, DSPARK_EINVAL, "act dtype"},
      {[](DraftCall& d) { d.in.kv_dtype = DSPARK_DT_FP8_E4M3; }, DSPARK_EINVAL, "kv dtype"},
      {[](DraftCall& d) { d.in.page_size = 48; d.in.max_pages = 8; d.in.block_table = (const int32_t*)fake(211); },
       DSPARK_EINVAL, "page size not a power of two"},
      {[](DraftCall& d) { d.in.page_size = 16; d.in.max_pages = 8; d.in.block_table = (const int32_t*)fake(211); },
       DSPARK_EINVAL, "page size < 32"},
      {[](DraftCall& d) { d.in.page_size = 64; d.in.max_pages = 8; }, DSPARK_EINVAL, "paged without table"},
      {[](DraftCall& d) { d.in.page_size = 64; d.in.block_table = (const int32_t*)fake(211); }, DSPARK_EINVAL,
       "paged, max_pages 0"},
      {[](DraftCall& d) {
         d.in.page_size = 64; d.in.max_pages = 8; d.in.block_table = (const int32_t*)fake(211);
         d.in.kv_dtype = DSPARK_DT_F32;
       },
       DSPARK_EUNSUPPORTED, "paged f32 caches"},
      {[](DraftCall& d) { d.in.sample_u = (const float*)fake(212); d.in.temperature = 0.f; }, DSPARK_EINVAL,
       "temperature 0"},
      {[](DraftCall& d) { d.in.sample_u = (const float*)fake(212); d.in.temperature = NAN; }, DSPARK_EINVAL,
       "temperature NaN"},
      {[](DraftCall& d) { d.ws = nullptr; }, DSPARK_EINVAL, "workspace NULL"},
      {[](DraftCall& d) { d.ws = (char*)d.ws + 16; }, DSPARK_EINVAL, "workspace misaligned"},
      {[](DraftCall& d) { d.ws_bytes -= 1; }, DSPARK_EWORKSPACE, "workspace short"},
  };
  for (const Mut& mu : muts) {
    DraftCall d = valid_draft(m);
    mu.f(d);
    expect(run(m, d), mu.want, mu.what);
  }
  {
    DraftCall d = valid_draft(m);
    expect(dspark_draft_block(nullptr, &d.in, &d.out, d.ws, d.ws_bytes, nullptr), DSPARK_EINVAL, "model NULL");
    expect(dspark_draft_block(m, nullptr, &d.out, d.ws, d.ws_bytes, nullptr), DSPARK_EINVAL, "in NULL");
    expect(dspark_draft_block(m, &d.in, nullptr, d.ws, d.ws_bytes, nullptr), DSPARK_EINVAL, "out NULL");
    expect(run(layers_only, d), DSPARK_EINVAL, "draft on a layers-only model");
  }
  {
    // the static-scratch form: same validation; sizes past the static array are refused
    DraftCall d = valid_draft(m);
    expect(dspark_draft_block_static(m, &d.in, &d.out, nullptr), DSPARK_EPLANONLY, "static: valid");
    d.in.n_seq = 0;
    expect(dspark_draft_block_static(m, &d.in, &d.out, nullptr), DSPARK_EINVAL, "static: n_seq 0");
    d = valid_draft(m);
    d.in.total_ctx = 1 << 26;
    expect(dspark_draft_block_static(m, &d.in, &d.out, nullptr), DSPARK_EWORKSPACE, "static: too large");
    expect_true(std::strstr(dspark_last_error(), "static scratch") != nullptr, "static: message");
    d = valid_draft(m);
    d.out.conf = nullptr;
    expect(dspark_draft_block_static(m, &d.in, &d.out, nullptr), DSPARK_EINVAL, "static: conf NULL");
    expect(dspark_draft_block_static(nullptr, &d.in, &d.out, nullptr), DSPARK_EINVAL, "static: model NULL");
  }
  expect_true(dspark_workspace_bytes(nullptr, 1, 10) == 0, "workspace query, model NULL");
  expect_true(dspark_workspace_bytes(m, 0, 10) == 0, "workspace query, n_seq 0");
  expect_true(dspark_workspace_bytes(m, 1, -1) == 0, "workspace query, total_ctx < 0");
  expect_true(dspark_workspace_bytes(m, 1, 100) < dspark_workspace_bytes(m, 1, 100000), "workspace grows with ctx");
}

void layer_checks(const dspark_model* m) {
  const size_t ws = dspark_workspace_bytes(m, 1, 300);
  void* w = (void*)fake(400);
  const float* x = (const float*)fake(401);
  float* y = (float*)fake(402);
  const void* kv = fake(403);
  const int32_t* off = (const int32_t*)fake(404);
  expect(dspark_layer_forward(m, 1, 1, 1, x, y, kv, DSPARK_DT_BF16, off, 300, w, ws, nullptr), DSPARK_EPLANONLY,
         "valid layer");
  expect(dspark_layer_forward(nullptr, 0, 1, 1, x, y, kv, DSPARK_DT_BF16, off, 300, w, ws, nullptr), DSPARK_EINVAL,
         "layer: model NULL");
  expect(dspark_layer_forward(m, 2, 1, 1, x, y, kv, DSPARK_DT_BF16, off, 300, w, ws, nullptr), DSPARK_EINVAL,
         "layer out of range");
  expect(dspark_layer_forward(m, -1, 1, 1, x, y, kv, DSPARK_DT_BF16, off, 300, w, ws, nullptr), DSPARK_EINVAL,
         "layer negative");
  expect(dspark_layer_forward(m, 0, 1, 0, x, y, kv, DSPARK_DT_BF16, off, 300, w, ws, nullptr), DSPARK_EINVAL,
         "layer n_seq 0");
  expect(dspark_layer_forward(m, 0, 1, 1, nullptr, y, kv, DSPARK_DT_BF16, off, 300, w, ws, nullptr), DSPARK_EINVAL,
         "layer x_in NULL");
  expect(dspark_layer_forward(m, 0, 1, 1, x, y, kv, DSPARK_DT_Q8_0, off, 300, w, ws, nullptr), DSPARK_EINVAL,
         "layer kv dtype");
  expect(dspark_layer_forward(m, 0, 1, 1, x + 1, y, kv, DSPARK_DT_BF16, off, 300, w, ws, nullptr), DSPARK_EINVAL,
         "layer x_in misaligned");
  expect(dspark_layer_forward(m, 0, 1, 1, x, y, kv, DSPARK_DT_BF16, off, -5, w, ws, nullptr), DSPARK_EINVAL,
         "layer total_ctx < 0");
  expect(dspark_layer_forward(m, 0, 1, 1, x, y, kv, DSPARK_DT_BF16, off, 300, w, ws - 256, nullptr), DSPARK_EWORKSPACE,
         "layer workspace short");
}

void append_checks(const dspark_model* m) {
  const void* kv[2] = {fake(500), fake(501)};
  dspark_append_in a{};
  a.n_new = 7; a.act_dtype = DSPARK_DT_BF16; a.kv_dtype = DSPARK_DT_BF16;
  a.captured = fake(502); a.positions = (const int32_t*)fake(503); a.slot_mapping = (const int64_t*)fake(504);
  a.kv = (void* const*)kv;
  const size_t ws = dspark_append_workspace_bytes(m, 7);
  void* w = (void*)fake(505);
  expect_true(ws > 0, "append workspace bytes");
  expect(dspark_cache_append(m, &a, w, ws, nullptr), DSPARK_EPLANONLY, "valid append");
  expect(dspark_cache_append(m, nullptr, w, ws, nullptr), DSPARK_EINVAL, "append in NULL");
  expect(dspark_cache_append(m, &a, w, ws - 1, nullptr), DSPARK_EWORKSPACE, "append workspace short");
  expect(dspark_cache_append(m, &a, (char*)w + 64, ws, nullptr), DSPARK_EINVAL, "append workspace misaligned");
  dspark_append_in b = a;
  b.n_new = 0;
  expect(dspark_cache_append(m, &b, w, ws, nullptr), DSPARK_EINVAL, "append n_new 0");
  b.n_new = DSPARK_APPEND_MAX + 1;
  expect(dspark_cache_append(m, &b, w, ws, nullptr), DSPARK_EINVAL, "append n_new too large");
  expect_true(dspark_append_workspace_bytes(m, 0) == 0, "append workspace query, n_new 0");
  b = a;
  b.positions = nullptr;
  expect(dspark_cache_append(m, &b, w, ws, nullptr), DSPARK_EINVAL, "append positions NULL");
  b = a;
  b.slot_mapping = (const int64_t*)((const char*)a.slot_mapping + 4);
  expect(dspark_cache_append(m, &b, w, ws, nullptr), DSPARK_EINVAL, "append slot_mapping misaligned");
  b = a;
  b.kv_dtype = DSPARK_DT_MXFP4;
  expect(dspark_cache_append(m, &b, w, ws, nullptr), DSPARK_EINVAL, "append kv dtype");
  const void* kv_bad[2] = {fake(500), nullptr};
  b = a;
  b.kv = (void* const*)kv_bad;
  expect(dspark_cache_append(m, &b, w, ws, nullptr), DSPARK_EINVAL, "append kv[1] NULL");
}

void verify_checks() {
  dspark_verify_in v{};
  v.n_seq = 2; v.block = 7; v.vocab = 1000; v.method = DSPARK_VERIFY_BLOCK; v.temperature = 1.f;
  v.draft = (const int32_t*)fake(600); v.draft_logits = (const float*)fake(601);
  v.target_logits = (const float*)fake(602); v.u = (const float*)fake(603);
  int32_t* len = (int32_t*)fake(604);
  int32_t* tok = (int32_t*)fake(605);
  const size_t ws = dspark_verify_workspace_bytes(2, 7);
  void* w = (void*)fake(606);
  expect_true(ws > 0, "verify workspace bytes");
  expect_true(dspark_verify_workspace_bytes(0, 7) == 0 && dspark_verify_workspace_bytes(2, 64) == 0,
              "verify workspace query, bad sizes");
  expect(dspark_verify(nullptr, len, tok, w, ws, nullptr), DSPARK_EINVAL, "verify in NULL");
  expect(dspark_verify(&v, nullptr, tok, w, ws, nullptr), DSPARK_EINVAL, "verify out NULL");
  expect(dspark_verify(&v, len, tok, w, ws - 4, nullptr), DSPARK_EWORKSPACE, "verify workspace short");
  expect(dspark_verify(&v, len, tok, (char*)w + 8, ws, nullptr), DSPARK_EINVAL, "verify workspace misaligned");
  dspark_verify_in b = v;
  b.block = 0;
  expect(dspark_verify(&b, len, tok, w, ws, nullptr), DSPARK_EINVAL, "verify block 0");
  b = v;
  b.method = 2;
  expect(dspark_verify(&b, len, tok, w, ws, nullptr), DSPARK_EINVAL, "verify method");
  b = v;
  b.temperature = -1.f;
  expect(dspark_verify(&b, len, tok, w, ws, nullptr), DSPARK_EINVAL, "verify temperature");
  b = v;
  b.u = nullptr;
  expect(dspark_verify(&b, len, tok, w, ws, nullptr), DSPARK_EINVAL, "verify u NULL");
}

// Largest k <= block with d[j] == v[j] for all j < k, as the index of the
// first mismatch (block when there is none).
int first_mismatch(const int32_t* d, const int32_t* v, int block) {
  for (int j = 0; j < block; ++j)
    if (d[j] != v[j]) return j;
  return block;
}

void accept_checks() {
  const int cases[][2] = {{3, 1}, {3, 2}, {3, 3}, {3, 4}, {2, 7}};
  for (const auto& cs : cases) {
    const int alpha = cs[0], block = cs[1];
    int n = 1;
    for (int i = 0; i < block; ++i) n *= alpha;
    // every (draft, verifier) pair: n * n sequences in one call
    std::vector<int32_t> d((size_t)n * n * block), v((size_t)n * n * block), out((size_t)n * n);
    for (int a = 0; a < n; ++a)
      for (int b = 0; b < n; ++b)
        for (int j = 0, xa = a, xb = b; j < block; ++j, xa /= alpha, xb /= alpha) {
          d[((size_t)a * n + b) * block + j] = xa % alpha;
          v[((size_t)a * n + b) * block + j] = xb % alpha;
        }
    expect(dspark_accept_len_host(d.data(), v.data(), n * n, block, out.data()), DSPARK_OK, "accept host");
    bool ok = true;
    for (size_t s = 0; s < (size_t)n * n; ++s)
      ok &= out[s] == first_mismatch(&d[s * block], &v[s * block], block);
    expect_true(ok, "accept host brute force");
  }
  int32_t x = 0, o = 0;
  expect(dspark_accept_len_host(nullptr, &x, 1, 1, &o), DSPARK_EINVAL, "accept host NULL");
  expect(dspark_accept_len_host(&x, &x, -1, 1, &o), DSPARK_EINVAL, "accept host n_seq < 0");
  expect(dspark_accept_len_host(&x, &x, 0, 7, &o), DSPARK_OK, "accept host n_seq 0");
  // device form: validation only (NULL pointers, negative sizes; zero sequences enqueue nothing)
  expect(dspark_accept_len(nullptr, (const int32_t*)fake(700), 1, 7, (int32_t*)fake(701), nullptr), DSPARK_EINVAL,
         "accept NULL");
  expect(dspark_accept_len((const int32_t*)fake(700), (const int32_t*)fake(700), 1, -7, (int32_t*)fake(701), nullptr),
         DSPARK_EINVAL, "accept block < 0");
  expect(dspark_accept_len((const int32_t*)fake(700), (const int32_t*)fake(700), 0, 7, (int32_t*)fake(701), nullptr),
         DSPARK_OK, "accept n_seq 0");
}

void dequant_checks(const dspark_model* m) {
  float* out = (float*)fake(800);
  expect(dspark_dequant(m, DSPARK_W_FC, out, nullptr), DSPARK_EPLANONLY, "valid dequant");
  expect(dspark_dequant(m, DSPARK_W_FC_NORM, out, nullptr), DSPARK_EINVAL, "dequant of a vector");
  expect(dspark_dequant(m, DSPARK_LAYER_W(7, DSPARK_L_O), out, nullptr), DSPARK_EINVAL, "dequant layer out of range");
  expect(dspark_dequant(nullptr, DSPARK_W_FC, out, nullptr), DSPARK_EINVAL, "dequant model NULL");
  expect(dspark_dequant(m, DSPARK_W_FC, nullptr, nullptr), DSPARK_EINVAL, "dequant out NULL");
}

}  // namespace

int main(int argc, char** argv) {
  const bool no_device = argc > 1 && std::strcmp(argv[1], "--no-device") == 0;
  config_and_table_checks(no_device);
  dspark_config c = small_cfg();
  std::vector<dspark_weight> w = table(c);
  dspark_model* m = nullptr;
  expect(create(c, w, &m), DSPARK_OK, "plan-only model");
  dspark_config lc = c;
  lc.flags |= DSPARK_CFG_LAYERS_ONLY;
  std::vector<dspark_weight> lw;
  for (const auto& x : w)
    if (x.id >= DSPARK_W_LAYER_BASE) lw.push_back(x);
  dspark_model* lm = nullptr;
  expect(create(lc, lw, &lm), DSPARK_OK, "plan-only layers-only model");
  if (m && lm) {
    draft_checks(m, lm);
    layer_checks(m);
    layer_checks(lm);
    append_checks(m);
    dequant_checks(m);
  }
  verify_checks();
  accept_checks();
  dspark_model_destroy(m);
  dspark_model_destroy(lm);
  expect(dspark_model_destroy(nullptr), DSPARK_OK, "destroy NULL");
  if (g_fail) {
    std::fprintf(stderr, "%d of %d checks failed\n", g_fail, g_checks);
    return 1;
  }
  std::printf("ok %d checks\n", g_checks);
  return 0;
}
