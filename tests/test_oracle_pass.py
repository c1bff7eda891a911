"""Pins of the oracle's layer / head / whole pass.

* absorbed MLA equals the decompressed form (huggingface.co card, "What is
  quantized to what": kv_b used through absorption; alphaneural.io card,
  "What's needed from llama.cpp": the decompression graph) in float64;
* an independent torch formulation (library RMSNorm, linear, silu,
  scaled_dot_product_attention; RoPE as complex multiplication) of the
  decompressed model agrees with the oracle end to end;
* special cases: uniform attention, permutation invariance (non-causal),
  identity layer, fc with one captured state, Markov reductions (parallel
  argmax; pure bigram walk brute-forced with the explicit V x V matrix),
  confidence closed forms.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import codecs, dspark as O
from synth import configs as C, gen


def _wl(model=None, formats=C.ALL_F32, lens=(40,), **kw):
    model = model or C.small_model(n_layers=1)
    return C.Workload("t", model, formats, seed=4242, kv_lens=tuple(lens), fixture_gains=True, **kw)


def _zero(st, name):
    s = st[name]
    st[name] = gen.Stored("f32", s.shape, np.zeros(s.shape, np.float32))


def _set(st, name, arr):
    st[name] = gen.Stored("f32", arr.shape, np.asarray(arr, np.float32))


# ------------------------------------------------------- absorbed form ----
@pytest.mark.parametrize("yarn", [1.0, 4.0])
def test_absorbed_equals_decompressed(yarn):
    wl = _wl(C.small_model(yarn_factor=yarn, yarn_orig_ctx=16), lens=(0, 5, 37))
    st, inp = gen.make_weights(wl), gen.make_inputs(wl)
    a = O.draft_block(wl, st, inp)
    b = O.draft_block(wl, st, inp, decompressed=True)
    np.testing.assert_allclose(a["hidden"], b["hidden"], rtol=0, atol=1e-11)
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=0, atol=1e-11)
    np.testing.assert_array_equal(a["tokens"], b["tokens"])


# ------------------------------------------- independent torch model ------
def _t(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64))


def _torch_rope(x, pos, m):
    d = x.shape[-1]
    inv = _t(m.rope_theta ** (-np.arange(0, d, 2) / d))
    if m.yarn_factor != 1.0:
        wavelen = 2 * math.pi / inv
        ramp = ((m.yarn_orig_ctx / wavelen) - m.yarn_beta_slow) / (m.yarn_beta_fast - m.yarn_beta_slow)
        keep = ramp.clamp(0, 1)
        inv = inv * keep + (inv / m.yarn_factor) * (1 - keep)
    rot = torch.polar(torch.ones_like(inv), _t(pos)[..., None] * inv)
    xc = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
    while rot.dim() < xc.dim():
        rot = rot.unsqueeze(-2)
    return torch.view_as_real(xc * rot).reshape(x.shape)


def _torch_pass(wl, st, inp):
    m = wl.model
    Wt = lambda n: _t(codecs.decode(st[n]))
    H, B, nh = m.hidden, m.block, m.n_heads
    r, dr, dn, dv = m.kv_lora, m.qk_rope, m.qk_nope, m.v_head
    msc = (0.1 * math.log(m.yarn_factor) + 1) ** 2 if m.yarn_factor > 1 else 1.0
    rms = lambda x, n: F.rms_norm(x, (x.shape[-1],), Wt(n), eps=m.rms_eps)
    cap = _t(inp.captured.astype(np.float32) if wl.formats.captured == "f32"
             else codecs.bf16_decode(inp.captured))
    xs = []
    for s in range(wl.n_seq):
        X = torch.cat([cap[s, k] for k in range(m.n_captured)], dim=-1)
        xs.append(rms(F.linear(X, Wt("fc")), "fc_norm"))
    x = torch.cat(xs)
    caches = [_t(c.astype(np.float32) if wl.formats.kv_cache == "f32" else codecs.bf16_decode(c))
              for c in inp.caches]
    for l in range(m.n_layers):
        p = f"L{l}."
        a = rms(x, p + "in_norm")
        outs = []
        for s in range(wl.n_seq):
            o0, o1 = int(inp.kv_offsets[s]), int(inp.kv_offsets[s + 1])
            pos = torch.arange(B, dtype=torch.float64) + (o1 - o0)
            ab = a[s * B:(s + 1) * B]
            cq = rms(F.linear(ab, Wt(p + "q_a")), p + "q_a_norm")
            kv = F.linear(ab, Wt(p + "kv_a"))
            c = rms(kv[:, :r], p + "kv_a_norm")
            kp = _torch_rope(kv[:, r:], pos, m)
            q = F.linear(cq, Wt(p + "q_b")).view(B, nh, dn + dr)
            q = torch.cat([q[..., :dn], _torch_rope(q[..., dn:], pos[:, None].expand(B, nh), m)], -1)
            lat = torch.cat([caches[l][o0:o1], torch.cat([c, kp], -1)])
            kvf = F.linear(lat[:, :r], Wt(p + "kv_b")).view(-1, nh, dn + dv)
            k = torch.cat([kvf[..., :dn], lat[:, None, r:].expand(-1, nh, dr)], -1)
            v = kvf[..., dn:]
            o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1).contiguous(),
                                               v.transpose(0, 1).contiguous(),
                                               scale=msc / math.sqrt(dn + dr))
            outs.append(o.transpose(0, 1).reshape(B, nh * dv))
        x = x + F.linear(torch.cat(outs), Wt(p + "o"))
        h = rms(x, p + "post_norm")
        x = x + F.linear(F.silu(F.linear(h, Wt(p + "gate"))) * F.linear(h, Wt(p + "up")), Wt(p + "down"))
    hf = rms(x, "final_norm")
    z = F.linear(hf, Wt("lm_head"))
    w1, w2, cw, cb = Wt("markov_w1"), Wt("markov_w2"), Wt("conf_w"), Wt("conf_b")
    toks = torch.zeros(wl.n_seq, B, dtype=torch.long)
    conf = torch.zeros(wl.n_seq, B, dtype=torch.float64)
    for s in range(wl.n_seq):
        prev = int(inp.prev_token[s])
        for i in range(B):
            u = w1[prev] if prev >= 0 else torch.zeros(m.markov_rank, dtype=torch.float64)
            li = z[s * B + i] + w2 @ u
            toks[s, i] = torch.argmax(li)
            conf[s, i] = torch.sigmoid(torch.dot(cw, torch.cat([hf[s * B + i], u])) + cb[0])
            prev = int(toks[s, i])
    return hf.numpy(), toks.numpy(), conf.numpy()


@pytest.mark.parametrize("which", ["tiny", "small_yarn_2seq"])
def test_whole_pass_vs_independent_torch_model(which):
    if which == "tiny":
        wl = C.CFG1.replace(fixture_gains=True)
    else:
        wl = _wl(C.small_model(n_layers=2, yarn_factor=4.0, yarn_orig_ctx=16), lens=(3, 29))
    st, inp = gen.make_weights(wl), gen.make_inputs(wl)
    out = O.draft_block(wl, st, inp)
    hf, toks, conf = _torch_pass(wl, st, inp)
    np.testing.assert_allclose(out["hidden"], hf, rtol=0, atol=1e-10)
    np.testing.assert_array_equal(out["tokens"], toks)
    np.testing.assert_allclose(out["conf"], conf, rtol=1e-12)


# ------------------------------------------------------- special cases ----
def test_uniform_attention_and_permutation_invariance():
    wl = _wl(lens=(23,))
    st, inp = gen.make_weights(wl), gen.make_inputs(wl)
    m = wl.model
    W = O.Weights(st)
    cache = O._decode_input(inp.caches[0], "f32")
    a = np.random.default_rng(0).standard_normal((7, m.hidden))
    tr = {}
    base = O.attention_absorbed(m, W, 0, a, cache, 23, trace=tr)
    perm = np.random.default_rng(1).permutation(23)
    np.testing.assert_allclose(O.attention_absorbed(m, W, 0, a, cache[perm], 23), base,
                               rtol=0, atol=1e-12)
    # q_b = 0 makes every score 0 (q_nope and q_rope vanish): the latent output
    # is the plain mean of all value rows (cache rows and the block's rows)
    st2 = dict(st)
    _zero(st2, "L0.q_b")
    tr2 = {}
    O.attention_absorbed(m, O.Weights(st2), 0, a, cache, 23, trace=tr2)
    vals = np.concatenate([cache[:, :m.kv_lora], tr2["c"]], axis=0)
    np.testing.assert_allclose(tr2["o_lat"], np.broadcast_to(vals.mean(0), tr2["o_lat"].shape),
                               atol=1e-12)


def test_sharp_attention_selects_one_key():
    """A single cache row aligned with the query dominates: the latent output
    equals that row (softmax of a very large gap is one-hot)."""
    wl = _wl(lens=(9,))
    st, inp = gen.make_weights(wl), gen.make_inputs(wl)
    m = wl.model
    W = O.Weights(st)
    a = np.random.default_rng(3).standard_normal((7, m.hidden))
    tr = {}
    O.attention_absorbed(m, W, 0, a, np.zeros((0, m.latent)), 0, trace=tr)
    cache = np.zeros((9, m.latent))
    # key 4 = 1e4 * q_lat of (token 0, head 0) direction -> dominates for that row
    cache[4, :m.kv_lora] = tr["q_lat"][0, 0] * (1e4 / np.linalg.norm(tr["q_lat"][0, 0]) ** 2) * 50
    tr2 = {}
    O.attention_absorbed(m, W, 0, a, cache, 9, trace=tr2)
    np.testing.assert_allclose(tr2["o_lat"][0, 0], cache[4, :m.kv_lora], rtol=1e-9)


def test_identity_layer_and_fc_special_case():
    wl = _wl(C.small_model(n_layers=2))
    st, inp = gen.make_weights(wl), gen.make_inputs(wl)
    for l in range(2):
        _zero(st, f"L{l}.o")
        _zero(st, f"L{l}.down")
    out = O.draft_block(wl, st, inp, keep_layers=True)
    for x in out["layers"][1:]:
        np.testing.assert_array_equal(x, out["layers"][0])
    # only captured state k nonzero -> x = RMSNorm(S_k W_fc[:, kH:(k+1)H]^T)
    m = wl.model
    H = m.hidden
    cap = inp.captured.copy()
    k = 3
    cap[:, [j for j in range(5) if j != k]] = 0
    inp.captured = cap
    out = O.draft_block(wl, st, inp, keep_layers=True)
    Wfc = codecs.decode(st["fc"])
    want = O.rmsnorm(cap[0, k].astype(np.float64) @ Wfc[:, k * H:(k + 1) * H].T,
                     codecs.decode(st["fc_norm"]), m.rms_eps)
    np.testing.assert_allclose(out["layers"][0], want, rtol=1e-12, atol=1e-14)


def test_markov_reductions():
    m = C.TINY
    wl = C.CFG1.replace(fixture_gains=True)
    st, inp = gen.make_weights(wl), gen.make_inputs(wl)
    # (1) W2 = 0: every position is the plain argmax of its backbone logits
    st0 = dict(st)
    _zero(st0, "markov_w2")
    out = O.draft_block(wl, st0, inp)
    np.testing.assert_array_equal(out["tokens"][0], np.argmax(out["z"], axis=1))
    # (2) lm_head = 0: a pure bigram walk t_i = argmax_v (W2 W1^T)[v, t_{i-1}]
    wl2 = C.CFG1.replace(markov_dominant=True)
    st2, inp2 = gen.make_weights(wl2), gen.make_inputs(wl2)
    out2 = O.draft_block(wl2, st2, inp2)
    M = codecs.decode(st2["markov_w2"]) @ codecs.decode(st2["markov_w1"]).T   # [V, V]
    t = int(inp2.prev_token[0])
    walk = []
    for _ in range(7):
        col = M[:, t]
        t = int(np.flatnonzero(col == col.max())[0])
        walk.append(t)
    np.testing.assert_array_equal(out2["tokens"][0], walk)
    assert len(set(walk)) > 1
    # (3) prev_token = -1 drops the term at position 0
    inp2.prev_token[:] = -1
    out3 = O.draft_block(wl2, st2, inp2)
    assert out3["tokens"][0, 0] == 0          # all-zero logits: lowest index wins
    # (4) teacher forcing: position i uses forced[i-1] as its predecessor
    forced = np.array([[5, 99, 4000, 7, 7, 1, 2]])
    out4 = O.draft_block(wl, st, inp, forced=forced)
    w1, w2 = codecs.decode(st["markov_w1"]), codecs.decode(st["markov_w2"])
    for i in range(1, 7):
        np.testing.assert_allclose(out4["logits"][0, i], out4["z"][i] + w2 @ w1[forced[0, i - 1]])


def test_confidence_closed_forms():
    wl = C.CFG1.replace(fixture_gains=True)
    st, inp = gen.make_weights(wl), gen.make_inputs(wl)
    b = float(codecs.decode(st["conf_b"])[0])
    st0 = dict(st)
    _zero(st0, "conf_w")
    out = O.draft_block(wl, st0, inp)
    np.testing.assert_allclose(out["conf"], 1 / (1 + math.exp(-b)))
    m = wl.model
    cw = codecs.decode(st["conf_w"]).copy()
    cw[m.hidden:] = 0
    st1 = dict(st)
    _set(st1, "conf_w", cw)
    out = O.draft_block(wl, st1, inp)
    np.testing.assert_allclose(out["conf"][0], O.sigmoid(out["hidden"] @ cw[:m.hidden] + b), rtol=1e-13)
