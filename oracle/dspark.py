"""Plain float64 CPU oracle of the DSpark draft pass.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import or run anything under oracle/.
It shares no code with the GPU library (mla_block_drafter_amd/).

What is computed (pages on "mla_block_drafter"; sections named per page):

* huggingface.co "Kimi-K3-DSpark-NVFP4", original card, "Model Overview":
  a backbone of 5 dense layers with non-causal attention drafts the whole
  7-token block in one parallel pass; a low-rank Markov head then adds the
  intra-block dependency sequentially; a confidence head scores the draft.
  MLA: one 576-element latent per token (512 compressed + 64 rope), shared
  layout with the target.
* same page, "What is quantized to what": q_a_proj + kv_a_proj_with_mqa fuse
  into one projection; kv_b_proj is used through MLA weight absorption;
  gate/up/down, o_proj, q_b_proj and context_proj (fc) are the quantised set.
* alphaneural.io "kimi-k3-dspark-gguf", "How it works" and "What's needed from
  llama.cpp": q_lora_rank 1536, kv_lora_rank 512, split rope dims
  (qk_nope + qk_rope); the decompression graph (latent -> full K/V through
  kv_b_proj) is the un-absorbed form, used here only as a self-check.
* graysoft.dev "Lucebox Kimi-K3-DSpark Q8_0 GGUF", "Architecture metadata":
  fc consumes five captured target hidden states; Markov rank 256;
  YaRN-16 from a 65,536 window.
* huggingface.co page, "Why acceptance is so sensitive" and "Sampling
  options": acceptance length is the prefix run length of matches; at
  temperature 0 verification is an argmax match.
* huggingface.co page, "Considerations": throughput a / (d + T).

Readings where the pages are silent (each listed in the design notes): fc
output RMSNorm; consecutive-pair RoPE, base 10,000; YaRN NTK-by-parts with
alpha 1, beta 32 and logit scale (0.1 ln s + 1)^2; positions N + i; softmax
scale 1/sqrt(qk_nope + qk_rope); RMSNorm g * x / sqrt(mean x^2 + eps);
Markov term l_i = z_i + W2 W1[t_{i-1}] with t_{-1} = prev_token (-1 = none);
confidence sigmoid(w_h . hf_i + w_m . W1[t_{i-1}] + b); argmax ties go to the
lowest index; the block's own 7 latent rows are appended as keys.

Parity status: each step is pinned by tests/test_oracle_*.py (closed forms,
library routines, brute force, printed values).  The composition of the whole
pass has no worked example on the pages: parity unpinned end to end beyond
the composition of the pinned steps and an independent torch formulation of
the decompressed model.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from . import codecs


# ------------------------------------------------------------- primitives --
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """g * x / sqrt(mean(x^2) + eps) over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return g * x / np.sqrt(ms + eps)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    e = np.exp(s - np.max(s, axis=axis, keepdims=True))
    return e / np.sum(e, axis=axis, keepdims=True)


def rope_frequencies(m) -> np.ndarray:
    """Angular frequency per rope pair k = 0 .. qk_rope/2 - 1.

    Base: theta_k = base^(-2k/d).  With a YaRN factor s > 1 (NTK-by-parts,
    Peng et al. 2023): r_k = L * theta_k / (2 pi) rotations over the original
    window L; gamma_k = clamp((r_k - alpha) / (beta - alpha), 0, 1);
    theta'_k = (1 - gamma_k) * theta_k / s + gamma_k * theta_k.
    """
    d = m.qk_rope
    k = np.arange(d // 2, dtype=np.float64)
    theta = m.rope_theta ** (-2.0 * k / d)
    s = float(m.yarn_factor)
    if s == 1.0:
        return theta
    r = m.yarn_orig_ctx * theta / (2.0 * math.pi)
    alpha, beta = float(m.yarn_beta_slow), float(m.yarn_beta_fast)
    gamma = np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / s + gamma * theta


def yarn_logit_scale(m) -> float:
    """YaRN attention temperature: logits are multiplied by (0.1 ln s + 1)^2."""
    s = float(m.yarn_factor)
    if s <= 1.0:
        return 1.0
    return (0.1 * math.log(s) + 1.0) ** 2


def rope(x: np.ndarray, pos: np.ndarray, freqs: np.ndarray) -> np.ndarray:
    """Rotate consecutive pairs (2k, 2k+1) of the last axis by pos * freqs[k].

    x: [..., d]; pos broadcasts against x[..., 0].
    """
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freqs      # [..., d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x, dtype=np.float64)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def argmax_lowest(v: np.ndarray) -> int:
    """Index of the maximum; ties go to the lowest index."""
    best = np.max(v)
    return int(np.flatnonzero(v == best)[0])


def accept_len(draft: np.ndarray, verifier: np.ndarray) -> np.ndarray:
    """Prefix run length: the largest k with draft[j] == verifier[j] for all j < k."""
    d = np.atleast_2d(np.asarray(draft))
    v = np.atleast_2d(np.asarray(verifier))
    out = np.zeros(d.shape[0], dtype=np.int32)
    for s in range(d.shape[0]):
        k = 0
        while k < d.shape[1] and d[s, k] == v[s, k]:
            k += 1
        out[s] = k
    return out


def throughput(a: float, d: float, T: float) -> float:
    """Accepted tokens per unit time: a / (d + T)."""
    return a / (d + T)


def throughput_ratio(a1: float, a2: float, d1: float, d2: float, T: float) -> float:
    """(a1 / (d1 + T)) / (a2 / (d2 + T)) = (a1 / a2) * (d2 + T) / (d1 + T)."""
    return throughput(a1, d1, T) / throughput(a2, d2, T)


# --------------------------------------------------------------- weights --
class Weights:
    """Decodes stored tensors on demand (no caching, bounded memory)."""

    def __init__(self, stored: Dict[str, object]):
        self.stored = stored

    def __call__(self, name: str) -> np.ndarray:
        return codecs.decode(self.stored[name])

    def matvec_rows(self, name: str, x: np.ndarray, chunk: int = 16384) -> np.ndarray:
        """x @ W^T for a large W, decoding W a band of output rows at a time."""
        st = self.stored[name]
        rows = st.shape[0]
        out = np.empty(x.shape[:-1] + (rows,), dtype=np.float64)
        for r0 in range(0, rows, chunk):
            r1 = min(rows, r0 + chunk)
            out[..., r0:r1] = x @ codecs.decode_rows(st, r0, r1).T
        return out


def _decode_input(arr: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    return codecs.bf16_decode(arr)


# ------------------------------------------------------------ one layer --
def attention_absorbed(m, W: Weights, l: int, a: np.ndarray, cache: np.ndarray,
                       pos0: int, trace: Optional[dict] = None) -> np.ndarray:
    """MLA attention of one sequence's block with absorbed kv_b.

    a: [B, H] input-normed hidden of the block; cache: [N, r + dr] latent rows
    (c_kv after its norm, k_pe after rope, used as stored); pos0 = N.
    Returns o_cat [B, nh * dv] (before o_proj).
    """
    p = f"L{l}."
    B = a.shape[0]
    r, dr, dn, dv, nh = m.kv_lora, m.qk_rope, m.qk_nope, m.v_head, m.n_heads
    freqs = rope_frequencies(m)
    pos = pos0 + np.arange(B)
    # fused q_a / kv_a projection, then their norms and the rope of k_pe
    cq = rmsnorm(a @ W(p + "q_a").T, W(p + "q_a_norm"), m.rms_eps)
    kv = a @ W(p + "kv_a").T
    c = rmsnorm(kv[:, :r], W(p + "kv_a_norm"), m.rms_eps)
    kp = rope(kv[:, r:], pos, freqs)
    # q_b and rope of the query's rope part
    q = (cq @ W(p + "q_b").T).reshape(B, nh, dn + dr)
    qn = q[:, :, :dn]
    qp = rope(q[:, :, dn:], pos[:, None], freqs)
    # absorption: q_lat[i, h] = W_UK[h]^T qn[i, h]
    wkvb = W(p + "kv_b").reshape(nh, dn + dv, r)
    w_uk, w_uv = wkvb[:, :dn, :], wkvb[:, dn:, :]
    q_lat = np.einsum("ihd,hdr->ihr", qn, w_uk)
    # keys: the cache, then the block's own latent rows (non-causal, no mask)
    K = np.concatenate([cache, np.concatenate([c, kp], axis=1)], axis=0)
    tau = yarn_logit_scale(m) / math.sqrt(dn + dr)
    s = tau * (np.einsum("ihr,jr->ihj", q_lat, K[:, :r]) +
               np.einsum("ihe,je->ihj", qp, K[:, r:]))
    pr = softmax(s, axis=-1)
    o_lat = np.einsum("ihj,jr->ihr", pr, K[:, :r])
    o = np.einsum("ihr,hvr->ihv", o_lat, w_uv)
    if trace is not None:
        trace.update(cq=cq, kv=kv, c=c, kp=kp, q=q, qp=qp, q_lat=q_lat, o_lat=o_lat, o=o)
    return o.reshape(B, nh * dv)


def attention_decompressed(m, W: Weights, l: int, a: np.ndarray, cache: np.ndarray,
                           pos0: int) -> np.ndarray:
    """Self-check form: decompress every latent row into per-head K/V through
    kv_b (the rope key is shared by all heads) and run standard attention."""
    p = f"L{l}."
    B = a.shape[0]
    r, dr, dn, dv, nh = m.kv_lora, m.qk_rope, m.qk_nope, m.v_head, m.n_heads
    freqs = rope_frequencies(m)
    pos = pos0 + np.arange(B)
    cq = rmsnorm(a @ W(p + "q_a").T, W(p + "q_a_norm"), m.rms_eps)
    kv = a @ W(p + "kv_a").T
    c = rmsnorm(kv[:, :r], W(p + "kv_a_norm"), m.rms_eps)
    kp = rope(kv[:, r:], pos, freqs)
    q = (cq @ W(p + "q_b").T).reshape(B, nh, dn + dr)
    q = np.concatenate([q[:, :, :dn], rope(q[:, :, dn:], pos[:, None], freqs)], axis=2)
    lat = np.concatenate([cache, np.concatenate([c, kp], axis=1)], axis=0)
    kvfull = (lat[:, :r] @ W(p + "kv_b").T).reshape(-1, nh, dn + dv)   # [J, nh, dn+dv]
    k_h = np.concatenate([kvfull[:, :, :dn],
                          np.broadcast_to(lat[:, None, r:], (lat.shape[0], nh, dr))], axis=2)
    v_h = kvfull[:, :, dn:]
    tau = yarn_logit_scale(m) / math.sqrt(dn + dr)
    s = tau * np.einsum("ihe,jhe->ihj", q, k_h)
    pr = softmax(s, axis=-1)
    o = np.einsum("ihj,jhv->ihv", pr, v_h)
    return o.reshape(B, nh * dv)


def mlp(m, W: Weights, l: int, x: np.ndarray) -> np.ndarray:
    """SwiGLU: (silu(h W_g^T) * (h W_u^T)) W_d^T with h = RMSNorm(x; g_post)."""
    p = f"L{l}."
    h = rmsnorm(x, W(p + "post_norm"), m.rms_eps)
    g = silu(h @ W(p + "gate").T) * (h @ W(p + "up").T)
    return g @ W(p + "down").T


def layer(m, W: Weights, l: int, x: np.ndarray, caches, kv_off, attn_only=False,
          decompressed=False, trace: Optional[dict] = None) -> np.ndarray:
    """One pre-norm decoder layer over all sequences' blocks.

    x: [n_seq * B, H] residual stream; caches[l]: [total_ctx, latent].
    """
    B = m.block
    n_seq = len(kv_off) - 1
    a = rmsnorm(x, W(f"L{l}.in_norm"), m.rms_eps)
    o_cat = np.empty((x.shape[0], m.n_heads * m.v_head))
    for s in range(n_seq):
        cache = caches[l][kv_off[s]:kv_off[s + 1]]
        rows = slice(s * B, (s + 1) * B)
        n_ctx = int(kv_off[s + 1] - kv_off[s])
        if decompressed:
            o_cat[rows] = attention_decompressed(m, W, l, a[rows], cache, n_ctx)
        else:
            tr = None if trace is None else trace.setdefault(s, {})
            o_cat[rows] = attention_absorbed(m, W, l, a[rows], cache, n_ctx, trace=tr)
    x = x + o_cat @ W(f"L{l}.o").T
    if attn_only:
        return x
    return x + mlp(m, W, l, x)


# ---------------------------------------------------------- paged caches --
def gather_pages(pool: np.ndarray, table: np.ndarray, lengths, page_size: int) -> np.ndarray:
    """Packed rows [sum(lengths), latent] of a paged cache (huggingface.co
    "Kimi-K3-DSpark-NVFP4", original card, "Model Overview": the draft's
    latent pages share the target's page format).  Token j of sequence s is
    row j mod page_size of page table[s, j div page_size]; sequences follow
    each other in order, as in the packed layout."""
    rows = []
    for s, n in enumerate(lengths):
        for j in range(int(n)):
            rows.append(pool[table[s, j // page_size], j % page_size])
    if not rows:
        return pool.reshape(-1, pool.shape[-1])[:0].copy()
    return np.stack(rows)


# ---------------------------------------------------------- cache append --
def cache_rows(m, W: Weights, captured: np.ndarray, positions, cap_fmt: str) -> np.ndarray:
    """Latent cache rows of newly verified positions, one per layer.

    Pages: huggingface.co "Kimi-K3-DSpark-NVFP4", original card, "Model
    Overview" (one 576-element latent per token, the target's page format);
    graysoft.dev "Lucebox Kimi-K3-DSpark Q8_0 GGUF", "Architecture metadata"
    (fc consumes the captured target states).  Reading where the pages stop:
    layer l's row at a position is its kv_a path applied to that position's
    fc output x = RMSNorm(concat(captured) W_fc^T; g_fc):
    [RMSNorm((RMSNorm(x; in_norm_l) W_kva^T)[:r]; g_kva) | RoPE(...[r:], pos)].
    captured: [n, n_captured, H] (storage format cap_fmt); returns [L, n, r + dr].
    """
    n = len(positions)
    cap = _decode_input(captured, cap_fmt).reshape(n, m.n_captured * m.hidden)
    x = rmsnorm(cap @ W("fc").T, W("fc_norm"), m.rms_eps)
    pos = np.asarray(positions, dtype=np.int64)
    freqs = rope_frequencies(m)
    r = m.kv_lora
    out = np.empty((m.n_layers, n, r + m.qk_rope))
    for l in range(m.n_layers):
        a = rmsnorm(x, W(f"L{l}.in_norm"), m.rms_eps)
        kv = a @ W(f"L{l}.kv_a").T
        out[l, :, :r] = rmsnorm(kv[:, :r], W(f"L{l}.kv_a_norm"), m.rms_eps)
        out[l, :, r:] = rope(kv[:, r:], pos, freqs)
    return out


# ----------------------------------------------------------- whole pass --
def backbone(m, W: Weights, inputs, kv_fmt: str, cap_fmt: str, decompressed=False,
             keep_layers=False):
    """fc over the captured states, then the decoder layers; returns hf and z."""
    n_seq = len(inputs.kv_offsets) - 1
    B, H = m.block, m.hidden
    cap = _decode_input(inputs.captured, cap_fmt).reshape(n_seq, m.n_captured, B, H)
    # concat the captured states along features, in capture order
    X = cap.transpose(0, 2, 1, 3).reshape(n_seq * B, m.n_captured * H)
    x = rmsnorm(X @ W("fc").T, W("fc_norm"), m.rms_eps)
    caches = [_decode_input(c, kv_fmt) for c in inputs.caches]
    per_layer = [x] if keep_layers else None
    for l in range(m.n_layers):
        x = layer(m, W, l, x, caches, inputs.kv_offsets, decompressed=decompressed)
        if keep_layers:
            per_layer.append(x)
    hf = rmsnorm(x, W("final_norm"), m.rms_eps)
    z = W.matvec_rows("lm_head", hf)
    return hf, z, per_layer


def gumbel(u: np.ndarray) -> np.ndarray:
    """Standard Gumbel variates -ln(-ln u) of uniforms u in (0, 1)."""
    return -np.log(-np.log(np.asarray(u, dtype=np.float64)))


def markov_rollout(m, W: Weights, hf: np.ndarray, z: np.ndarray, prev_token,
                   forced: Optional[np.ndarray] = None, sample_u: Optional[np.ndarray] = None,
                   temperature: float = 1.0):
    """Sequential Markov head and confidence over each sequence's block.

    For i = 0..B-1: u = W1[t_{i-1}] (zero when t_{i-1} = -1), l_i = z_i + W2 u,
    t_i = argmax l_i (lowest index on ties), conf_i = sigmoid(w_h . hf_i +
    w_m . u + b).  t_{-1} = prev_token; with `forced`, t_{i-1} for i >= 1 is
    forced[s, i-1] instead of the drafted token (teacher-forced rollout).

    Probabilistic drafting (huggingface.co "Kimi-K3-DSpark-NVFP4", "Sampling
    options": the draft sampled from its own distribution): with `sample_u`
    ([n_seq, B, V] uniforms in (0, 1), an input), t_i is a draw from
    softmax(l_i / temperature) by the Gumbel-max rule, t_i = argmax_v
    (l_i[v] / temperature - ln(-ln u[s, i, v])).  The logits returned stay l_i.
    """
    B, H, V = m.block, m.hidden, m.vocab
    n_seq = len(prev_token)
    w1, w2 = W("markov_w1"), W("markov_w2")
    cw, cb = W("conf_w"), W("conf_b")
    w_h, w_m = cw[:H], cw[H:]
    tokens = np.zeros((n_seq, B), dtype=np.int64)
    conf = np.zeros((n_seq, B))
    logits = np.zeros((n_seq, B, V))
    for s in range(n_seq):
        t_prev = int(prev_token[s])
        for i in range(B):
            if i > 0:
                t_prev = int(forced[s, i - 1]) if forced is not None else int(tokens[s, i - 1])
            u = w1[t_prev] if t_prev >= 0 else np.zeros(m.markov_rank)
            li = z[s * B + i] + w2 @ u
            if sample_u is None:
                tokens[s, i] = argmax_lowest(li)
            else:
                tokens[s, i] = argmax_lowest(li / temperature + gumbel(sample_u[s, i]))
            logits[s, i] = li
            conf[s, i] = sigmoid(w_h @ hf[s * B + i] + w_m @ u + cb[0])
    return tokens, conf, logits


def draft_block(wl, stored, inputs, forced: Optional[np.ndarray] = None,
                decompressed: bool = False, keep_layers: bool = False,
                sample_u: Optional[np.ndarray] = None, temperature: float = 1.0) -> dict:
    """The whole draft pass for every sequence of the workload."""
    m = wl.model
    W = Weights(stored)
    hf, z, per_layer = backbone(m, W, inputs, wl.formats.kv_cache, wl.formats.captured,
                                decompressed=decompressed, keep_layers=keep_layers)
    tokens, conf, logits = markov_rollout(m, W, hf, z, inputs.prev_token, forced, sample_u, temperature)
    out = dict(tokens=tokens, conf=conf, logits=logits, z=z, hidden=hf)
    if keep_layers:
        out["layers"] = per_layer
    return out


def attn_layer_unit(wl, stored, inputs, decompressed: bool = False) -> np.ndarray:
    """The single-layer unit: x + o_proj(MLA(RMSNorm(x))) for layer 0."""
    m = wl.model
    W = Weights(stored)
    caches = [_decode_input(c, wl.formats.kv_cache) for c in inputs.caches]
    x = np.asarray(inputs.x_in, dtype=np.float64)
    return layer(m, W, 0, x, caches, inputs.kv_offsets, attn_only=True,
                 decompressed=decompressed)
