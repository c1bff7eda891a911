"""Verification of a drafted block under sampling: the plain CPU reference.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import or run anything under oracle/.

Pages: huggingface.co "Kimi-K3-DSpark-NVFP4", "Sampling options": the draft
may be sampled from its own distribution (draft_sample_method
"probabilistic"), and the block may be verified "as a unit rather than
token by token" (rejection_sample_method "block"); under greedy decoding
verification is an argmax match ("Why acceptance is so sensitive").  The
pages name the two verifiers but define neither; this module writes out:

* token: the standard rejection rule of speculative sampling, position by
  position: accept x_i when r_i < min(1, p_i(x_i) / q_i(x_i)); at the first
  rejection emit a draw from the normalised residual max(p_i - q_i, 0);
  with the whole block accepted emit a draw from p_B;
* block: the block rule (verification of the block as a unit): prefix
  weights w_0 = 1, w_k = min(w_{k-1} p_{k-1}(x_{k-1}) / q_{k-1}(x_{k-1}), 1);
  residuals res_k = max(w_k p_k - q_k, 0) with mass S_k; acceptance
  probabilities h_k = S_k / (S_k + 1 - w_k) (k < B) and h_B = w_B; the
  accepted length is the largest k with r_k < h_k (k = 0 always qualifies);
  then a draw from res_k / S_k (or from p_B when k = B).

Both must leave the target's distribution unchanged; tests pin that by
sampling (distribution preservation) and with exact special cases.  Draws
from a distribution use the inverse CDF: the lowest index whose cumulative
mass exceeds u times the total.
"""
from __future__ import annotations

import numpy as np


def softmax_t(logits: np.ndarray, temperature: float) -> np.ndarray:
    z = np.asarray(logits, dtype=np.float64) / temperature
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def inverse_cdf(weights: np.ndarray, u: float) -> int:
    """Lowest index v with sum(weights[:v+1]) > u * sum(weights)."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    return int(min(np.searchsorted(c, u * c[-1], side="right"), len(c) - 1))


def token_verify(draft, q: np.ndarray, p: np.ndarray, r, u_res: float):
    """draft [B]; q [B, V] draft distributions; p [B + 1, V] target
    distributions; r [B] acceptance uniforms.  Returns (accepted, next token)."""
    B = len(draft)
    for i in range(B):
        x = int(draft[i])
        if r[i] < min(1.0, p[i, x] / q[i, x]):
            continue
        return i, inverse_cdf(np.maximum(p[i] - q[i], 0.0), u_res)
    return B, inverse_cdf(p[B], u_res)


def block_weights(draft, q: np.ndarray, p: np.ndarray) -> np.ndarray:
    """w_0 .. w_B of the block rule."""
    B = len(draft)
    w = np.ones(B + 1)
    for k in range(1, B + 1):
        x = int(draft[k - 1])
        w[k] = min(w[k - 1] * p[k - 1, x] / q[k - 1, x], 1.0)
    return w


def block_verify(draft, q: np.ndarray, p: np.ndarray, r, u_res: float):
    """As token_verify, with the block rule; r [B]: r[k - 1] decides k."""
    B = len(draft)
    w = block_weights(draft, q, p)
    tau = 0
    for k in range(1, B + 1):
        if k < B:
            S = np.maximum(w[k] * p[k] - q[k], 0.0).sum()
            h = S / (S + 1.0 - w[k]) if S + 1.0 - w[k] > 0 else 1.0
        else:
            h = w[B]
        if r[k - 1] < h:
            tau = k
    if tau == B:
        return B, inverse_cdf(p[B], u_res)
    res = np.maximum(w[tau] * p[tau] - q[tau], 0.0)
    return tau, inverse_cdf(res, u_res)
