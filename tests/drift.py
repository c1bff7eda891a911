"""Drift harness: a quantised draft pass against an fp32-weight reference.

The metrics follow huggingface.co "Kimi-K3-DSpark-NVFP4", sections
"Measurement" and "Detail": drift of a weight format against a reference
with unquantised weights, on synthetic captured states ("gauss" N(0,1) and
"heavy" Student-t; the pages' "boot" regime needs a trained drafter).

* ceiling: drift-limited acceptance ceiling, the mean acceptance length of
  the variant's free-running block with the reference's block as verifier;
* greedy: agreement of the argmax per position when both see the
  reference's predecessors (teacher forcing);
* sequential: per-position prefix agreement of the free-running blocks,
  P(tokens 1..k all equal), k = 1..block;
* kl_mean / kl_p99 and tv_coupling (1 - TV) of the per-position softmax
  distributions of the logits (teacher forced);
* hidden_rel: mean over rows of |h - h_ref| / |h_ref| (final-normed hidden);
* conf_r: Pearson correlation of the confidences (teacher forced), and
  flip_rate of the decision conf > 0.5 (the pages give no threshold; 0.5 is
  this harness's reading).

TEST INFRASTRUCTURE (uses the oracle).
"""
from __future__ import annotations

import numpy as np

from oracle import dspark as O


def log_softmax(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, np.float64)
    mx = z.max(axis=-1, keepdims=True)
    return z - mx - np.log(np.exp(z - mx).sum(axis=-1, keepdims=True))


def kl(lp: np.ndarray, lq: np.ndarray) -> np.ndarray:
    """KL(p || q) over the last axis from log-probabilities."""
    p = np.exp(lp)
    return (p * (lp - lq)).sum(axis=-1)


def tv(lp: np.ndarray, lq: np.ndarray) -> np.ndarray:
    return 0.5 * np.abs(np.exp(lp) - np.exp(lq)).sum(axis=-1)


def prefix_agreement(tok: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """P(tokens 1..k all equal) for k = 1..block, over the blocks."""
    eq = np.asarray(tok) == np.asarray(ref)
    return np.cumprod(eq, axis=1).mean(axis=0)


def metrics(ref: dict, free: dict, forced: dict) -> dict:
    """ref: the reference pass; free / forced: the variant free running and
    teacher forced on ref's tokens.  Each: tokens [n, B], logits [n, B, V],
    hidden [n*B, H], conf [n, B]."""
    lp_r, lp_v = log_softmax(ref["logits"]), log_softmax(forced["logits"])
    k = kl(lp_r, lp_v).ravel()
    h, hr = np.asarray(forced["hidden"], np.float64), np.asarray(ref["hidden"], np.float64)
    cr, cv = np.asarray(ref["conf"], np.float64).ravel(), np.asarray(forced["conf"], np.float64).ravel()
    r = float(np.corrcoef(cr, cv)[0, 1]) if cr.std() > 0 and cv.std() > 0 else float("nan")
    return dict(
        ceiling=float(O.accept_len(free["tokens"], ref["tokens"]).mean()),
        greedy=float((np.asarray(forced["tokens"]) == np.asarray(ref["tokens"])).mean()),
        sequential=[float(v) for v in prefix_agreement(free["tokens"], ref["tokens"])],
        kl_mean=float(k.mean()),
        kl_p99=float(np.percentile(k, 99)),
        tv_coupling=float(1.0 - tv(lp_r, lp_v).mean()),
        hidden_rel=float((np.linalg.norm(h - hr, axis=1) / np.linalg.norm(hr, axis=1)).mean()),
        conf_r=r,
        flip_rate=float(((cr > 0.5) != (cv > 0.5)).mean()),
    )


def oracle_pass(wl, stored, inputs, forced=None) -> dict:
    out = O.draft_block(wl, stored, inputs, forced=forced)
    n, B = wl.n_seq, wl.model.block
    return dict(tokens=np.asarray(out["tokens"]), logits=np.asarray(out["logits"]).reshape(n, B, -1),
                hidden=np.asarray(out["hidden"]).reshape(n * B, -1), conf=np.asarray(out["conf"]))


def fmt_row(name: str, m: dict) -> str:
    seq = " ".join(f"{100 * v:5.1f}" for v in m["sequential"])
    return (f"{name:28s} ceiling {m['ceiling']:5.2f}  greedy {100 * m['greedy']:6.2f}%  1-TV "
            f"{100 * m['tv_coupling']:6.2f}%  KL {m['kl_mean']:.5f} (p99 {m['kl_p99']:.5f})  hidden "
            f"{100 * m['hidden_rel']:5.2f}%  conf r {m['conf_r']:.4f} flips {100 * m['flip_rate']:4.1f}%  "
            f"seq [{seq}]")
