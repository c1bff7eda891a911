"""Algorithmic byte and flop counts of one draft pass (measurement only).

Every weight and every latent-cache row is counted once per pass; re-reads
(W2 once per Markov step, key tiles per query-row group, split-K partials) are
not counted.  Q8_0 = 34 bytes per 32 weights, FP8 = 1 byte per weight + one
fp32 scale per row, MXFP4 = 17 bytes per 32 weights, bf16 = 2, f32 = 4.  W1 contributes only the gathered
rows (n_seq * block rows).  Outputs and intermediate activations are not
counted.
"""
from __future__ import annotations

from typing import Dict

from . import configs as C


def storage_bytes(fmt: str, rows: int, cols: int) -> int:
    if fmt == C.Q8_0:
        return rows * (cols // 32) * 34
    if fmt == C.FP8:
        return rows * cols + 4 * rows
    if fmt == C.MXFP4:
        return rows * (cols // 32) * 17
    if fmt == C.BF16:
        return 2 * rows * cols
    return 4 * rows * cols


def pass_bytes(wl: C.Workload) -> Dict[str, int]:
    """Per-item algorithmic bytes of one pass over all of the workload's blocks."""
    m, f = wl.model, wl.formats
    n_seq, B = wl.n_seq, m.block
    out: Dict[str, int] = {}
    for name in C.tensor_names(m, wl.attn_only):
        shape = C.tensor_shape(m, name)
        fmt = C.tensor_format(f, name)
        rows, cols = (shape[0], shape[1]) if len(shape) == 2 else (shape[0], 1)
        if name == "markov_w1":
            out[name] = storage_bytes(fmt, n_seq * B, cols)
        else:
            out[name] = storage_bytes(fmt, rows, cols)
    kv_e = 4 if f.kv_cache == C.F32 else 2
    out["kv_cache"] = m.n_layers * wl.total_ctx * m.latent * kv_e
    if wl.attn_only:
        out["x_in"] = n_seq * B * m.hidden * 2
    else:
        cap_e = 4 if f.captured == C.F32 else 2
        out["captured"] = n_seq * m.n_captured * B * m.hidden * cap_e
    return out


def total_bytes(wl: C.Workload) -> int:
    return int(sum(pass_bytes(wl).values()))


def lm_head_launch_bytes(wl: C.Workload) -> int:
    """One lm_head launch: the weight stream, the fp32 normed hidden rows in,
    the fp32 logits out."""
    m = wl.model
    M = wl.n_seq * m.block
    w = storage_bytes(wl.formats.lm_head, m.vocab, m.hidden)
    return w + 4 * M * m.hidden + 4 * M * m.vocab


def attention_flops(wl: C.Workload) -> int:
    """2 * rows * (latent + kv_lora) flops per key per layer, rows = heads * block."""
    m = wl.model
    per_key = 2 * m.n_heads * m.block * (m.latent + m.kv_lora)
    keys = wl.total_ctx + wl.n_seq * m.block
    return m.n_layers * per_key * keys


def append_bytes(wl: C.Workload, n_new: int) -> int:
    """One cache append of n_new rows: the fc weights, the kv_a rows of every
    layer's fused q_a / kv_a projection, the captured states read and the
    latent rows written (every layer)."""
    m, f = wl.model, wl.formats
    w = storage_bytes(C.tensor_format(f, "fc"), m.hidden, m.n_captured * m.hidden)
    w += m.n_layers * storage_bytes(C.tensor_format(f, "L0.kv_a"), m.latent, m.hidden)
    cap_e = 4 if f.captured == C.F32 else 2
    kv_e = 4 if f.kv_cache == C.F32 else 2
    return w + n_new * m.n_captured * m.hidden * cap_e + m.n_layers * n_new * m.latent * kv_e
