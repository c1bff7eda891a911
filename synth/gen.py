"""Seeded synthetic weights and inputs for the DSpark draft pass.

Both sides of every parity check (the CPU oracle and the GPU library) consume
the exact stored values produced here.  Nothing in this module computes any
step of the draft pass; it draws random numbers and stores them in the
weight formats the pages name (BF16, Q8_0 with 32-element blocks and an fp16
scale, FP8 E4M3 with per-output-channel fp32 scales).  The stored encodings are
produced once on the host; the device only decodes them.

Random streams: tensor i of workload seed s draws element chunk j (2**22
elements, row-major flat order) from
``default_rng(SeedSequence(s, spawn_key=(i, j)))``, so the values do not depend
on the number of threads used to draw them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

from . import configs as C

CHUNK = 1 << 22
_N_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _pool():
    return ThreadPoolExecutor(max_workers=_N_THREADS)


def _fill(out_flat: np.ndarray, seed: int, idx: int, kind: str, a: float, b: float) -> None:
    n = out_flat.size
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(j):
        lo, hi = j * CHUNK, min(n, (j + 1) * CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(idx, j)))
        if kind == "normal":
            v = rng.standard_normal(hi - lo, dtype=np.float32)
            if a != 1.0:
                v *= np.float32(a)
        elif kind == "uniform":
            v = rng.random(hi - lo, dtype=np.float32) * np.float32(b - a) + np.float32(a)
        else:
            raise ValueError(kind)
        out_flat[lo:hi] = v

    if nchunks == 1:
        work(0)
    else:
        with _pool() as ex:
            list(ex.map(work, range(nchunks)))


def normal(shape, seed: int, idx: int, std: float = 1.0) -> np.ndarray:
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    _fill(out, seed, idx, "normal", std, 0.0)
    return out.reshape(shape)


def student_t(shape, seed: int, idx: int, df: float) -> np.ndarray:
    """Student-t draws with `df` degrees of freedom scaled to unit variance."""
    n = int(np.prod(shape))
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(idx, 0)))
    v = rng.standard_t(df, size=n) * np.sqrt((df - 2.0) / df)
    return v.astype(np.float32).reshape(shape)


def uniform(shape, seed: int, idx: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    _fill(out, seed, idx, "uniform", lo, hi)
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# storage encoders (host-side weight conversion; the device only decodes)
# ----------------------------------------------------------------------------

def _bf16_chunk(u: np.ndarray) -> np.ndarray:
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if u.size <= CHUNK:
        return _bf16_chunk(u)
    flat = u.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)

    def work(j):
        lo, hi = j * CHUNK, min(flat.size, (j + 1) * CHUNK)
        out[lo:hi] = _bf16_chunk(flat[lo:hi])

    with _pool() as ex:
        list(ex.map(work, range((flat.size + CHUNK - 1) // CHUNK)))
    return out.reshape(u.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_q8_0(w: np.ndarray) -> np.ndarray:
    """[rows, K] float32 -> [rows, K/32*34] uint8 of 34-byte blocks (fp16 d, 32 x int8)."""
    rows, K = w.shape
    if K % 32:
        raise ValueError("Q8_0 needs K % 32 == 0")
    nb = K // 32
    out = np.empty((rows, nb, 34), dtype=np.uint8)

    def work(r0):
        r1 = min(rows, r0 + 2048)
        x = w[r0:r1].reshape(r1 - r0, nb, 32).astype(np.float32, copy=False)
        amax = np.abs(x).max(axis=2)
        d = amax / np.float32(127.0)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = x / d[..., None]
        q = np.where(d[..., None] > 0, q, np.float32(0))
        q = np.sign(q) * np.floor(np.abs(q) + np.float32(0.5))  # half away from zero
        q = np.clip(q, -127, 127).astype(np.int8)
        out[r0:r1, :, 0:2] = d.astype(np.float16).view(np.uint8).reshape(r1 - r0, nb, 2)
        out[r0:r1, :, 2:] = q.view(np.uint8)

    with _pool() as ex:
        list(ex.map(work, range(0, rows, 2048)))
    return out.reshape(rows, nb * 34)


def to_fp8_e4m3_per_channel(w: np.ndarray):
    """[rows, K] float32 -> (uint8 codes [rows, K], float32 scales [rows]).

    scale_n = amax_n / 448 (1 for an all-zero row); code = saturating RNE E4M3FN
    of w / scale_n, using torch's float8_e4m3fn conversion.
    """
    import torch
    rows, K = w.shape
    amax = np.abs(w).max(axis=1)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = np.empty((rows, K), dtype=np.uint8)

    def work(r0):
        r1 = min(rows, r0 + 2048)
        v = np.clip(w[r0:r1] / s[r0:r1, None], -448.0, 448.0).astype(np.float32)
        t = torch.from_numpy(v).to(torch.float8_e4m3fn)
        codes[r0:r1] = t.view(torch.uint8).numpy()

    with _pool() as ex:
        list(ex.map(work, range(0, rows, 2048)))
    return codes, s


_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def to_mxfp4(w: np.ndarray) -> np.ndarray:
    """[rows, K] float32 -> [rows, K/32*17] uint8 MX blocks (E8M0 scale code,
    then 16 bytes of E2M1 pairs, element 2i in the low nibble).

    X = 2^(floor(log2 amax) - 2) (2^-127 for an all-zero block); each x / X is
    rounded on its own grid: steps of 0.5 below 2, of 1 in [2, 4), of 2 from 4,
    ties to even, capped at 6."""
    rows, K = w.shape
    if K % 32:
        raise ValueError("MXFP4 needs K % 32 == 0")
    nb = K // 32
    out = np.empty((rows, nb, 17), dtype=np.uint8)

    def work(r0):
        r1 = min(rows, r0 + 2048)
        x = w[r0:r1].reshape(r1 - r0, nb, 32).astype(np.float32, copy=False)
        amax = np.abs(x).max(axis=2)
        bits = amax.view(np.int32)
        e = ((bits >> 23) & 0xFF) - 127                   # floor(log2 amax) for normal amax
        e = np.where(amax > 0, e, -125)
        sexp = np.clip(e - 2, -127, 127)
        a = np.abs(x) / np.ldexp(np.float32(1.0), sexp)[..., None].astype(np.float32)
        q = np.where(a < 2, np.rint(a * 2) / 2, np.where(a < 4, np.rint(a), 2 * np.rint(a / 2)))
        q = np.minimum(q, 6.0).astype(np.float32)
        c = np.searchsorted(_E2M1_POS, q).astype(np.uint8)
        c = c | np.where((x < 0) & (c > 0), 8, 0).astype(np.uint8)
        out[r0:r1, :, 0] = (sexp + 127).astype(np.uint8)
        out[r0:r1, :, 1:] = c[:, :, 0::2] | (c[:, :, 1::2] << 4)

    with _pool() as ex:
        list(ex.map(work, range(0, rows, 2048)))
    return out.reshape(rows, nb * 17)


@dataclass
class Stored:
    """One weight tensor in its storage format.

    f32:  data float32 [rows, cols] (or [n] for vectors)
    bf16: data uint16 [rows, cols] (bf16 bit patterns)
    q8_0: data uint8 [rows, cols/32*34] (canonical 34-byte blocks)
    fp8_e4m3: data uint8 [rows, cols], scales float32 [rows]
    mxfp4: data uint8 [rows, cols/32*17] (MX blocks of 32: E8M0 scale, 16 B of E2M1)
    """
    fmt: str
    shape: tuple
    data: np.ndarray
    scales: Optional[np.ndarray] = None

    @property
    def nbytes(self) -> int:
        return int(self.data.nbytes + (0 if self.scales is None else self.scales.nbytes))


def store(w: np.ndarray, fmt: str) -> Stored:
    if fmt == C.F32:
        return Stored(fmt, w.shape, np.ascontiguousarray(w, dtype=np.float32))
    if fmt == C.BF16:
        return Stored(fmt, w.shape, to_bf16_bits(w))
    if fmt == C.Q8_0:
        return Stored(fmt, w.shape, to_q8_0(w))
    if fmt == C.FP8:
        codes, s = to_fp8_e4m3_per_channel(w)
        return Stored(fmt, w.shape, codes, s)
    if fmt == C.MXFP4:
        return Stored(fmt, w.shape, to_mxfp4(w))
    raise ValueError(fmt)


def make_weights(wl: C.Workload, names: Optional[List[str]] = None) -> Dict[str, Stored]:
    """Draw every tensor of the workload (or the listed subset) and store it."""
    m = wl.model
    all_names = C.tensor_names(m, wl.attn_only)
    want = all_names if names is None else names
    out: Dict[str, Stored] = {}
    for idx, name in enumerate(all_names):
        if name not in want:
            continue
        shape = C.tensor_shape(m, name)
        fmt = C.tensor_format(wl.formats, name)
        base = name.split(".")[-1]
        if base.endswith("norm"):
            if wl.fixture_gains:
                w = uniform(shape, wl.seed, idx, 0.5, 1.5)
            else:
                w = np.ones(shape, np.float32)
        elif base == "conf_b":
            w = (normal(shape, wl.seed, idx, 0.5) if wl.fixture_gains
                 else np.zeros(shape, np.float32))
        elif base == "conf_w":
            w = normal(shape, wl.seed, idx, wl.weight_std)
        elif base in ("markov_w1", "markov_w2") and wl.markov_dominant:
            w = normal(shape, wl.seed, idx, float(m.markov_rank) ** -0.25)
        elif base == "lm_head" and wl.markov_dominant:
            w = np.zeros(shape, np.float32)
        else:
            w = normal(shape, wl.seed, idx, wl.weight_std)
            if base == "kv_b" and wl.sharp_attention:
                w3 = w.reshape(m.n_heads, m.qk_nope + m.v_head, m.kv_lora)
                w3[:, :m.qk_nope, :] *= np.float32(10.0)
        out[name] = store(w, fmt)
        del w
    return out


@dataclass
class Inputs:
    captured: Optional[np.ndarray]     # [n_seq, n_cap, block, H] f32 or bf16 bits
    x_in: Optional[np.ndarray]         # [n_seq*block, H] float32 (attention-only unit)
    caches: List[np.ndarray]           # per layer [total_ctx, latent] f32 or bf16 bits
    kv_offsets: np.ndarray             # int32 [n_seq+1]
    prev_token: np.ndarray             # int32 [n_seq]
    verifier: np.ndarray               # int32 [n_seq, block], uniform over vocab
    plant_pos: np.ndarray              # int32 [n_seq], first mismatch planted at this pos
    plant_delta: np.ndarray            # int32 [n_seq], token offset used to corrupt


def make_inputs(wl: C.Workload) -> Inputs:
    m = wl.model
    base = 1000  # input streams use spawn keys above the tensor list
    n_seq, blk = wl.n_seq, m.block
    latent = m.latent
    kv_off = np.zeros(n_seq + 1, dtype=np.int32)
    kv_off[1:] = np.cumsum(np.asarray(wl.kv_lens, dtype=np.int64)).astype(np.int32)
    total = int(kv_off[-1])

    def as_fmt(x, fmt):
        return x if fmt == C.F32 else to_bf16_bits(x)

    captured = x_in = None
    if wl.attn_only:
        x = normal((n_seq * blk, m.hidden), wl.seed, base + 0)
        x_in = bf16_bits_to_f32(to_bf16_bits(x))
    else:
        shape = (n_seq, m.n_captured, blk, m.hidden)
        cap = (student_t(shape, wl.seed, base + 0, 3.0) if wl.captured_dist == "heavy"
               else normal(shape, wl.seed, base + 0))
        captured = as_fmt(cap, wl.formats.captured)
    caches = []
    for l in range(m.n_layers):
        c = normal((total, latent), wl.seed, base + 1 + l)
        if wl.spike:
            c[wl.spike[0]] *= np.float32(wl.spike[1])
        caches.append(as_fmt(c, wl.formats.kv_cache))
    rng = np.random.default_rng(np.random.SeedSequence(wl.seed, spawn_key=(base + 500,)))
    prev = rng.integers(0, m.vocab, size=n_seq).astype(np.int32)
    ver = rng.integers(0, m.vocab, size=(n_seq, blk)).astype(np.int32)
    plant_pos = rng.integers(0, blk + 1, size=n_seq).astype(np.int32)
    plant_delta = rng.integers(1, m.vocab, size=n_seq).astype(np.int32)
    return Inputs(captured, x_in, caches, kv_off, prev, ver, plant_pos, plant_delta)


def planted_verifier(draft: np.ndarray, plant_pos: np.ndarray, plant_delta: np.ndarray,
                     vocab: int) -> np.ndarray:
    """Copy `draft` [n_seq, block] and corrupt position plant_pos[s] (if < block)."""
    v = np.array(draft, dtype=np.int32, copy=True)
    for s in range(v.shape[0]):
        k = int(plant_pos[s])
        if k < v.shape[1]:
            v[s, k] = (int(v[s, k]) + int(plant_delta[s])) % vocab
    return v


@dataclass
class PagedCaches:
    pools: List[np.ndarray]   # per layer [n_pages, page_size, latent], storage format of the caches
    table: np.ndarray         # int32 [n_seq, max_pages]: page of each sequence page (every entry valid)
    page_size: int


def paged_layout(caches: List[np.ndarray], kv_offsets: np.ndarray, page_size: int, seed: int,
                 spare_pages: int = 3) -> PagedCaches:
    """Scatter packed per-layer caches into page pools (a layout change only).

    Sequence s needs ceil(len_s / page_size) pages; all pages (plus
    `spare_pages` unused ones) get a seeded random placement in the pool.
    Rows a sequence does not reach (the tail of its last page, unused pages)
    hold random garbage, so a wrong page or row index shows up in results.
    Unused block-table entries point at valid pages too.
    """
    n_seq = len(kv_offsets) - 1
    lens = np.diff(np.asarray(kv_offsets, dtype=np.int64))
    need = [int(-(-int(n) // page_size)) for n in lens]
    max_pages = max(1, max(need))
    n_pages = sum(need) + spare_pages
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(7001,)))
    order = rng.permutation(n_pages).astype(np.int32)
    table = rng.integers(0, n_pages, size=(n_seq, max_pages)).astype(np.int32)
    k = 0
    for s in range(n_seq):
        table[s, :need[s]] = order[k:k + need[s]]
        k += need[s]
    pools = []
    for l, c in enumerate(caches):
        latent = c.shape[1]
        garbage = normal((n_pages, page_size, latent), seed, 7002 + l, std=3.0)
        pool = garbage if c.dtype == np.float32 else to_bf16_bits(garbage)
        for s in range(n_seq):
            off, n = int(kv_offsets[s]), int(lens[s])
            for p in range(need[s]):
                r0, r1 = p * page_size, min(n, (p + 1) * page_size)
                pool[table[s, p], :r1 - r0] = c[off + r0:off + r1]
        pools.append(pool)
    return PagedCaches(pools, table, page_size)
