#!/usr/bin/env python
"""Benchmark of one DSpark draft pass on one MI355X.

A step is one pass of the whole hot path (fc, 5 MLA decoder layers, lm_head,
Markov rollout, confidence) over one 7-token block of the full-size Q8_0
workload at context 8192 (seeded synthetic weights ~N(0, 0.02) and inputs),
with every input already resident in HBM.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--config 3]

value = draft-pass latency in microseconds per 7-token block (lower is
better), timed over K replays of the pass captured in a HIP graph (the pass
is a chain of 53 dependent launches, so a serving loop replays it as a
graph; with --no-graph, or should capture fail, K eager passes); the eager
time is reported beside it.  The JSON also carries the achieved algorithmic HBM bandwidth of the
pass, the roofline of the dominant kernel (the lm_head GEMM, one launch per
pass, timed live with HIP events recorded on the library's stream around
that launch), and the CPU oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft-pass latency (us/7-token block, bs=1) + achieved HBM GB/s % of peak"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(wl, stored, inp, budget_s: float = 40.0):
    """The oracle (float64 numpy, as it stands) on the same workload: whole
    draft passes (fc, every decoder layer, lm_head, the Markov rollout and the
    confidence; the stored weights are decoded inside the pass, as the oracle
    does).  One pass is timed; when it took under a third of the budget, two
    more are and the median is reported."""
    import numpy as np
    from oracle import dspark as O
    times = []
    while True:
        t0 = time.perf_counter()
        out = O.draft_block(wl, stored, inp)
        times.append(time.perf_counter() - t0)
        assert np.isfinite(out["logits"]).all()
        if len(times) >= 3 or sum(times) + times[0] > budget_s or times[0] > budget_s / 3:
            break
    dt = float(np.median(times))
    cores = len(os.sched_getaffinity(0))
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            cores = max(i.get("num_threads", 0) for i in info) or cores
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
    except Exception:
        pass
    return {"value": round(dt * 1e6 / wl.n_seq, 1), "unit": "us/block", "cores": int(cores), "kind": "oracle",
            "sample": f"whole draft pass of {wl.name} ({wl.n_seq} block(s)), float64 numpy with {blas}, weights "
                      f"decoded inside the pass; median of {len(times)} pass(es): "
                      + ", ".join(f"{t:.1f} s" for t in times)}


KERNEL_SOURCES = ["common.h", "kernels.h", "gemv_impl.h", "k_gemv.hip", "k_gemv_bf16.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lm_head_gemv_bf16_q8_0_ctx8192_traffic.txt")


def kernel_source_hash() -> str:
    """Hash of the sources the lm_head GEMM kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mla_block_drafter_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per lm_head launch from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split("=", 1) for line in f.read().splitlines() if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("source_hash", "").strip() != kernel_source_hash():
        return None
    return int(kv["traffic_bytes_per_launch"])


def copy_calibration():
    """A plain device copy of known size (for scaling rocprofv3 byte counters)."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def read_calibration():
    """A plain device read of known size (a second kernel for scaling the
    rocprofv3 FETCH_SIZE counter): torch's sum over 1 GiB, five times."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    acc = torch.zeros((), dtype=torch.float32, device="cuda")
    for _ in range(5):
        acc += src.sum()
    torch.cuda.synchronize()
    print(json.dumps({"read_bytes": n, "launches": 5, "sum": float(acc)}), flush=True)


def read_probe_gbs(torch) -> float:
    """Device read bandwidth of the library's streaming-read probe over 1 GiB
    (dspark_read_probe: 16-byte non-temporal loads, 2048 workgroups; bytes
    read / time): the achievable rate for a read-only weight stream."""
    from mla_block_drafter_amd import dspark as D
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    out = torch.zeros(D.READ_PROBE_WORDS, dtype=torch.int32, device="cuda")
    D.read_probe(src, out)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        D.read_probe(src, out)
    b.record()
    torch.cuda.synchronize()
    gbs = n * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, out
    torch.cuda.empty_cache()
    return gbs


def copy_probe_gbs(torch) -> float:
    """Device copy bandwidth (read + write bytes / time) of a 1 GiB copy."""
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * n * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def secondary_record(k: int, steps: int, warmup: int) -> dict:
    """One more workload (graph replays of its pass, checked bit for bit
    against the eager pass; eager timing if capture fails), for the record:
    not the headline."""
    import numpy as np
    import torch
    from mla_block_drafter_amd import dspark as D
    from synth import accounting as A, configs as C, gen
    wl = C.PRESETS[k]
    m = wl.model
    t = time.time()
    stored = gen.make_weights(wl)
    inp = gen.make_inputs(wl)
    model = D.Model(m, D.upload_stored(stored))
    del stored
    dev = "cuda"
    cap = torch.from_numpy(inp.captured.view(np.int16)).to(dev).view(torch.bfloat16)
    kv = [torch.from_numpy(c.view(np.int16)).to(dev).view(torch.bfloat16) for c in inp.caches]
    offs = torch.from_numpy(inp.kv_offsets).to(dev)
    prev = torch.from_numpy(inp.prev_token).to(dev)
    n, B = wl.n_seq, m.block
    ws = model.workspace(n, wl.total_ctx)
    tokens = torch.empty((n, B), dtype=torch.int32, device=dev)
    conf = torch.empty((n, B), dtype=torch.float32, device=dev)

    def run():
        model.draft_block(cap, kv, offs, prev, wl.total_ctx, tokens, conf, ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        run()
    b.record()
    torch.cuda.synchronize()
    eager_ms = a.elapsed_time(b) / steps
    ref_t, ref_c = tokens.clone(), conf.clone()
    graph_ms = None
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        if torch.equal(tokens, ref_t) and torch.equal(conf.view(torch.int32), ref_c.view(torch.int32)):
            graph_ms = a.elapsed_time(b) / steps
    except Exception as e:
        log(f"[bench] graph capture of {wl.name} skipped: {e!r}")
    ms = graph_ms if graph_ms is not None else eager_ms
    total = A.total_bytes(wl)
    gbs = total / (ms * 1e-3) / 1e9
    rec = {"workload": wl.name, "n_seq": n, "us_per_call": round(ms * 1e3, 2),
           "us_per_block": round(ms * 1e3 / n, 2), "eager_us_per_call": round(eager_ms * 1e3, 2),
           "launch": "hip graph" if graph_ms is not None else "eager", "algorithmic_bytes": total,
           "hbm_gbs": round(gbs, 1), "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    log(f"[bench] secondary {wl.name}: {rec['us_per_call']} us per call ({time.time() - t:.0f}s with generation)")
    del model, ws, kv, cap
    torch.cuda.empty_cache()
    return rec


def layer_record(steps: int, warmup: int) -> dict:
    """One full-size MLA layer, attention half (input norm, q/kv projections,
    absorbed attention over 4,096 latent rows, o_proj and the residual), all
    bf16, through dspark_layer_forward.  Its 207 MB fit in the 256 MB
    Infinity Cache, so a 1 GiB buffer is read and written between timed calls
    (outside each call's events); back-to-back calls are reported as warm."""
    import numpy as np
    import torch
    from mla_block_drafter_amd import dspark as D
    from synth import accounting as A, configs as C, gen
    wl = C.CFG2
    m = wl.model
    t = time.time()
    stored = gen.make_weights(wl)
    inp = gen.make_inputs(wl)
    model = D.Model(m, D.upload_stored(stored), layers_only=True)
    del stored
    xi = torch.from_numpy(np.ascontiguousarray(inp.x_in, np.float32)).cuda()
    xo = torch.empty_like(xi)
    kv = torch.from_numpy(inp.caches[0].view(np.int16)).cuda().view(torch.bfloat16)
    offs = torch.from_numpy(inp.kv_offsets.astype(np.int32)).cuda()
    ws = model.workspace(wl.n_seq, wl.total_ctx)
    flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")

    def run():
        model.layer_forward(0, False, xi, xo, kv, offs, wl.total_ctx, ws)

    for _ in range(warmup):
        flush.add_(1.0)
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        flush.add_(1.0)
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    cold = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    for a, b in ev:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    warm = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    total = A.total_bytes(wl)
    med = float(np.median(cold))
    gbs = total / (med * 1e-6) / 1e9
    rec = {"workload": wl.name, "calls": steps, "us_median_p10_p90": [round(med, 2), round(float(np.percentile(cold, 10)), 2),
                                                                     round(float(np.percentile(cold, 90)), 2)],
           "warm_us_median": round(float(np.median(warm)), 2), "infinity_cache": "flushed (1 GiB read and written between calls)",
           "algorithmic_bytes": total, "hbm_gbs": round(gbs, 1), "hbm_frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
           "launch": "eager"}
    log(f"[bench] layer {wl.name}: {rec['us_median_p10_p90']} us flushed, {rec['warm_us_median']} us warm "
        f"({time.time() - t:.0f}s with generation)")
    del model, ws, kv, flush
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip the cache-append timing")
    ap.add_argument("--no-sampling", action="store_true",
                    help="skip the sampled-pass and block-verification timings")
    ap.add_argument("--page-size", type=int, default=0,
                    help="latent caches as page pools of this many tokens (seeded page placement)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (byte-counter calibration) and exit")
    ap.add_argument("--read-calibration", action="store_true",
                    help="only run a 1 GiB device read (second byte-counter calibration) and exit")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary records (long-context BF16, batched FP8, one MLA layer)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.read_calibration:
        read_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the draft pass is not "
              "sharded across GPUs.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from mla_block_drafter_amd import dspark as D
    from synth import accounting as A, configs as C, gen

    wl = C.PRESETS[args.config]
    m = wl.model
    if wl.attn_only:
        # the single-layer workload: its own record (not the headline metric)
        print(json.dumps(layer_record(steps=max(args.steps, 10), warmup=args.warmup)), flush=True)
        return
    t = time.time()
    stored = gen.make_weights(wl)
    inp = gen.make_inputs(wl)
    log(f"[bench] generated {wl.name} in {time.time() - t:.1f}s")
    t = time.time()
    model = D.Model(m, D.upload_stored(stored))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"[bench] model packed ({model.packed_bytes / 1e9:.2f} GB) in {time.time() - t:.1f}s")

    dev = "cuda"
    cap = (torch.from_numpy(inp.captured).to(dev) if wl.formats.captured == "f32"
           else torch.from_numpy(inp.captured.view(np.int16)).to(dev).view(torch.bfloat16))
    kv = [(torch.from_numpy(c).to(dev) if wl.formats.kv_cache == "f32"
           else torch.from_numpy(c.view(np.int16)).to(dev).view(torch.bfloat16)) for c in inp.caches]
    offs = torch.from_numpy(inp.kv_offsets).to(dev)
    prev = torch.from_numpy(inp.prev_token).to(dev)
    n, B = wl.n_seq, m.block
    ws = model.workspace(n, wl.total_ctx)
    tokens = torch.empty((n, B), dtype=torch.int32, device=dev)
    conf = torch.empty((n, B), dtype=torch.float32, device=dev)

    table = None
    if args.page_size:
        pc = gen.paged_layout(inp.caches, inp.kv_offsets, args.page_size, seed=wl.seed)
        kv = [torch.from_numpy(p.view(np.int16)).to(dev).view(torch.bfloat16) for p in pc.pools]
        table = torch.from_numpy(pc.table).to(dev)
        del pc

    def run(evs=None):
        model.draft_block(cap, kv, offs, prev, wl.total_ctx, tokens, conf, ws, stage_events=evs,
                          page_size=args.page_size, block_table=table)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    K = args.steps
    # the timed passes: back to back, nothing else in the stream
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record()
    for k in range(K):
        run()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_begin.elapsed_time(t_end) / K
    # per-pass spread and per-stage times, from a second set of passes with
    # events between them (the events themselves cost a little)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * D.N_STAGES)] for _ in range(K)]
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for k in range(K):
        step_ev[k].record()
        run(evs[k])
    step_ev[K].record()
    torch.cuda.synchronize()
    per_step = np.array([step_ev[k].elapsed_time(step_ev[k + 1]) for k in range(K)])
    stage_ms = np.array([[evs[k][2 * s].elapsed_time(evs[k][2 * s + 1]) for s in range(D.N_STAGES)]
                         for k in range(K)]).mean(axis=0)
    log("[bench] eager: %.1f us/pass; stages (us): %s" % (
        ms_step * 1e3, ", ".join(f"{nm} {v * 1e3:.1f}" for nm, v in zip(D.STAGES, stage_ms))))

    eager_tokens, eager_conf = tokens.clone(), conf.clone()
    graph_ms = None
    if not args.no_graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                run()
            torch.cuda.current_stream().wait_stream(s)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run()
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(K):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            graph_ms = a.elapsed_time(b) / K
            # the replays must reproduce the eager outputs bit for bit
            if not (torch.equal(tokens, eager_tokens) and torch.equal(conf.view(torch.int32), eager_conf.view(torch.int32))):
                log("[bench] graph replay outputs differ from the eager pass: eager timing is the headline")
                graph_ms = None
            else:
                log("[bench] graph: %.1f us/pass" % (graph_ms * 1e3))
        except Exception as e:  # capture failure: the eager timing is the headline
            log(f"[bench] graph capture skipped: {e!r}")
            graph_ms = None

    append = None
    if not args.no_append:
        # dspark_cache_append of one block's worth of verified positions (the
        # rows go to a separate pool, so the pass inputs stay as they are)
        n_new = B
        cap_new = gen.normal((n_new, m.n_captured, m.hidden), wl.seed, 9000)
        cap_new = (torch.from_numpy(cap_new).to(dev) if wl.formats.captured == "f32" else
                   torch.from_numpy(gen.to_bf16_bits(cap_new).view(np.int16)).to(dev).view(torch.bfloat16))
        pos_new = torch.arange(n_new, dtype=torch.int32, device=dev) + int(wl.total_ctx // n)
        slot_new = torch.arange(n_new, dtype=torch.int64, device=dev)
        pool_new = [torch.zeros((n_new, m.latent), dtype=kv[0].dtype, device=dev) for _ in range(m.n_layers)]
        ws_app = model.append_workspace(n_new)
        for _ in range(args.warmup):
            model.cache_append(cap_new, pos_new, slot_new, pool_new, ws_app)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(K):
            model.cache_append(cap_new, pos_new, slot_new, pool_new, ws_app)
        b.record()
        torch.cuda.synchronize()
        app_ms = a.elapsed_time(b) / K
        app_bytes = A.append_bytes(wl, n_new)
        append = {"rows": n_new, "us": round(app_ms * 1e3, 2), "algorithmic_bytes": app_bytes,
                  "gbs": round(app_bytes / (app_ms * 1e-3) / 1e9, 1)}
        log(f"[bench] cache append of {n_new} rows: {app_ms * 1e3:.1f} us")

    sampling = None
    if not args.no_sampling:
        # probabilistic drafting (Gumbel-max draws from resident uniforms at
        # temperature 1) and block verification of the sampled block against
        # synthetic target logits (the draft's logits plus noise)
        V = m.vocab
        u = torch.rand((n, B, V), generator=torch.Generator(device=dev).manual_seed(wl.seed), device=dev)
        u.clamp_(1e-7, 1 - 1e-7)
        for _ in range(args.warmup):
            model.draft_block(cap, kv, offs, prev, wl.total_ctx, tokens, conf, ws, sample_u=u, temperature=1.0,
                              page_size=args.page_size, block_table=table)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(K):
            model.draft_block(cap, kv, offs, prev, wl.total_ctx, tokens, conf, ws, sample_u=u, temperature=1.0,
                              page_size=args.page_size, block_table=table)
        b.record()
        torch.cuda.synchronize()
        samp_ms = a.elapsed_time(b) / K
        dlog = torch.empty((n, B, V), dtype=torch.float32, device=dev)
        model.draft_block(cap, kv, offs, prev, wl.total_ctx, tokens, conf, ws, logits=dlog, sample_u=u,
                          temperature=1.0, page_size=args.page_size, block_table=table)
        g = torch.Generator(device=dev).manual_seed(wl.seed + 1)
        tlog = torch.cat([dlog, dlog[:, -1:]], dim=1) + torch.randn((n, B + 1, V), generator=g, device=dev)
        r = torch.rand((n, B + 1), generator=g, device=dev)
        out_len = torch.empty(n, dtype=torch.int32, device=dev)
        out_tok = torch.empty(n, dtype=torch.int32, device=dev)
        vws = torch.empty(D.verify_workspace_bytes(n, B), dtype=torch.uint8, device=dev)
        def verify():
            D.verify(tokens, dlog, tlog, r, 1.0, D.VERIFY_BLOCK, out_len, out_tok, workspace=vws)

        for _ in range(args.warmup):
            verify()
        torch.cuda.synchronize()
        # eager calls through the Python binding are host-bound (four small
        # launches): the device time is taken from a captured graph's replays
        vs = torch.cuda.Stream()
        vs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(vs):
            verify()
        torch.cuda.current_stream().wait_stream(vs)
        vg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(vg):
            verify()
        vg.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(K):
            vg.replay()
        b.record()
        torch.cuda.synchronize()
        ver_ms = a.elapsed_time(b) / K
        ver_bytes = 4 * n * V * (2 * B + 1)  # draft and target logits once
        sampling = {"sampled_pass_us": round(samp_ms * 1e3, 2), "verify_block_us": round(ver_ms * 1e3, 2),
                    "verify_algorithmic_bytes": ver_bytes,
                    "verify_gbs": round(ver_bytes / (ver_ms * 1e-3) / 1e9, 1),
                    "accepted": out_len.cpu().tolist()}
        log(f"[bench] sampled pass {samp_ms * 1e3:.1f} us; block verification {ver_ms * 1e3:.1f} us")

    copy_gbs = copy_probe_gbs(torch)
    read_gbs = read_probe_gbs(torch)
    log(f"[bench] device copy probe: {copy_gbs:.0f} GB/s; read probe: {read_gbs:.0f} GB/s")
    total_bytes = A.total_bytes(wl)
    blocks = n
    lm_bytes = A.lm_head_launch_bytes(wl)
    lm_ms = float(stage_ms[2])
    lm_gbs = lm_bytes / (lm_ms * 1e-3) / 1e9
    head_ms = graph_ms if graph_ms is not None else ms_step
    pass_gbs = total_bytes / (head_ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        t = time.time()
        cpu = cpu_baseline(wl, stored, inp)
        log(f"[bench] cpu baseline in {time.time() - t:.1f}s: {cpu}")
    fmt = {C.Q8_0: "q8_0", C.FP8: "fp8_e4m3", C.MXFP4: "mxfp4", C.BF16: "bf16", C.F32: "f32"}[wl.formats.mlp]
    out = {
        "metric": METRIC,
        "value": round(head_ms * 1e3 / blocks, 2),
        "unit": "us/block",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(head_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "n_seq": n, "block": B, "ctx": int(wl.total_ctx // n),
                   "hidden": m.hidden, "layers": m.n_layers, "vocab": m.vocab, "weights": fmt,
                   "algorithmic_bytes": total_bytes, "kv_layout": f"paged{args.page_size}" if args.page_size else "packed",
                   "launch": "hip graph" if graph_ms is not None else "eager"},
        "hbm_gbs": round(pass_gbs, 1),
        "hbm_frac_of_peak": round(pass_gbs / HBM_PEAK_GBS, 4),
        "hbm_frac_of_copy_probe": round(pass_gbs / copy_gbs, 4),
        "copy_probe_gbs": round(copy_gbs, 1),
        "hbm_frac_of_read_probe": round(pass_gbs / read_gbs, 4),
        "read_probe_gbs": round(read_gbs, 1),
        "step_us_median_p10_p90": [round(float(np.percentile(per_step, q)) * 1e3, 2) for q in (50, 10, 90)],
        "eager_us_per_block": round(ms_step * 1e3 / blocks, 2),
        "graph_us_per_block": None if graph_ms is None else round(graph_ms * 1e3 / blocks, 2),
        "stage_us": {nm: round(v * 1e3, 2) for nm, v in zip(D.STAGES, stage_ms)},
        "roofline": {"bound": "hbm", "kernel": "lm_head GEMM (k_gemv_bf, BF16 weights)",
                     "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(lm_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "bytes_per_launch": lm_bytes, "avg_launch_us": round(lm_ms * 1e3, 2),
                     "frac_of_read_probe": round(lm_gbs / read_gbs, 4)},
        "cpu_baseline": cpu,
        "cache_append": append,
        "sampling": sampling,
    }
    if not args.no_secondary and args.config == 3:
        del model, ws, kv, cap
        torch.cuda.empty_cache()
        out["secondary"] = [secondary_record(k, steps=min(K, 20), warmup=min(args.warmup, 3)) for k in (4, 5)]
        out["layer"] = layer_record(steps=max(K, 50), warmup=args.warmup)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
