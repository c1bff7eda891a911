"""Drift report at the full geometry (needs the GPU; not collected by pytest):

    python -m tests.drift_report [--dist gauss|heavy] [--n-seq 16] [--formats q8_0,fp8,mxfp4,bf16]

Reference: the oracle with the fp32 master weights; variants: the GPU draft
pass with the weights stored as each format (same master values), on the
same seeded captured states and bf16 latent caches.  Prints one metric row
per format (tests/drift.py)."""
from __future__ import annotations

import argparse
import dataclasses
import sys
import time

import numpy as np


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--dist", default="gauss")
    ap.add_argument("--n-seq", type=int, default=16)
    ap.add_argument("--formats", default="q8_0,fp8,mxfp4,bf16")
    args = ap.parse_args()
    import torch
    from synth import configs as C, gen
    from tests import drift as DR
    from tests.gpu_common import GpuWorkload
    fmts = {"bf16": C.ALL_BF16, "q8_0": C.Q8, "fp8": C.FP8_PC, "mxfp4": C.MX4}
    lens = tuple(int(v) for v in np.random.default_rng(11).integers(256, 2048, size=args.n_seq))
    base = C.Workload(f"drift_full_{args.dist}", C.FULL, dataclasses.replace(C.ALL_F32, kv_cache=C.BF16,
                                                                            captured=C.BF16),
                      seed=C.SEED_BASE + 77, kv_lens=lens, captured_dist=args.dist)
    t = time.time()
    inputs = gen.make_inputs(base)
    stored = gen.make_weights(base)
    print(f"[drift] fp32 master weights in {time.time() - t:.0f}s", flush=True)
    t = time.time()
    ref = DR.oracle_pass(base, stored, inputs)
    del stored
    print(f"[drift] reference pass (oracle, fp32 weights, {args.n_seq} blocks) in {time.time() - t:.0f}s", flush=True)
    n, B = base.n_seq, base.model.block
    for name in args.formats.split(","):
        wl = base.replace(formats=fmts[name])
        g = GpuWorkload(wl, inputs=inputs)
        free, forced = g.draft(), g.draft(forced=ref["tokens"])
        sh = lambda o: dict(tokens=o["tokens"], logits=o["logits"].reshape(n, B, -1),
                            hidden=o["hidden"].reshape(n * B, -1), conf=o["conf"])
        print(DR.fmt_row(f"{name} {args.dist}", DR.metrics(ref, sh(free), sh(forced))), flush=True)
        del g, free, forced
        torch.cuda.empty_cache()


if __name__ == "__main__":
    sys.exit(main())
