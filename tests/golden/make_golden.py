"""Write the oracle's outputs for the full-size draft-pass workloads.

Calls only synth (seeded inputs) and oracle (float64 reference).  Usage:

    python tests/golden/make_golden.py 3 4 5 6 7

Per workload it stores, in tests/golden/pass_cfg<k>.npz:
  tokens [n_seq, block], conf [n_seq, block]      free-running oracle draft
  hidden_idx, hidden_val                           sampled (row, col) of the
                                                   final-normed hidden state
  top_idx, top_val [n_seq, block, 64]              the 64 largest logits
  smp_idx, smp_val [n_seq, block, 2048]            a fixed random sample of logits
  logit_absmax [n_seq, block]                      max |logit| per position
The logits are the Markov-augmented l_i on the oracle's own token path.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import dspark as O  # noqa: E402
from synth import configs as C, gen  # noqa: E402

TOPK = 64
NSAMPLE = 2048
NHIDDEN = 16384


def make(k: int) -> str:
    wl = C.PRESETS[k]
    t = time.time()
    stored = gen.make_weights(wl)
    inp = gen.make_inputs(wl)
    ref = O.draft_block(wl, stored, inp)
    lg = ref["logits"]                                    # [n_seq, B, V] float64
    n, B, V = lg.shape
    top_idx = np.argsort(-lg, axis=2, kind="stable")[:, :, :TOPK].astype(np.int32)
    top_val = np.take_along_axis(lg, top_idx, axis=2)
    rng = np.random.default_rng(np.random.SeedSequence(wl.seed, spawn_key=(777,)))
    smp_idx = rng.integers(0, V, size=(n, B, NSAMPLE)).astype(np.int32)
    smp_val = np.take_along_axis(lg, smp_idx, axis=2)
    hid = ref["hidden"]                                   # [n*B, H]
    M, H = hid.shape
    if M * H <= NHIDDEN * 4:
        hidden_idx = np.arange(M * H, dtype=np.int64)
    else:
        hidden_idx = np.sort(rng.choice(M * H, size=NHIDDEN, replace=False)).astype(np.int64)
    hidden_val = hid.reshape(-1)[hidden_idx]
    path = os.path.join(HERE, f"pass_cfg{k}.npz")
    np.savez_compressed(path, tokens=ref["tokens"].astype(np.int32), conf=ref["conf"],
                        hidden_idx=hidden_idx, hidden_val=hidden_val, hidden_absmax=np.abs(hid).max(),
                        top_idx=top_idx, top_val=top_val, smp_idx=smp_idx, smp_val=smp_val,
                        logit_absmax=np.abs(lg).max(axis=2))
    print(f"cfg{k}: {wl.name} in {time.time() - t:.1f}s -> {path}", flush=True)
    return path


if __name__ == "__main__":
    for a in sys.argv[1:]:
        make(int(a))
