"""The C ABI's host side without a device (include/dspark.h).

* Every pre-enqueue validation error of every call, driven on plan-only
  models (DSPARK_CFG_PLAN_ONLY) by tests/abi_host_check.cpp, built with
  AddressSanitizer, UndefinedBehaviorSanitizer and leak checking against a
  host-side sanitized build of the library: nothing is enqueued, no device
  is touched.
* dspark_accept_len_host brute-forced against the oracle's prefix run length
  over every (draft, verifier) pair of small alphabets (huggingface.co
  "Kimi-K3-DSpark-NVFP4", "Why acceptance is so sensitive": a block is
  accepted up to its first mismatch).
* The library loads, answers plan-only calls and unloads with a clean exit.
"""
import ctypes as C
import itertools
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import dspark as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mla_block_drafter_amd", "libdspark.so")
need_lib = pytest.mark.skipif(not os.path.exists(LIB), reason="libdspark.so not built (run __graft_entry__.build())")


@need_lib
def test_validation_paths_under_sanitizers():
    from mla_block_drafter_amd import build as B
    exe = B.build_host_sanitized(os.path.join(ROOT, "tests", "abi_host_check.cpp"))
    args = [exe] + ([] if os.path.exists("/dev/kfd") else ["--no-device"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run(args, capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) >= 150


@need_lib
@pytest.mark.parametrize("alpha,block", [(3, 1), (3, 2), (3, 3), (3, 4), (3, 5), (2, 7)])
def test_accept_len_host_vs_oracle(alpha, block):
    from mla_block_drafter_amd import dspark as D
    seqs = np.array(list(itertools.product(range(alpha), repeat=block)), np.int32)
    d = np.repeat(seqs, len(seqs), axis=0)
    v = np.tile(seqs, (len(seqs), 1))
    got = D.accept_len_host(d, v)
    np.testing.assert_array_equal(got, O.accept_len(d, v))
    assert got.min() == 0 and got.max() == block


@need_lib
def test_accept_len_host_planted():
    from mla_block_drafter_amd import dspark as D
    rng = np.random.default_rng(5)
    d = rng.integers(0, 163840, size=(64, 7), dtype=np.int32)
    k = rng.integers(0, 8, size=64)
    v = d.copy()
    for s in range(64):
        if k[s] < 7:
            v[s, k[s]] = (v[s, k[s]] + 1 + rng.integers(0, 100)) % 163840
    np.testing.assert_array_equal(D.accept_len_host(d, v), k)


@need_lib
def test_plan_only_model_through_the_binding():
    """Sizes are answered and validation runs with no device: a plan-only
    model of the full geometry."""
    from mla_block_drafter_amd import dspark as D
    from synth import configs as Cf
    L = D.lib()
    m = Cf.FULL
    wl = Cf.CFG3
    names = Cf.tensor_names(m)
    table = (D.Weight * len(names))()
    for i, name in enumerate(names):
        shape = Cf.tensor_shape(m, name)
        fmt = Cf.tensor_format(wl.formats, name)
        table[i].id = D.weight_id(name)
        table[i].dtype = D.FMT_CODE[fmt]
        table[i].data = 0x10000000 + i * 0x1000000          # never read
        table[i].scales = None
        table[i].rows, table[i].cols = shape[0], (shape[1] if len(shape) == 2 else 1)
    cfg = D.make_config(m, plan_only=True)
    packed = L.dspark_packed_bytes(C.byref(cfg), table, len(names))
    assert packed > 5_000_000_000 // 1                      # the repacked weights, padded to tiles
    h = C.c_void_p()
    assert L.dspark_model_create(C.byref(cfg), table, len(names), None, 0, None, C.byref(h)) == D.OK
    ws8k = L.dspark_workspace_bytes(h, 1, 8192)
    ws98k = L.dspark_workspace_bytes(h, 1, 98304)
    assert 0 < ws8k < ws98k
    bad = L.dspark_workspace_bytes(h, 0, 8192)
    assert bad == 0 and "n_seq" in D.last_error()
    assert L.dspark_model_destroy(h) == D.OK


@need_lib
def test_library_unloads_cleanly():
    """Load, use and exit: no crash in static destructors or at unload (the
    library's teardown makes no HIP call)."""
    code = ("import ctypes, sys; sys.path.insert(0, %r); "
            "from mla_block_drafter_amd import dspark as D; import numpy as np; "
            "D.accept_len_host(np.zeros((2, 7), np.int32), np.zeros((2, 7), np.int32)); "
            "L = D.lib(); assert L.dspark_accept_len_host(None, None, 1, 1, None) == D.EINVAL; "
            "print(D.last_error())" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "NULL" in r.stdout
