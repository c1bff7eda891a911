"""The C ABI without a GPU: the shared library loads and exports every
function that include/dspark.h declares, and the binding refuses to run when
the library is missing (no CPU fallback).  No compute call is made."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")
LIB = os.path.join(ROOT, "mla_block_drafter_amd", "libdspark.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(dspark_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("dspark_draft_block", "dspark_accept_len", "dspark_model_create", "dspark_model_destroy",
                     "dspark_packed_bytes", "dspark_workspace_bytes", "dspark_last_error"):
        assert required in names, required


@pytest.mark.skipif(not os.path.exists(LIB), reason="libdspark.so not built (run __graft_entry__.build())")
def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # the exports are plain C symbols (extern "C"), not C++-mangled names
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in declared_functions():
        assert n in exported, n


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    from mla_block_drafter_amd import dspark as D
    monkeypatch.setattr(D, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(D, "_lib", None, raising=False)
    with pytest.raises(ImportError):
        D.lib()


@pytest.mark.skipif(not os.path.exists(LIB), reason="libdspark.so not built (run __graft_entry__.build())")
def test_read_probe_rejects_bad_arguments_before_enqueue():
    """dspark_read_probe validates on the host (no device is touched)."""
    lib = ctypes.CDLL(LIB)
    lib.dspark_read_probe.restype = ctypes.c_int32
    lib.dspark_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    EINVAL = -1
    assert lib.dspark_read_probe(None, 16, 0x2000, None) == EINVAL
    assert lib.dspark_read_probe(0x1000, 16, None, None) == EINVAL
    assert lib.dspark_read_probe(0x1008, 16, 0x2000, None) == EINVAL   # buf not 16-byte aligned
    assert lib.dspark_read_probe(0x1000, 24, 0x2000, None) == EINVAL   # bytes not a multiple of 16
    assert lib.dspark_read_probe(0x1000, 16, 0x2002, None) == EINVAL   # out not 4-byte aligned
