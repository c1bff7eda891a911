"""Cache append on the GPU (dspark_cache_append) against the oracle's cache
rows: every layer's row of each new position lands at its slot, within the
tolerance of the storage precision, and no other row of the caches changes."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import codecs, dspark as O
from synth import configs as C, gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_block_drafter_amd import dspark as D
    D.lib()


def _dev(a, fmt):
    t = torch.from_numpy(np.ascontiguousarray(a) if fmt == "f32" else np.ascontiguousarray(a).view(np.int16))
    t = t.to("cuda")
    return t if fmt == "f32" else t.view(torch.bfloat16)


def _host(t, fmt):
    if fmt == "f32":
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _decode(a, fmt):
    return np.asarray(a, np.float64) if fmt == "f32" else codecs.bf16_decode(a)


def _append_case(wl, n_new, pool_rows, seed, tol):
    from tests.gpu_common import GpuWorkload
    m = wl.model
    g = GpuWorkload(wl)
    rng = np.random.default_rng(seed)
    cap = gen.normal((n_new, m.n_captured, m.hidden), seed, 1)
    cap = cap if wl.formats.captured == "f32" else gen.to_bf16_bits(cap)
    positions = rng.integers(0, 70000, size=n_new).astype(np.int32)
    slots = rng.choice(pool_rows, size=n_new, replace=False).astype(np.int64)
    kvf = wl.formats.kv_cache
    pools = []
    for l in range(m.n_layers):
        p = gen.normal((pool_rows, m.latent), seed, 10 + l, std=5.0)
        pools.append(p if kvf == "f32" else gen.to_bf16_bits(p))
    dpools = [_dev(p, kvf) for p in pools]
    ws = g.model.append_workspace(n_new)
    g.model.cache_append(_dev(cap, wl.formats.captured), torch.from_numpy(positions).cuda(),
                         torch.from_numpy(slots).cuda(), dpools, ws)
    torch.cuda.synchronize()
    ref = O.cache_rows(m, O.Weights(g.stored), cap, positions, wl.formats.captured)
    keep = np.setdiff1d(np.arange(pool_rows), slots)
    for l in range(m.n_layers):
        after = _host(dpools[l], kvf)
        assert np.array_equal(after[keep], pools[l][keep]), f"layer {l}: a row outside the slots changed"
        got = _decode(after[slots], kvf)
        err = float(np.max(np.abs(got - ref[l])) / np.max(np.abs(ref[l])))
        print(f"{wl.name} layer {l}: rel err {err:.2e}", flush=True)
        assert err < tol, (l, err)


def test_append_small_bf16_nine_rows():
    wl = C.Workload("append_small_bf16", C.small_model(), C.ALL_BF16, seed=901, kv_lens=(10,), fixture_gains=True)
    _append_case(wl, 9, 300, 5, 1e-2)


def test_append_small_q8_five_rows():
    wl = C.Workload("append_small_q8", C.small_model(), C.Q8, seed=902, kv_lens=(10,), fixture_gains=True)
    _append_case(wl, 5, 100, 6, 1e-2)


@pytest.mark.parametrize("name,formats", [("fp8", C.FP8_PC), ("mxfp4", C.MX4)])
def test_append_small_fp8_mxfp4_fc(name, formats):
    """fc in FP8 or MXFP4 (bf16 hi/lo activation fragments for the fc GEMM)."""
    wl = C.Workload(f"append_small_{name}", C.small_model(), formats, seed=904, kv_lens=(10,), fixture_gains=True)
    _append_case(wl, 6, 120, 9, 1e-2)


def test_append_tiny_f32():
    _append_case(C.CFG1.replace(fixture_gains=True), 7, 64, 7, 1e-4)


def test_append_full_size_q8_seven_rows():
    _append_case(C.CFG3, 7, 4096, 8, 1e-2)


def test_append_rejects_bad_counts():
    from mla_block_drafter_amd import dspark as D
    from tests.gpu_common import GpuWorkload
    wl = C.Workload("append_bad", C.small_model(), C.ALL_BF16, seed=903, kv_lens=(10,))
    g = GpuWorkload(wl)
    with pytest.raises(D.DsparkError):
        g.model.append_workspace(0)
    with pytest.raises(D.DsparkError):
        g.model.append_workspace(D.APPEND_MAX + 1)
