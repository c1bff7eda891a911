"""Paged latent caches on the GPU: the draft pass over page pools (seeded page
placement, garbage in every row no sequence reaches) against the oracle, and
bit for bit against the same pass over the packed caches (the paged layout
changes addressing only)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import dspark as O
from synth import configs as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_block_drafter_amd import dspark as D
    D.lib()


def _same(a, b):
    for k in ("tokens", "conf", "logits", "hidden"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("page_size", [32, 64, 512])
def test_small_ragged_paged_equals_packed_and_oracle(page_size):
    from tests.gpu_common import GpuWorkload, full_parity
    wl = C.Workload(f"small_paged_{page_size}", C.small_model(), C.ALL_BF16, seed=801,
                    kv_lens=(0, 37, 300), fixture_gains=True)
    g = GpuWorkload(wl)
    packed = g.draft()
    pc = g.use_pages(page_size, seed=page_size)
    print(f"page_size {page_size}: pool pages {pc.pools[0].shape[0]}, table {pc.table.shape}", flush=True)
    paged = g.draft()
    _same(paged, packed)
    ref = O.draft_block(wl, g.stored, g.inputs)
    full_parity(g, ref, tol=2e-2, max_ties=2)


def test_small_bs1_q8_paged_equals_packed():
    from tests.gpu_common import GpuWorkload
    wl = C.Workload("small_paged_bs1", C.small_model(), C.Q8, seed=802, kv_lens=(333,), fixture_gains=True)
    g = GpuWorkload(wl)
    packed = g.draft()
    g.use_pages(64, seed=5)
    _same(g.draft(), packed)


def test_full_size_q8_paged_equals_packed():
    """Full-size Q8_0 drafter, one sequence at context 8192, pages of 64 keys."""
    from tests.gpu_common import GpuWorkload
    g = GpuWorkload(C.CFG3)
    packed = g.draft()
    g.use_pages(64, seed=3)
    paged = g.draft()
    _same(paged, packed)
    print("cfg3 paged tokens", paged["tokens"].tolist(), flush=True)


@pytest.mark.parametrize("lens", [(40960,), (30000, 50000, 20000)])
def test_full_size_long_context_paged_equals_packed(lens):
    """Long contexts take larger attention slots (512 keys for one sequence
    at 40,960, 1024 keys for the three sequences), so with pages of 32 keys
    a slot spans 16 or 32 pages."""
    from tests.gpu_common import GpuWorkload
    wl = C.CFG3.replace(name=f"long_paged_{len(lens)}", kv_lens=lens)
    print("case", lens, flush=True)
    g = GpuWorkload(wl)
    packed = g.draft()
    assert (packed["tokens"] >= 0).all()
    g.use_pages(32, seed=7)
    paged = g.draft()
    _same(paged, packed)


def test_paged_rejects_bad_page_size():
    from mla_block_drafter_amd import dspark as D
    from tests.gpu_common import GpuWorkload
    wl = C.Workload("small_paged_bad", C.small_model(), C.ALL_BF16, seed=803, kv_lens=(40,), fixture_gains=True)
    g = GpuWorkload(wl)
    g.use_pages(32, seed=1)
    g.page_size = 48
    with pytest.raises(D.DsparkError) as e:
        g.draft()
    assert e.value.code == D.EINVAL
