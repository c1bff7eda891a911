"""Reads of unwritten device memory: the workspace and the optional outputs are
filled with byte patterns before each draft pass (zeros, NaN, a finite
value); every output must come out bit-identical under every pattern and free
of NaN.  Covers the small-geometry workloads in each weight format (one, and
three ragged sequences including an empty cache, packed and paged), the tiny
all-fp32 drafter and the full-size Q8_0 pass at context 8192."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from synth import configs as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_block_drafter_amd import dspark as D
    D.lib()


def _bits(out):
    return {k: np.ascontiguousarray(v).view(np.uint8) for k, v in out.items()}


def _check_patterns(g, forced=None):
    from tests.gpu_common import POISON_PATTERNS
    runs = []
    for pat in (0x00,) + POISON_PATTERNS:
        g.poison = pat
        out = g.draft(forced=forced)
        for k in ("conf", "logits", "hidden"):
            assert np.isfinite(out[k]).all(), (pat, k)
        assert (out["tokens"] >= 0).all(), pat
        runs.append(_bits(out))
    for pat, r in zip(POISON_PATTERNS, runs[1:]):
        for k in runs[0]:
            np.testing.assert_array_equal(r[k], runs[0][k], err_msg=f"pattern {pat:#x}, {k}")


SMALL = {
    "bf16": C.ALL_BF16,
    "q8_0": C.Q8,
    "fp8": C.FP8_PC,
    "mxfp4": C.MX4,
}


@pytest.mark.parametrize("fmt", list(SMALL))
@pytest.mark.parametrize("lens", [(300,), (0, 37, 300)])
def test_poisoned_workspace_small(fmt, lens):
    from tests.gpu_common import GpuWorkload
    wl = C.Workload(f"poison_{fmt}", C.small_model(), SMALL[fmt], seed=1301, kv_lens=lens, fixture_gains=True)
    print("case", fmt, lens, flush=True)
    g = GpuWorkload(wl)
    _check_patterns(g)
    if fmt == "bf16":
        g.use_pages(64, seed=5)
        _check_patterns(g)


def test_poisoned_workspace_tiny_f32():
    from tests.gpu_common import GpuWorkload
    g = GpuWorkload(C.CFG1.replace(fixture_gains=True))
    _check_patterns(g)


def test_poisoned_workspace_full_q8_0():
    from tests.gpu_common import GpuWorkload
    print("case full q8_0 ctx 8192", flush=True)
    g = GpuWorkload(C.CFG3)
    _check_patterns(g)
