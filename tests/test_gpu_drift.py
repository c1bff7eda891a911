"""Drift of the GPU draft pass with BF16 / Q8_0 / FP8 weights against the
oracle with the same master weights in fp32 (huggingface.co
"Kimi-K3-DSpark-NVFP4", "Measurement" and "Detail"), on "gauss" and "heavy"
captured states, 16 sequences of the mid-size geometry.  The oracle with the
quantised weights is measured alongside: the GPU's drift must match it."""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from synth import configs as C, gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_block_drafter_amd import dspark as D
    D.lib()


FORMATS = {"bf16": C.ALL_BF16, "q8_0": C.Q8, "fp8": C.FP8_PC, "mxfp4": C.MX4}
F32_WEIGHTS = dataclasses.replace(C.ALL_F32, kv_cache=C.BF16, captured=C.BF16)


@pytest.mark.parametrize("dist", ["gauss", "heavy"])
def test_drift_gpu_matches_oracle_drift(dist):
    from tests import drift as DR
    from tests.gpu_common import GpuWorkload
    lens = tuple(int(v) for v in np.random.default_rng(5).integers(0, 400, size=16))
    base = C.Workload(f"drift_{dist}", C.small_model(), F32_WEIGHTS, seed=4242, kv_lens=lens,
                      captured_dist=dist)
    inputs = gen.make_inputs(base)
    ref = DR.oracle_pass(base, gen.make_weights(base), inputs)
    for name, fm in FORMATS.items():
        wl = base.replace(formats=fm)
        g = GpuWorkload(wl, inputs=inputs)
        free = g.draft()
        forced = g.draft(forced=ref["tokens"])
        m_gpu = DR.metrics(ref, _shape(wl, free), _shape(wl, forced))
        ofree = DR.oracle_pass(wl, g.stored, inputs)
        oforced = DR.oracle_pass(wl, g.stored, inputs, forced=ref["tokens"])
        m_or = DR.metrics(ref, ofree, oforced)
        print(DR.fmt_row(f"gpu    {name} {dist}", m_gpu), flush=True)
        print(DR.fmt_row(f"oracle {name} {dist}", m_or), flush=True)
        # the GPU adds its own rounding to the format's drift, not a drift of its own
        assert abs(m_gpu["greedy"] - m_or["greedy"]) <= 0.05, name
        assert abs(m_gpu["ceiling"] - m_or["ceiling"]) <= 0.75, name
        assert m_gpu["hidden_rel"] <= m_or["hidden_rel"] + 0.02, name
        del g
        torch.cuda.empty_cache()


def _shape(wl, out):
    n, B = wl.n_seq, wl.model.block
    return dict(tokens=out["tokens"], logits=out["logits"].reshape(n, B, -1),
                hidden=out["hidden"].reshape(n * B, -1), conf=out["conf"])
