"""The drift harness (tests/drift.py) on the CPU: its metric functions against
closed forms and brute force, then a whole drift measurement of the oracle
with quantised weights against the oracle with fp32 weights (the same master
values, huggingface.co "Kimi-K3-DSpark-NVFP4", "Measurement")."""
import dataclasses

import numpy as np
import pytest

from oracle import dspark as O
from synth import configs as C, gen
from tests import drift as DR


def test_kl_tv_closed_forms():
    lp = DR.log_softmax(np.array([[0.0, 0.0]]))
    lq = DR.log_softmax(np.array([[np.log(3.0), 0.0]]))  # q = (3/4, 1/4)
    # KL((1/2, 1/2) || (3/4, 1/4)) = 1/2 ln(2/3) + 1/2 ln 2
    np.testing.assert_allclose(DR.kl(lp, lq), [0.5 * np.log(2 / 3) + 0.5 * np.log(2)], rtol=1e-12)
    np.testing.assert_allclose(DR.tv(lp, lq), [0.25], rtol=1e-12)
    np.testing.assert_allclose(DR.kl(lp, lp), [0.0], atol=1e-15)
    big = DR.log_softmax(np.array([[60.0, -60.0]]))
    other = DR.log_softmax(np.array([[-60.0, 60.0]]))
    np.testing.assert_allclose(DR.tv(big, other), [1.0], atol=1e-12)


def test_prefix_agreement_brute_force():
    rng = np.random.default_rng(1)
    for _ in range(20):
        ref = rng.integers(0, 3, size=(9, 4))
        tok = rng.integers(0, 3, size=(9, 4))
        want = [np.mean([all(tok[b, :k + 1] == ref[b, :k + 1]) for b in range(9)]) for k in range(4)]
        np.testing.assert_allclose(DR.prefix_agreement(tok, ref), want)
    # the ceiling is the mean of the prefix agreements (E[len] = sum_k P(len >= k))
    np.testing.assert_allclose(DR.prefix_agreement(tok, ref).sum(), O.accept_len(tok, ref).mean())


def test_identical_passes_give_perfect_metrics():
    wl = C.CFG1.replace(kv_lens=(40, 9), fixture_gains=True)
    ref = DR.oracle_pass(wl, gen.make_weights(wl), gen.make_inputs(wl))
    m = DR.metrics(ref, ref, ref)
    assert m["ceiling"] == 7 and m["greedy"] == 1 and m["sequential"] == [1.0] * 7
    assert m["kl_mean"] == 0 and m["tv_coupling"] == 1 and m["hidden_rel"] == 0 and m["flip_rate"] == 0
    assert m["conf_r"] == pytest.approx(1.0)


@pytest.mark.parametrize("dist", ["gauss", "heavy"])
def test_oracle_bf16_weights_drift_against_fp32(dist):
    """Quantising the tiny drafter's weights to bf16 moves it only slightly."""
    wl32 = C.CFG1.replace(kv_lens=(40, 9, 100, 1), captured_dist=dist)
    wlq = wl32.replace(formats=dataclasses.replace(C.ALL_BF16, kv_cache=C.F32, captured=C.F32))
    inputs = gen.make_inputs(wl32)
    ref = DR.oracle_pass(wl32, gen.make_weights(wl32), inputs)
    sq = gen.make_weights(wlq)
    free = DR.oracle_pass(wlq, sq, inputs)
    forced = DR.oracle_pass(wlq, sq, inputs, forced=ref["tokens"])
    m = DR.metrics(ref, free, forced)
    print(DR.fmt_row(f"oracle bf16 weights {dist}", m))
    assert 0 <= m["ceiling"] <= 7 and 0 < m["hidden_rel"] < 0.05 and m["kl_mean"] >= 0
    assert m["greedy"] >= 0.5 and m["tv_coupling"] > 0.9
