"""The candidate rollout of the Markov head (greedy passes without logits or
hidden outputs): only rows whose Cauchy-Schwarz upper bound reaches the
largest lower bound are evaluated (huggingface.co "Kimi-K3-DSpark-NVFP4",
original card, "Model Overview": the sequential low-rank Markov head).

* It drafts the full rollout's tokens: at the first position where the two
  differ (if any), the full rollout's own logits must hold a rounding tie
  between the two picks (the paths sum W2 u in different orders); the
  confidences agree to rounding.
* The Markov-dominant fixture (lm_head = 0, so every row is a candidate)
  takes the fallback: status 0 and the full rollout's bits.
* Poisoned workspaces give the same bits.
* The bench workload (full Q8_0, context 8192) takes the candidate path.
* The batched FP8 workload (16 sequences) has a vocabulary chunk with more
  rows above its own lower bound than the chunk's slots hold (14 > 8, while
  at most 8 per position pass the position's threshold): the chunk is
  rescanned and the candidate path still drafts the full rollout's tokens.
"""
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


def _run(g, full, forced=None, poison=None):
    m = g.wl.model
    n, B = g.wl.n_seq, m.block
    tokens = torch.full((n, B), -7, dtype=torch.int32, device="cuda")
    conf = torch.full((n, B), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.full((1,), -3, dtype=torch.int32, device="cuda")
    logits = torch.empty((n, B, m.vocab), dtype=torch.float32, device="cuda") if full else None
    if poison is not None:
        g.ws.view(torch.uint8).fill_(poison)
    fp = None if forced is None else torch.from_numpy(np.asarray(forced, np.int32)).cuda()
    g.model.draft_block(g.cap, g.kv, g.offs, g.prev, g.wl.total_ctx, tokens, conf, g.ws, logits=logits,
                        forced_prev=fp, status=status, page_size=g.page_size, block_table=g.table)
    torch.cuda.synchronize()
    out = dict(tokens=tokens.cpu().numpy(), conf=conf.cpu().numpy(), status=int(status.item()))
    if full:
        out["logits"] = logits.cpu().numpy()
    return out


def _check_same_draft(full, pr, rtol=2e-6):
    n, B = full["tokens"].shape
    for s in range(n):
        for i in range(B):
            a, b = int(full["tokens"][s, i]), int(pr["tokens"][s, i])
            if a != b:
                lg = full["logits"][s, i].astype(np.float64)
                assert abs(lg[a] - lg[b]) <= rtol * np.max(np.abs(lg)), (s, i, a, b, lg[a], lg[b])
                break   # later positions have other predecessors
            assert abs(float(full["conf"][s, i]) - float(pr["conf"][s, i])) <= 1e-6, (s, i)


WLS = {
    "small_bs1": C.Workload("prune_bs1", C.small_model(), C.ALL_BF16, seed=1601, kv_lens=(300,), fixture_gains=True),
    "small_3seq": C.Workload("prune_3seq", C.small_model(), C.Q8, seed=1602, kv_lens=(0, 37, 300), fixture_gains=True),
    "tiny_bf16": C.CFG1.replace(fixture_gains=True, formats=C.Formats(fc="f32", q_a="f32", q_b="f32", kv_b="f32",
                                                                       o="f32", mlp="f32", lm_head="f32",
                                                                       markov="bf16", kv_cache="f32", captured="f32")),
}


@pytest.mark.parametrize("name", list(WLS))
def test_candidate_rollout_matches_full(name):
    from tests.gpu_common import GpuWorkload
    g = GpuWorkload(WLS[name])
    full = _run(g, True)
    pr = _run(g, False)
    assert full["status"] == 0
    assert pr["status"] == 2, "the candidate rollout did not run"
    _check_same_draft(full, pr)
    # teacher forcing: every position independent, same predecessors
    ff = _run(g, True, forced=full["tokens"])
    fp = _run(g, False, forced=full["tokens"])
    assert fp["status"] == 2
    _check_same_draft(ff, fp)
    # poisoned workspaces: the same bits
    for pat in (0xFF, 0x3C):
        again = _run(g, False, poison=pat)
        np.testing.assert_array_equal(again["tokens"], pr["tokens"])
        np.testing.assert_array_equal(again["conf"].view(np.int32), pr["conf"].view(np.int32))


def test_markov_dominant_falls_back():
    """lm_head = 0: every row stays a candidate, so the full rollout runs and
    the outputs are its bits (with or without the logits output)."""
    from tests.gpu_common import GpuWorkload
    wl = C.Workload("prune_dom", C.small_model(), C.ALL_BF16, seed=1603, kv_lens=(0, 37, 300),
                    fixture_gains=True, markov_dominant=True)
    g = GpuWorkload(wl)
    full = _run(g, True)
    pr = _run(g, False)
    assert pr["status"] == 0, "expected the fallback to the full rollout"
    np.testing.assert_array_equal(pr["tokens"], full["tokens"])
    np.testing.assert_array_equal(pr["conf"].view(np.int32), full["conf"].view(np.int32))


def test_bench_workload_takes_the_candidate_path():
    from tests.gpu_common import GpuWorkload
    g = GpuWorkload(C.CFG3)
    full = _run(g, True)
    pr = _run(g, False)
    assert pr["status"] == 2
    _check_same_draft(full, pr)


def test_batched_workload_rescans_overflowing_chunks():
    from tests.gpu_common import GpuWorkload
    g = GpuWorkload(C.CFG5)
    full = _run(g, True)
    pr = _run(g, False)
    assert pr["status"] == 2, "expected the candidate path"
    _check_same_draft(full, pr)
