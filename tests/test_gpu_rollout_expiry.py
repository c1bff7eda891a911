"""The Markov rollout's bounded wait, forced to expire from the host
(dspark_block_in.poll_limit < 0: no wait at all).  Every kernel must finish
normally, every token of the call must be -1 and the status output 1; the
next call on the same workspace, with the default bound, must give the normal
draft again (status 0, tokens and confidences equal to a call that never
expired).  Teacher-forced rollouts poll nothing, so they never expire."""
import dataclasses

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


def _call(g, poll_limit, forced=None):
    m = g.wl.model
    n, B = g.wl.n_seq, m.block
    tokens = torch.full((n, B), -7, dtype=torch.int32, device="cuda")
    conf = torch.full((n, B), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.full((1,), -3, dtype=torch.int32, device="cuda")
    fp = None if forced is None else torch.from_numpy(np.asarray(forced, np.int32)).cuda()
    g.model.draft_block(g.cap, g.kv, g.offs, g.prev, g.wl.total_ctx, tokens, conf, g.ws, forced_prev=fp,
                        status=status, poll_limit=poll_limit)
    torch.cuda.synchronize()
    return tokens.cpu().numpy(), conf.cpu().numpy(), int(status.item())


@pytest.mark.parametrize("wl", [
    C.Workload("expiry_small", C.small_model(), C.ALL_BF16, seed=1401, kv_lens=(0, 37, 300), fixture_gains=True),
    C.CFG1.replace(fixture_gains=True, formats=dataclasses.replace(C.ALL_F32, markov=C.BF16)),
], ids=["small_bf16_3seq", "tiny_bf16_markov"])
def test_forced_expiry_is_loud_and_harmless(wl):
    from tests.gpu_common import GpuWorkload
    g = GpuWorkload(wl)
    t0, c0, s0 = _call(g, 0)
    assert s0 in (0, 2) and (t0 >= 0).all()   # 2: drafted by the candidate rollout
    t1, c1, s1 = _call(g, -1)
    assert s1 == 1
    assert (t1 == -1).all(), t1
    assert np.isfinite(c1).all()
    t2, c2, s2 = _call(g, 0)
    assert s2 == s0
    np.testing.assert_array_equal(t2, t0)
    np.testing.assert_array_equal(c2.view(np.int32), c0.view(np.int32))
    # a generous explicit bound: the full rollout, the same draft (up to
    # rounding ties against the candidate rollout, none in these fixtures)
    t3, c3, s3 = _call(g, 1 << 20)
    assert s3 == 0
    np.testing.assert_array_equal(t3, t0)
    # teacher forcing: positions are independent, nothing is polled
    t4, c4, s4 = _call(g, -1, forced=t0)
    assert s4 == 0
    np.testing.assert_array_equal(t4, t0)
