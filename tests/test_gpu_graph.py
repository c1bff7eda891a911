"""The draft pass captured in a HIP graph (as a serving loop or the benchmark
replays it) gives bit-identical outputs on every replay, with eager passes on
other inputs and synchronisations between the replays.  The pass zeroes its
scratch with a kernel (no memset node enters the graph)."""
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


@pytest.mark.parametrize("wl", [C.Workload("graph_small_q8", C.small_model(), C.Q8, seed=1201, kv_lens=(0, 37, 300),
                                           fixture_gains=True),
                                C.Workload("graph_small_bs1_mx", C.small_model(), C.MX4, seed=1202, kv_lens=(77,),
                                           fixture_gains=True),
                                C.CFG3], ids=lambda w: w.name)
def test_graph_replays_match_eager(wl):
    from tests.gpu_common import GpuWorkload
    g = GpuWorkload(wl)
    m = wl.model
    n, B = wl.n_seq, m.block
    tokens = torch.empty((n, B), dtype=torch.int32, device="cuda")
    conf = torch.empty((n, B), dtype=torch.float32, device="cuda")
    logits = torch.empty((n, B, m.vocab), dtype=torch.float32, device="cuda")

    def run():
        g.model.draft_block(g.cap, g.kv, g.offs, g.prev, wl.total_ctx, tokens, conf, g.ws, logits=logits)

    run()
    torch.cuda.synchronize()
    want = (tokens.cpu().numpy().copy(), conf.cpu().numpy().copy(), logits.cpu().numpy().copy())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    other_prev = torch.remainder(g.prev + 17, m.vocab).to(torch.int32)
    for rep in range(4):
        # eager work on other inputs between replays, then clear the outputs
        g.model.draft_block(g.cap, g.kv, g.offs, other_prev, wl.total_ctx, tokens, conf, g.ws, logits=logits)
        torch.cuda.synchronize()
        tokens.fill_(-1)
        conf.fill_(float("nan"))
        logits.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(tokens.cpu().numpy(), want[0], err_msg=f"replay {rep}")
        np.testing.assert_array_equal(conf.cpu().numpy().view(np.uint32), want[1].view(np.uint32))
        np.testing.assert_array_equal(logits.cpu().numpy().view(np.uint32), want[2].view(np.uint32))
    print(wl.name, "tokens", want[0].tolist()[0], flush=True)
