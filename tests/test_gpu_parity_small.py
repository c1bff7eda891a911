"""GPU parity at sizes the oracle finishes in seconds: the tiny all-fp32
drafter, a ragged mid-size geometry (hidden 352, vocab 1000, inter 480,
v_head 24, three sequences with cache lengths 0 / 37 / 300) in every weight
format, the same geometry with the full model's MLA head sizes, plus decoding
and acceptance checks."""
import itertools

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


def _gw(wl):
    from tests.gpu_common import GpuWorkload
    return GpuWorkload(wl)


SMALL = C.small_model()
FORMATS = {
    "bf16": C.ALL_BF16,
    "q8_0": C.Q8,
    "fp8": C.FP8_PC,
    "mxfp4": C.MX4,
    "f32w_bf16kv": C.Formats(fc="f32", q_a="f32", q_b="f32", kv_b="f32", o="f32", mlp="f32",
                              lm_head="f32", markov="f32"),
}


def test_tiny_f32_exact_tokens():
    """The tiny all-fp32 drafter: tokens exact (no near-ties), fp32 tolerance."""
    from tests.gpu_common import full_parity
    wl = C.CFG1.replace(fixture_gains=True)
    g = _gw(wl)
    ref = O.draft_block(wl, g.stored, g.inputs)
    print("tiny ref tokens", ref["tokens"].tolist(), flush=True)
    out, free, ties = full_parity(g, ref, tol=1e-4, max_ties=0)
    np.testing.assert_array_equal(free["tokens"], ref["tokens"])
    np.testing.assert_array_equal(out["tokens"], ref["tokens"])


def test_tiny_metric_config_and_markov_dominant():
    from tests.gpu_common import full_parity
    for wl in (C.CFG1, C.CFG1.replace(markov_dominant=True, fixture_gains=True)):
        g = _gw(wl)
        ref = O.draft_block(wl, g.stored, g.inputs)
        out, free, ties = full_parity(g, ref, tol=1e-4, max_ties=0)
        np.testing.assert_array_equal(free["tokens"], ref["tokens"])


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_small_ragged_all_formats(fmt):
    from tests.gpu_common import full_parity
    wl = C.Workload(f"small_{fmt}", SMALL, FORMATS[fmt], seed=777, kv_lens=(0, 37, 300),
                    fixture_gains=True)
    g = _gw(wl)
    ref = O.draft_block(wl, g.stored, g.inputs)
    out, free, ties = full_parity(g, ref, tol=2e-2, max_ties=2)
    print(fmt, "near-ties", ties, flush=True)


@pytest.mark.parametrize("fmt", ["q8_0", "bf16", "fp8", "mxfp4"])
def test_small_bs1_formats(fmt):
    """One sequence (7 activation rows): the hi/lo activation paths, including
    the int8 MFMA path of Q8_0 weights."""
    from tests.gpu_common import full_parity
    wl = C.Workload(f"small_bs1_{fmt}", SMALL, FORMATS[fmt], seed=779, kv_lens=(77,), fixture_gains=True)
    g = _gw(wl)
    ref = O.draft_block(wl, g.stored, g.inputs)
    full_parity(g, ref, tol=2e-2, max_ties=1)


# The full model's MLA head geometry (qk_nope 128, qk_rope 64, kv_lora 512)
# with the other sizes small: one sequence (7 rows) takes the per-head fused
# q_b + absorb kernel with Q8_0 q_b weights and the fused post + absorb with
# bf16 ones; three sequences (21 rows) the split-K q_b GEMM.
MLA_MID = C.small_model(n_heads=4, q_lora=256, kv_lora=512, qk_nope=128, qk_rope=64, v_head=128)


@pytest.mark.parametrize("fmt", ["q8_0", "bf16"])
@pytest.mark.parametrize("lens", [(77,), (0, 37, 300)])
def test_mla_head_geometry(fmt, lens):
    from tests.gpu_common import full_parity
    wl = C.Workload(f"mla_mid_{fmt}", MLA_MID, FORMATS[fmt], seed=781, kv_lens=lens, fixture_gains=True)
    print("case", fmt, lens, flush=True)
    g = _gw(wl)
    ref = O.draft_block(wl, g.stored, g.inputs)
    full_parity(g, ref, tol=2e-2, max_ties=2)


MLA_WIDE = C.small_model(n_heads=16, q_lora=256, kv_lora=512, qk_nope=128, qk_rope=64, v_head=128)


@pytest.mark.parametrize("lens", [(300,), (0, 37, 600)])
def test_mla_head_geometry_sharp(lens):
    """The full model's latent and head sizes with 16 heads (112 query rows:
    two groups of 64 per attention workgroup grid) and W_UK scaled x10, so
    the scores span several units: probabilities formed against different
    reference maxima would show."""
    from tests.gpu_common import full_parity
    wl = C.Workload("mla_wide_sharp", MLA_WIDE, C.ALL_BF16, seed=783, kv_lens=lens, fixture_gains=True,
                    sharp_attention=True)
    print("case", lens, flush=True)
    g = _gw(wl)
    ref = O.draft_block(wl, g.stored, g.inputs)
    full_parity(g, ref, tol=2e-2, max_ties=2)


def test_small_sharp_attention_bf16():
    from tests.gpu_common import full_parity
    wl = C.Workload("small_sharp", SMALL, C.ALL_BF16, seed=778, kv_lens=(129,), fixture_gains=True,
                    sharp_attention=True)
    g = _gw(wl)
    ref = O.draft_block(wl, g.stored, g.inputs)
    full_parity(g, ref, tol=2e-2, max_ties=2)


def test_small_far_dominant_key_bf16():
    """One cache row scaled x200 far from the first key tile of its slot: its
    scores exceed the slot's first-tile maximum by far more than 60, so the
    attention workgroup takes its exact-reference second pass."""
    from tests.gpu_common import full_parity
    wl = C.Workload("small_spike", SMALL, C.ALL_BF16, seed=780, kv_lens=(300,), fixture_gains=True,
                    spike=(200, 200.0))
    g = _gw(wl)
    ref = O.draft_block(wl, g.stored, g.inputs)
    full_parity(g, ref, tol=2e-2, max_ties=2)


def test_dequant_bit_exact():
    """Decoding the repacked planes gives exactly the oracle's decoded values
    (Q8_0 d*q, MXFP4 X*e2m1(q) and bf16 exact in fp32; FP8 s*e4m3(q)
    correctly rounded)."""
    from mla_block_drafter_amd import dspark as D
    for fmt, names in [("q8_0", ["L0.q_b", "L1.o", "L0.down", "fc"]), ("fp8", ["L0.q_b", "L1.down", "fc"]),
                       ("mxfp4", ["L0.q_b", "L1.o", "L1.down", "fc"]),
                       ("bf16", ["lm_head", "L0.o", "markov_w2"]), ("f32w_bf16kv", ["L0.o", "lm_head"])]:
        wl = C.Workload("deq", SMALL, FORMATS[fmt], seed=31, kv_lens=(5,))
        g = _gw(wl)
        for name in names:
            st = g.stored[name]
            rows, cols = st.shape
            out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
            g.model.dequant(name, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            want = codecs.decode(st).astype(np.float32)   # exact for q8_0 / bf16 / f32; RNE for fp8
            np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32), err_msg=f"{fmt} {name}")
        # fused gate/up and q_a/kv_a decode as stacked rows
        out = torch.empty((2 * SMALL.inter, SMALL.hidden), dtype=torch.float32, device="cuda")
        g.model.dequant("L0.gate", out)
        torch.cuda.synchronize()
        want = np.concatenate([codecs.decode(g.stored["L0.gate"]), codecs.decode(g.stored["L0.up"])])
        np.testing.assert_array_equal(out.cpu().numpy(), want.astype(np.float32))


def test_accept_len_device_brute_force():
    from mla_block_drafter_amd import dspark as D
    for alpha, blk in [(3, 4), (2, 7)]:
        seqs = np.array(list(itertools.product(range(alpha), repeat=blk)), dtype=np.int32)
        rng = np.random.default_rng(blk)
        d = seqs[rng.integers(0, len(seqs), size=len(seqs))]
        dt, vt = torch.from_numpy(d).cuda(), torch.from_numpy(seqs).cuda()
        out = torch.empty(len(seqs), dtype=torch.int32, device="cuda")
        D.accept_len(dt, vt, out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), O.accept_len(d, seqs))
    # planted first mismatch
    d = np.random.default_rng(0).integers(0, 163840, size=(8, 7)).astype(np.int32)
    v = gen.planted_verifier(d, np.arange(8, dtype=np.int32), np.full(8, 5, np.int32), 163840)
    out = torch.empty(8, dtype=torch.int32, device="cuda")
    D.accept_len(torch.from_numpy(d).cuda(), torch.from_numpy(v).cuda(), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), np.arange(8))


def test_determinism_bitwise():
    wl = C.Workload("small_det", SMALL, C.Q8, seed=9, kv_lens=(300, 11), fixture_gains=True)
    g = _gw(wl)
    a = g.draft()
    b = g.draft()
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_determinism_interleaved_workloads():
    """Passes of three different workloads interleaved (different geometries
    and kernels run in between, leaving other data in LDS, registers, the
    caches and the workspaces' previous owners): every repeat of a workload
    reproduces its first pass bit for bit, greedy and sampled, packed and
    paged."""
    from tests.gpu_common import GpuWorkload
    wa = C.Workload("det_a", SMALL, C.ALL_BF16, seed=1103, kv_lens=(0, 37, 300), fixture_gains=True)
    wb = C.Workload("det_b", C.small_model(hidden=256, vocab=777), C.Q8, seed=31, kv_lens=(129,))
    wc = C.CFG1.replace(fixture_gains=True)
    ga, gb, gc = GpuWorkload(wa), GpuWorkload(wb), GpuWorkload(wc)
    m = wa.model
    u = torch.from_numpy(np.random.default_rng(8).uniform(1e-6, 1 - 1e-6, (wa.n_seq, m.block, m.vocab))
                         .astype(np.float32)).cuda()

    def sampled(g):
        tokens = torch.empty((wa.n_seq, m.block), dtype=torch.int32, device="cuda")
        conf = torch.empty((wa.n_seq, m.block), dtype=torch.float32, device="cuda")
        g.model.draft_block(g.cap, g.kv, g.offs, g.prev, wa.total_ctx, tokens, conf, g.ws, sample_u=u,
                            temperature=0.8, page_size=g.page_size, block_table=g.table)
        torch.cuda.synchronize()
        return dict(tokens=tokens.cpu().numpy(), conf=conf.cpu().numpy())

    first = {}
    for rep in range(4):
        runs = [("a", ga.draft), ("b", gb.draft), ("as", lambda: sampled(ga)), ("c", gc.draft)]
        if rep == 2:
            ga.use_pages(64, seed=3)   # same rows, paged: same bits
        for name, fn in (runs if rep % 2 == 0 else runs[::-1]):
            out = fn()
            if name not in first:
                first[name] = out
                continue
            for k in out:
                np.testing.assert_array_equal(np.ascontiguousarray(out[k]).view(np.uint8),
                                              np.ascontiguousarray(first[name][k]).view(np.uint8),
                                              err_msg=f"{name} repeat {rep}: {k}")
