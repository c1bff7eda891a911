"""Probabilistic drafting and block / token verification on the GPU against
the oracle (huggingface.co "Kimi-K3-DSpark-NVFP4", "Sampling options").

Drafting: the GPU's sampled tokens equal the oracle's Gumbel-max draws from the
same uniforms, except at a certified near-tie of the perturbed scores (as for
greedy tokens).  Verification: accepted lengths and next tokens equal the
oracle's on logits whose decisions all clear a margin of 1e-3 (inputs drawn
until they do), so float32 and float64 take the same decisions."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import dspark as O, verify as VF
from synth import configs as C, gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mla_block_drafter_amd import dspark as D
    D.lib()


def _uniforms(shape, seed):
    u = np.random.default_rng(seed).random(shape, dtype=np.float32)
    return np.clip(u, np.float32(1e-7), np.float32(1 - 1e-7))


def _check_sampled(tok_g, log_g, log_r, u, T, max_ties):
    ties = 0
    n, B, V = log_r.shape
    for s in range(n):
        for i in range(B):
            sel_r = log_r[s, i] / T + O.gumbel(u[s, i])
            sel_g = np.asarray(log_g[s, i], np.float64) / T + O.gumbel(u[s, i])
            t_r = int(np.argmax(sel_r))
            if tok_g[s, i] != t_r:
                delta = float(np.max(np.abs(sel_g - sel_r)))
                assert sel_r[t_r] - sel_r[tok_g[s, i]] <= 2 * delta + 1e-5 * np.max(np.abs(sel_r)), (s, i)
                ties += 1
                break  # later positions follow a different predecessor
    assert ties <= max_ties
    return ties


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_sampled_draft_small(T):
    from tests.gpu_common import GpuWorkload
    wl = C.Workload("sample_small", C.small_model(), C.Q8, seed=1101, kv_lens=(0, 37, 300), fixture_gains=True)
    g = GpuWorkload(wl)
    m = wl.model
    u = _uniforms((wl.n_seq, m.block, m.vocab), 5)
    du = torch.from_numpy(u).cuda()
    n, B = wl.n_seq, m.block
    tokens = torch.empty((n, B), dtype=torch.int32, device="cuda")
    conf = torch.empty((n, B), dtype=torch.float32, device="cuda")
    logits = torch.empty((n, B, m.vocab), dtype=torch.float32, device="cuda")
    g.model.draft_block(g.cap, g.kv, g.offs, g.prev, wl.total_ctx, tokens, conf, g.ws, logits=logits,
                        sample_u=du, temperature=T)
    torch.cuda.synchronize()
    ref = O.draft_block(wl, g.stored, g.inputs, sample_u=u, temperature=T)
    ties = _check_sampled(tokens.cpu().numpy(), logits.cpu().numpy(), ref["logits"], u, T, max_ties=1)
    # sampling differs from the greedy draft somewhere (the uniforms matter)
    greedy = g.draft()["tokens"]
    assert not np.array_equal(greedy, tokens.cpu().numpy())
    print("T", T, "sampled", tokens.cpu().numpy().tolist(), "ties", ties, flush=True)


def test_sampled_draft_full_size_teacher_forced():
    """Full Q8_0 geometry (ctx 8192): with the oracle's greedy tokens as
    predecessors the logits do not depend on the uniforms, so they match the
    stored oracle values; the sampled token is the Gumbel-max pick of the
    GPU's own logits (up to a 1e-5 relative near-tie of the scores)."""
    import os
    from tests.gpu_common import GpuWorkload
    path = os.path.join(os.path.dirname(__file__), "golden", "pass_cfg3.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    gold = np.load(path)
    wl = C.CFG3
    m = wl.model
    g = GpuWorkload(wl)
    g.stored = None
    T = 0.7
    u = _uniforms((1, m.block, m.vocab), 6)
    du = torch.from_numpy(u).cuda()
    tokens = torch.empty((1, m.block), dtype=torch.int32, device="cuda")
    conf = torch.empty((1, m.block), dtype=torch.float32, device="cuda")
    logits = torch.empty((1, m.block, m.vocab), dtype=torch.float32, device="cuda")
    fp = torch.from_numpy(np.asarray(gold["tokens"], np.int32)).cuda()
    g.model.draft_block(g.cap, g.kv, g.offs, g.prev, wl.total_ctx, tokens, conf, g.ws, logits=logits,
                        forced_prev=fp, sample_u=du, temperature=T)
    torch.cuda.synchronize()
    lg_all, tok = logits.cpu().numpy(), tokens.cpu().numpy()
    greedy = 0
    for i in range(m.block):
        idx = np.concatenate([gold["top_idx"][0, i], gold["smp_idx"][0, i]])
        ref = np.concatenate([gold["top_val"][0, i], gold["smp_val"][0, i]])
        lg = lg_all[0, i]
        assert np.max(np.abs(lg[idx].astype(np.float64) - ref)) <= 1e-2 * gold["logit_absmax"][0, i], i
        sel = lg.astype(np.float64) / T + O.gumbel(u[0, i])
        t = int(tok[0, i])
        assert sel.max() - sel[t] <= 1e-5 * np.max(np.abs(sel)), (i, t, int(np.argmax(sel)))
        greedy += t == int(np.argmax(lg))
    print("sampled", tok.tolist(), "greedy picks", greedy, flush=True)
    assert greedy < m.block  # the draw is not the argmax everywhere


def test_sampling_bad_arguments():
    from mla_block_drafter_amd import dspark as D
    from tests.gpu_common import GpuWorkload
    wl = C.Workload("sample_bad", C.small_model(), C.Q8, seed=1102, kv_lens=(20,))
    g = GpuWorkload(wl)
    m = wl.model
    du = torch.full((1, m.block, m.vocab), 0.5, dtype=torch.float32, device="cuda")
    tokens = torch.empty((1, m.block), dtype=torch.int32, device="cuda")
    conf = torch.empty((1, m.block), dtype=torch.float32, device="cuda")
    for T in (0.0, -1.0, float("nan")):
        with pytest.raises(D.DsparkError):
            g.model.draft_block(g.cap, g.kv, g.offs, g.prev, wl.total_ctx, tokens, conf, g.ws, sample_u=du,
                                temperature=T)
    B, V = 4, 50
    d = torch.zeros((2, B), dtype=torch.int32, device="cuda")
    dl = torch.zeros((2, B, V), dtype=torch.float32, device="cuda")
    tl = torch.zeros((2, B + 1, V), dtype=torch.float32, device="cuda")
    uu = torch.full((2, B + 1), 0.51, dtype=torch.float32, device="cuda")
    ol = torch.empty(2, dtype=torch.int32, device="cuda")
    ot = torch.empty(2, dtype=torch.int32, device="cuda")
    with pytest.raises(D.DsparkError):
        D.verify(d, dl, tl, uu, 1.0, 7, ol, ot)
    with pytest.raises(D.DsparkError):
        D.verify(d, dl, tl, uu, 0.0, D.VERIFY_BLOCK, ol, ot)
    # identical draft and target: everything accepted under both rules
    for meth in (D.VERIFY_TOKEN, D.VERIFY_BLOCK):
        D.verify(d, dl, torch.zeros((2, B + 1, V), dtype=torch.float32, device="cuda"), uu, 1.0, meth, ol, ot)
        torch.cuda.synchronize()
        assert ol.cpu().tolist() == [B, B] and ot.cpu().tolist() == [V // 2, V // 2]


def _margins_ok(draft, dl, tl, r, T, method):
    """All decisions of the oracle clear 1e-3 (acceptance tests and the draw)."""
    B = len(draft)
    q, p = VF.softmax_t(dl, T), VF.softmax_t(tl, T)
    if method == "token":
        tau, _ = VF.token_verify(draft, q, p, r[:B], r[B])
        for i in range(min(tau + 1, B)):
            if abs(r[i] - min(1.0, p[i, draft[i]] / q[i, draft[i]])) < 1e-3:
                return False
        res = np.maximum(p[tau] - q[tau], 0.0) if tau < B else p[B]
    else:
        tau, _ = VF.block_verify(draft, q, p, r[:B], r[B])
        w = VF.block_weights(draft, q, p)
        for k in range(1, B + 1):
            if k < B:
                S = np.maximum(w[k] * p[k] - q[k], 0.0).sum()
                h = S / (S + 1 - w[k]) if S + 1 - w[k] > 0 else 1.0
            else:
                h = w[B]
            if abs(r[k - 1] - h) < 1e-3:
                return False
        res = np.maximum(w[tau] * p[tau] - q[tau], 0.0) if tau < B else p[B]
    c = np.cumsum(res) / res.sum()
    return np.min(np.abs(c - r[B])) > 1e-3


@pytest.mark.parametrize("method", ["token", "block"])
@pytest.mark.parametrize("V", [1000, 163840])
def test_verify_matches_oracle(method, V):
    from mla_block_drafter_amd import dspark as D
    n, B, T = 6, 7, 0.8
    rng = np.random.default_rng(V + (method == "block"))
    drafts, dls, tls, us = [], [], [], []
    while len(drafts) < n:
        dl = (2.0 * rng.standard_normal((B, V))).astype(np.float32)
        # the target agrees with the draft up to noise of varying size, so acceptance lengths spread
        tl = (dl[np.r_[0:B, B - 1]] + rng.uniform(0.0, 1.5) * rng.standard_normal((B + 1, V))).astype(np.float32)
        q = VF.softmax_t(dl, T)
        draft = np.array([VF.inverse_cdf(q[i], rng.random()) for i in range(B)], np.int32)
        r = rng.random(B + 1).astype(np.float32)
        if _margins_ok(draft, np.asarray(dl, np.float64), np.asarray(tl, np.float64), np.asarray(r, np.float64),
                       T, method):
            drafts.append(draft), dls.append(dl), tls.append(tl), us.append(r)
    d = torch.from_numpy(np.stack(drafts)).cuda()
    dl = torch.from_numpy(np.stack(dls)).cuda()
    tl = torch.from_numpy(np.stack(tls)).cuda()
    u = torch.from_numpy(np.stack(us)).cuda()
    out_len = torch.full((n,), -5, dtype=torch.int32, device="cuda")
    out_tok = torch.full((n,), -5, dtype=torch.int32, device="cuda")
    D.verify(d, dl, tl, u, T, D.VERIFY_TOKEN if method == "token" else D.VERIFY_BLOCK, out_len, out_tok)
    torch.cuda.synchronize()
    fn = VF.token_verify if method == "token" else VF.block_verify
    lens = []
    for s in range(n):
        q = VF.softmax_t(np.asarray(dls[s], np.float64), T)
        p = VF.softmax_t(np.asarray(tls[s], np.float64), T)
        tau, y = fn(drafts[s], q, p, np.asarray(us[s][:B], np.float64), float(us[s][B]))
        assert int(out_len[s]) == tau and int(out_tok[s]) == y, (s, int(out_len[s]), tau, int(out_tok[s]), y)
        lens.append(tau)
    print(method, V, "accepted", lens, flush=True)


@pytest.mark.parametrize("method", ["token", "block"])
def test_verify_single_token_blocks(method):
    """Blocks of one drafted token (the degenerate block length) over five
    sequences: the same decisions as the oracle."""
    from mla_block_drafter_amd import dspark as D
    n, B, T, V = 5, 1, 1.0, 1000
    rng = np.random.default_rng(77 + (method == "block"))
    drafts, dls, tls, us = [], [], [], []
    while len(drafts) < n:
        dl = (2.0 * rng.standard_normal((B, V))).astype(np.float32)
        tl = (dl[np.r_[0:B, B - 1]] + rng.uniform(0.0, 2.0) * rng.standard_normal((B + 1, V))).astype(np.float32)
        q = VF.softmax_t(dl, T)
        draft = np.array([VF.inverse_cdf(q[0], rng.random())], np.int32)
        r = rng.random(B + 1).astype(np.float32)
        if _margins_ok(draft, np.asarray(dl, np.float64), np.asarray(tl, np.float64), np.asarray(r, np.float64),
                       T, method):
            drafts.append(draft), dls.append(dl), tls.append(tl), us.append(r)
    out_len = torch.full((n,), -5, dtype=torch.int32, device="cuda")
    out_tok = torch.full((n,), -5, dtype=torch.int32, device="cuda")
    D.verify(torch.from_numpy(np.stack(drafts)).cuda(), torch.from_numpy(np.stack(dls)).cuda(),
             torch.from_numpy(np.stack(tls)).cuda(), torch.from_numpy(np.stack(us)).cuda(), T,
             D.VERIFY_TOKEN if method == "token" else D.VERIFY_BLOCK, out_len, out_tok)
    torch.cuda.synchronize()
    fn = VF.token_verify if method == "token" else VF.block_verify
    for s in range(n):
        tau, y = fn(drafts[s], VF.softmax_t(np.asarray(dls[s], np.float64), T),
                    VF.softmax_t(np.asarray(tls[s], np.float64), T), np.asarray(us[s][:B], np.float64), float(us[s][B]))
        assert (int(out_len[s]), int(out_tok[s])) == (tau, y), s


def test_sampled_draft_paged_matches_packed():
    """Sampling over page pools draws exactly the packed pass's tokens and
    confidences, bit for bit; the workspace is NaN-filled before each pass, so
    a read of memory the pass has not written cannot go unnoticed."""
    from tests.gpu_common import GpuWorkload
    wl = C.Workload("sample_paged", C.small_model(), C.ALL_BF16, seed=1103, kv_lens=(0, 37, 300), fixture_gains=True)
    g = GpuWorkload(wl)
    m = wl.model
    du = torch.from_numpy(_uniforms((wl.n_seq, m.block, m.vocab), 8)).cuda()
    outs = []
    for paged in (False, True):
        if paged:
            g.use_pages(64, seed=3)
        tokens = torch.empty((wl.n_seq, m.block), dtype=torch.int32, device="cuda")
        conf = torch.empty((wl.n_seq, m.block), dtype=torch.float32, device="cuda")
        g.ws.fill_(0xFF)
        g.model.draft_block(g.cap, g.kv, g.offs, g.prev, wl.total_ctx, tokens, conf, g.ws, sample_u=du,
                            temperature=0.8, page_size=g.page_size, block_table=g.table)
        torch.cuda.synchronize()
        outs.append((tokens.cpu().numpy(), conf.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[1][1].view(np.int32), outs[0][1].view(np.int32))
