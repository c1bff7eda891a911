"""Pins of the oracle's building blocks: closed forms, library routines,
invariants, special cases and brute force."""
import itertools
import math

import numpy as np
import pytest
import scipy.special as sps
import torch
import torch.nn.functional as F

from oracle import dspark as O
from synth import configs as C


# --------------------------------------------------------------- norms ----
def test_rmsnorm_vs_torch_and_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 96))
    g = rng.uniform(0.5, 1.5, 96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rmsnorm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-15)
    c = np.full(64, -3.0)                       # constant row -> -g * 3/sqrt(9+eps)
    np.testing.assert_allclose(O.rmsnorm(c, np.ones(64), 1e-6), -3 / math.sqrt(9 + 1e-6))
    np.testing.assert_allclose(O.rmsnorm(5 * x, g, 0.0), O.rmsnorm(x, g, 0.0), rtol=1e-13)


def test_activations_vs_library():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(O.sigmoid(x), sps.expit(x), rtol=1e-13)
    s = np.random.default_rng(1).standard_normal((3, 4, 50)) * 20
    np.testing.assert_allclose(O.softmax(s), sps.softmax(s, axis=-1), rtol=1e-12)


# ---------------------------------------------------------------- rope ----
def _cfg(**kw):
    return C.small_model(**kw)


def test_rope_identities():
    m = _cfg(yarn_factor=1.0)
    f = O.rope_frequencies(m)
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(16), rng.standard_normal(16)
    np.testing.assert_allclose(O.rope(q, 0, f), q)                                  # pos 0
    np.testing.assert_allclose(np.linalg.norm(O.rope(q, 1234, f)), np.linalg.norm(q))
    d1 = O.rope(q, 40, f) @ O.rope(k, 33, f)
    d2 = O.rope(q, 1007, f) @ O.rope(k, 1000, f)                                     # same offset
    np.testing.assert_allclose(d1, d2, rtol=1e-10)
    # consecutive pairs rotate like complex numbers x0 + i x1 times e^{i p theta}
    z = (q[0::2] + 1j * q[1::2]) * np.exp(1j * 77 * f)
    r = O.rope(q, 77, f)
    np.testing.assert_allclose(r[0::2] + 1j * r[1::2], z, rtol=1e-12)
    np.testing.assert_allclose(f, 10000.0 ** (-np.arange(8) / 8))                   # base 1e4


def test_yarn_frequencies_limits():
    for m in (C.FULL, C.small_model(yarn_factor=4.0, yarn_orig_ctx=2048)):
        s = m.yarn_factor
        plain = O.rope_frequencies(m.__class__(**{**m.__dict__, "yarn_factor": 1.0}))
        yarn = O.rope_frequencies(m)
        r = m.yarn_orig_ctx * plain / (2 * math.pi)
        hi, lo = r > 32, r < 1
        mid = ~hi & ~lo
        assert hi.any() and mid.any()
        np.testing.assert_allclose(yarn[hi], plain[hi])                  # gamma = 1: unchanged
        np.testing.assert_allclose(yarn[lo], plain[lo] / s)              # gamma = 0: f / s
        assert np.all((yarn[mid] < plain[mid]) & (yarn[mid] > plain[mid] / s))
    assert lo.any()
    assert O.yarn_logit_scale(C.FULL) == pytest.approx(1.63139, abs=5e-6)
    assert O.yarn_logit_scale(C.TINY) == 1.0


@pytest.mark.parametrize("k", [3, 7, 11])
def test_yarn_ramp_interior(k):
    """Inside the band alpha < r_k < beta the NTK-by-parts ramp is linear in
    the rotation count r_k (YaRN paper, Peng et al. 2023): the pair whose
    window holds exactly (alpha + beta) / 2 rotations gets the mean of the
    interpolated and the original frequency, and the pair at alpha + (beta -
    alpha) / 4 rotations three quarters interpolated, one quarter original.
    The original window is chosen so that pair k sits at that point; a log
    ramp, swapped alpha / beta roles or swapped f / (f / s) roles each move
    one of the two points."""
    base = C.FULL
    d, s = base.qk_rope, base.yarn_factor
    alpha, beta = base.yarn_beta_slow, base.yarn_beta_fast
    theta_k = base.rope_theta ** (-2.0 * k / d)
    for frac, want_interp in ((0.5, 0.5), (0.25, 0.75)):
        r_k = alpha + frac * (beta - alpha)
        L = 2 * math.pi * r_k / theta_k                    # window with r_k rotations at pair k
        m = C.ModelConfig(**{**base.__dict__, "yarn_orig_ctx": L})
        f = O.rope_frequencies(m)
        want = want_interp * theta_k / s + (1 - want_interp) * theta_k
        assert f[k] == pytest.approx(want, rel=1e-12), (k, frac)
        # pairs below / above in index sit at more / fewer rotations: the
        # ramp is monotone and the endpoints are reached outside the band
        assert f[k - 1] / (base.rope_theta ** (-2.0 * (k - 1) / d)) > f[k] / theta_k


# ----------------------------------------------------------- acceptance ----
def test_accept_len_brute_force():
    for alpha, blk in [(3, 1), (3, 2), (3, 3), (3, 4), (3, 5), (2, 7)]:
        seqs = np.array(list(itertools.product(range(alpha), repeat=blk)))
        for d in seqs:
            got = O.accept_len(np.broadcast_to(d, seqs.shape), seqs)
            want = np.array([next((k for k in range(blk) if d[k] != v[k]), blk) for v in seqs])
            np.testing.assert_array_equal(got, want)


def test_accept_len_planted():
    rng = np.random.default_rng(4)
    d = rng.integers(0, 163840, size=(8, 7))
    for k in range(8):
        v = d.copy()
        if k < 7:
            v[:, k] += 1
        assert (O.accept_len(d, v) == k).all()


# ------------------------------------------------------------- argmax ------
def test_argmax_ties_lowest():
    v = np.zeros(4096)
    v[[17, 900, 4000]] = 3.0
    assert O.argmax_lowest(v) == 17 == int(np.argmax(v))
    assert O.argmax_lowest(-np.ones(5)) == 0


# ------------------------------------------------- throughput closed form ---
def test_throughput_printed_break_even():
    """huggingface.co "Kimi-K3-DSpark-NVFP4", "Considerations": acceptance
    ratio 3.29 / 5.70 = 0.577, so a 1.73x draft speedup is needed to break even;
    with d_nvfp4 = 0.81 d_fp8 the factor tops out at 1.23; with d_nvfp4 =
    0.5 d_fp8 break-even needs d_fp8 >= 5.5 T; at d/T = 0.14 the draft win is
    (1 + 0.14) / (1 + 0.81 * 0.14) = 1.024 (printed as "~1.03x")."""
    a_nv, a_fp8 = 3.29, 5.70
    assert round(a_nv / a_fp8, 3) == 0.577
    assert round(a_fp8 / a_nv, 2) == 1.73
    big = 1e9
    assert round(O.throughput_ratio(1, 1, 0.81 * big, big, 1.0), 2) == 1.23
    # break-even d with d_nv = 0.5 d: (a_nv/a_fp8) * (d + T) / (0.5 d + T) = 1
    T = 1.0
    d_star = (a_fp8 / a_nv - 1) * T / (1 - 0.5 * a_fp8 / a_nv)
    assert round(d_star, 1) == 5.5
    assert O.throughput_ratio(a_nv, a_fp8, 0.5 * d_star, d_star, T) == pytest.approx(1.0)
    assert O.throughput_ratio(1, 1, 0.81 * 0.14, 0.14, 1.0) == pytest.approx(1.0239, abs=1e-4)
    assert O.throughput(3, 1, 2) == 1.0


# -------------------------------------------------------- size arithmetic ---
def _params(m, conf_plain=False):
    names = C.tensor_names(m)
    n = 0
    for nm in names:
        shp = C.tensor_shape(m, nm)
        if nm == "conf_w" and conf_plain:
            shp = (m.hidden,)
        n += int(np.prod(shp))
    return n - m.vocab * m.hidden  # the lm_head is the target's, not the drafter's


def test_full_geometry_reproduces_printed_sizes():
    """alphaneural.io card: GGUF without embed_tokens "2.4B params (4.45 GB)",
    original with the 1.17B embedding "4B params (7.12 GB)"; huggingface.co
    card: "2.19 B of 3.56 B params quantized (61%)", BF16 6.6 GiB, FP8 4.6 GiB."""
    m = C.FULL
    p = _params(m, conf_plain=True)
    assert p == 2_387_907_585
    assert round(2 * p / 2 ** 30, 2) == 4.45
    embed = m.vocab * m.hidden
    assert round(embed / 1e9, 2) == 1.17
    tot = p + embed
    assert round(tot / 1e9, 2) == 3.56 and round(2 * tot / 1e9, 2) == 7.12
    assert round(2 * tot / 2 ** 30, 1) == 6.6
    quant = sum(int(np.prod(C.tensor_shape(m, nm))) for nm in C.tensor_names(m)
                if nm.split(".")[-1] in ("fc", "q_b", "o", "gate", "up", "down"))
    assert quant == 2_186_280_960 and round(quant / 1e9, 2) == 2.19
    assert round(100 * quant / tot) == 61
    rows = sum(C.tensor_shape(m, nm)[0] for nm in C.tensor_names(m)
               if nm.split(".")[-1] in ("fc", "q_b", "o", "gate", "up", "down"))
    fp8 = quant + 4 * rows + 2 * (tot - quant)
    assert round(fp8 / 2 ** 30, 1) == 4.6
