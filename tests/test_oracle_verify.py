"""Probabilistic drafting and verification in the oracle (huggingface.co
"Kimi-K3-DSpark-NVFP4", "Sampling options"): the Gumbel-max draw follows
softmax(l / T), and both verifiers (token by token, block as a unit) leave
the target's distribution unchanged, pinned by sampling against the exact
target joint distribution on a small vocabulary, plus exact special cases."""
import itertools

import numpy as np
import pytest

from oracle import dspark as O, verify as VF


def test_gumbel_max_draws_follow_the_tempered_softmax():
    rng = np.random.default_rng(3)
    l, T, N = np.array([0.3, -1.0, 1.2, 0.0]), 0.7, 200_000
    u = rng.random((N, 4))
    counts = np.bincount(np.argmax(l / T + O.gumbel(u), axis=1), minlength=4) / N
    want = VF.softmax_t(l, T)
    assert np.all(np.abs(counts - want) < 5 * np.sqrt(want * (1 - want) / N)), (counts, want)


def _tables(rng, V, B, sharp):
    """Random prefix-dependent distributions of a draft and a target model."""
    tab = {}
    for n in range(B + 1):
        for pre in itertools.product(range(V), repeat=n):
            tab[pre] = (VF.softmax_t(sharp * rng.standard_normal(V), 1.0),
                        VF.softmax_t(sharp * rng.standard_normal(V), 1.0))
    return tab  # prefix -> (draft q, target p)


@pytest.mark.parametrize("verifier", ["token", "block"])
@pytest.mark.parametrize("B", [2, 3])
def test_verifiers_preserve_the_target_distribution(verifier, B):
    V, N = 3, 60_000
    rng = np.random.default_rng(10 + B)
    tab = _tables(rng, V, B, 1.5)
    fn = VF.token_verify if verifier == "token" else VF.block_verify
    counts = {}
    acc = 0
    for _ in range(N):
        x = []
        for i in range(B):
            x.append(int(rng.choice(V, p=tab[tuple(x)][0])))
        q = np.stack([tab[tuple(x[:i])][0] for i in range(B)])
        p = np.stack([tab[tuple(x[:i])][1] for i in range(B + 1)])
        tau, y = fn(x, q, p, rng.random(B), rng.random())
        acc += tau
        seq = x[:tau] + [y]
        while len(seq) < B + 1:  # continue with the target
            seq.append(int(rng.choice(V, p=tab[tuple(seq)][1])))
        counts[tuple(seq)] = counts.get(tuple(seq), 0) + 1
    for seq in itertools.product(range(V), repeat=B + 1):
        want = np.prod([tab[seq[:j]][1][seq[j]] for j in range(B + 1)])
        got = counts.get(seq, 0) / N
        assert abs(got - want) < 5 * np.sqrt(want * (1 - want) / N) + 1e-4, (seq, got, want)
    print(verifier, B, "mean accepted", acc / N)


def test_block_accepts_at_least_as_much_as_token_on_average():
    V, B, N = 3, 3, 40_000
    rng = np.random.default_rng(7)
    tab = _tables(rng, V, B, 1.0)
    tot = {"token": 0, "block": 0}
    for _ in range(N):
        x = []
        for i in range(B):
            x.append(int(rng.choice(V, p=tab[tuple(x)][0])))
        q = np.stack([tab[tuple(x[:i])][0] for i in range(B)])
        p = np.stack([tab[tuple(x[:i])][1] for i in range(B + 1)])
        r, u = rng.random(B), rng.random()
        tot["token"] += VF.token_verify(x, q, p, r, u)[0]
        tot["block"] += VF.block_verify(x, q, p, r, u)[0]
    assert tot["block"] >= tot["token"] - 3 * np.sqrt(N), tot


def test_verifier_special_cases():
    V, B = 5, 4
    rng = np.random.default_rng(1)
    p = VF.softmax_t(rng.standard_normal((B + 1, V)), 1.0)
    draft = [1, 4, 0, 2]
    for fn in (VF.token_verify, VF.block_verify):
        # identical draft and target distributions: everything is accepted
        tau, y = fn(draft, p[:B].copy(), p, np.full(B, 0.999), 0.5)
        assert tau == B and y == VF.inverse_cdf(p[B], 0.5)
        # a draft token the target never emits is rejected at once
        p0 = p.copy()
        p0[0, 1] = 0.0
        p0[0] /= p0[0].sum()
        tau, y = fn(draft, p[:B].copy(), p0, np.zeros(B), 0.3)
        assert tau == 0 and y != 1
    assert VF.inverse_cdf(np.array([0.0, 1.0, 1.0]), 0.0) == 1
    assert VF.inverse_cdf(np.array([1.0, 1.0]), 0.5) == 1
