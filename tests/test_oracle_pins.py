"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests compares the oracle with a re-typed copy of itself:
  * hand-derived exact cases (tests/golden/hand_exact.json);
  * the lossless theorem of speculative sampling (ReSpec notes, '2 . background':
    the marginal of every emitted token equals the target distribution; NeMo RL
    post, 'lossless'): chi-square of emitted tokens against p over 10^6 trials at
    V <= 8;
  * closed forms: P(accepted_len >= i) = prod_{l<i} sum_x min(p_l, q_l), and the
    residual distribution max(0,p-q)/sum max(0,p-q) conditioned on a rejection;
  * greedy verification as the T -> 0 limit of sampling;
  * power-of-two temperature scaling, which is exact in binary;
  * normaliser closed forms and an exactly rounded (math.fsum) log-sum-exp;
  * top-32 against a brute-force lexicographic sort on tie-heavy rows.
"""
import math

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import sv_inputs
import golden_cases

CASES = golden_cases.load()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_exact(oracle_mod, case):
    w = golden_cases.workload(case)
    got = oracle_mod.verify_workload(w)
    golden_cases.check(case, got)


def _fixed_logits(seed, k, V, sigma_d):
    rng = np.random.default_rng(seed)
    t = rng.standard_normal((k + 1, V)).astype(np.float32)
    d = (t[:k] + sigma_d * rng.standard_normal((k, V))).astype(np.float32)
    return t, d


@pytest.mark.parametrize("V,T,seed", [(8, 1.0, 11), (6, 0.8, 12)])
def test_lossless_marginal_and_closed_forms(oracle_mod, V, T, seed):
    k, N = 3, 10 ** 6
    t, d = _fixed_logits(seed, k, V, 0.8)
    w = sv_inputs.fixed_rows(N, t, d, T, seed)
    r = oracle_mod.verify_workload(w, aux=False)
    assert (r.status == 0).all()
    p = softmax(t.astype(np.float64) / T, axis=1)
    q = softmax(d.astype(np.float64) / T, axis=1)
    beta = np.minimum(p[:k], q).sum(axis=1)
    n_tests = 2 * (k + 1) + k
    alpha = 1e-4 / n_tests
    acc = r.accepted_len
    for i in range(k + 1):
        # emitted token at position i, among sequences that reached position i
        reach = acc >= i
        counts = np.bincount(r.out_tokens[reach, i], minlength=V)
        assert counts.sum() == reach.sum()
        _, pv = stats.chisquare(counts, p[i] * reach.sum())
        assert pv > alpha, (i, pv)
        # P(reach i) = prod_{l<i} beta_l (binomial z-score)
        pr = float(np.prod(beta[:i]))
        z = (reach.sum() - N * pr) / math.sqrt(N * pr * (1 - pr) + 1e-300)
        assert abs(z) < 5.0, (i, z)
    for i in range(k):
        # token drawn at the first rejection follows the residual
        rej = acc == i
        res = np.maximum(p[i] - q[i], 0.0)
        res /= res.sum()
        counts = np.bincount(r.out_tokens[rej, i], minlength=V)
        keep = res > 0
        assert counts[~keep].sum() == 0           # zero residual mass is never drawn
        _, pv = stats.chisquare(counts[keep], res[keep] * rej.sum())
        assert pv > alpha, ("residual", i, pv)


def test_chi_square_detects_a_wrong_residual(oracle_mod):
    """Power check: the marginal test rejects the draft distribution q in place
    of p at the same sample size, so a sign slip in the residual would fail."""
    V, k, N, T = 8, 3, 10 ** 6, 1.0
    t, d = _fixed_logits(11, k, V, 0.8)
    w = sv_inputs.fixed_rows(N, t, d, T, 11)
    r = oracle_mod.verify_workload(w, aux=False)
    q = softmax(d.astype(np.float64) / T, axis=1)
    counts = np.bincount(r.out_tokens[:, 0], minlength=V)
    _, pv = stats.chisquare(counts, q[0] * N)
    assert pv < 1e-12


def _gapped_rows(rng, n, V, gap):
    x = rng.standard_normal((n, V)).astype(np.float32)
    top = rng.integers(0, V, n)
    x[np.arange(n), top] = x.max(axis=1) + np.float32(gap)
    return x


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_greedy_is_the_zero_temperature_limit(oracle_mod, seed):
    """With a unique maximum at least 0.1 above the rest, T=1e-4 makes every
    non-maximal exp((t-m)/T) underflow to 0 in fp64: sampling must then equal
    the T=0 argmax-prefix match bit for bit, whatever the uniforms."""
    rng = np.random.default_rng(seed)
    B, k, V = 64, 3, 257
    t = _gapped_rows(rng, B * (k + 1), V, 0.25).reshape(B, k + 1, V)
    d = _gapped_rows(rng, B * k, V, 0.25).reshape(B, k, V)
    # half the drafts agree with the target argmax, so accept chains vary
    agree = rng.random((B, k)) < 0.6
    d_arg = d.argmax(axis=2)
    t_arg = t[:, :k].argmax(axis=2)
    tokens = np.where(agree, t_arg, d_arg).astype(np.int32)
    # the drafter puts its own top on the drafted token
    for b in range(B):
        for i in range(k):
            x = tokens[b, i]
            d[b, i, x] = d[b, i].max() + np.float32(0.25)
    u = rng.random((B, k + 2)).astype(np.float32)
    greedy = oracle_mod.verify(t, None, tokens, None, 0.0, 0)
    cold = oracle_mod.verify(t, d, tokens, u, 1e-4, 0)
    assert (greedy.status == 0).all() and (cold.status == 0).all()
    np.testing.assert_array_equal(greedy.accepted_len, cold.accepted_len)
    np.testing.assert_array_equal(greedy.out_tokens, cold.out_tokens)
    assert 0 < greedy.accepted_len.mean() < k


def test_temperature_power_of_two_scaling(oracle_mod):
    """softmax(t / (1/2)) == softmax(2t / 1) exactly in binary arithmetic."""
    w = sv_inputs.tiny(seed=31, B=16)
    half = oracle_mod.verify(w.target, w.draft, w.draft_tokens, w.uniforms, 0.5, 0)
    dbl = oracle_mod.verify(w.target * np.float32(2), w.draft * np.float32(2), w.draft_tokens, w.uniforms, 1.0, 0)
    for key in ("accepted_len", "out_tokens", "margin_accept", "margin_cdf", "p_tok", "q_tok", "lse_target"):
        np.testing.assert_array_equal(half[key], dbl[key], err_msg=key)
    # temperature matters: T=1 on the unscaled rows gives other draws
    one = oracle_mod.verify(w.target, w.draft, w.draft_tokens, w.uniforms, 1.0, 0)
    assert not np.array_equal(one.p_tok, half.p_tok)


def test_lse_closed_forms(oracle_mod):
    V, k = 1000, 1
    for c, T in ((0.0, 1.0), (2.5, 0.5), (-7.0, 2.0)):
        t = np.full((1, k + 1, V), c, np.float32)
        r = oracle_mod.verify(t, t[:, :k].copy(), np.zeros((1, k), np.int32), np.zeros((1, k + 2), np.float32), T, 0)
        want = c / T + math.log(V)
        np.testing.assert_allclose(r.lse_target[0], want, rtol=1e-14)
        np.testing.assert_allclose(r.p_tok[0], 1.0 / V, rtol=1e-14)
    # half the row at c, half at c - ln 3: s = V/2 (1 + 1/3) relative to the max
    t = np.zeros((1, 2, 1000), np.float32)
    t[..., 500:] = np.float32(-math.log(3.0))
    r = oracle_mod.verify(t, t[:, :1].copy(), np.zeros((1, 1), np.int32), np.zeros((1, 3), np.float32), 1.0, 0)
    lnthird = float(np.float32(-math.log(3.0)))
    np.testing.assert_allclose(r.lse_target[0], math.log(500 + 500 * math.exp(lnthird)), rtol=1e-14)


def test_lse_against_exact_summation(oracle_mod):
    w = sv_inputs.steady(B=1, seed=41)
    r = oracle_mod.verify_workload(w)
    T = w.temperature
    for i in range(w.k + 1):
        row = w.target_f32()[0, i].astype(np.float64)
        m = row.max()
        want = m / T + math.log(math.fsum(math.exp((v - m) / T) for v in row))
        assert abs(r.lse_target[0, i] - want) <= 1e-12 * abs(want)


@pytest.mark.parametrize("seed,V", [(51, 5000), (52, 151936), (53, 40)])
def test_top32_brute_force_with_ties(oracle_mod, seed, V):
    rng = np.random.default_rng(seed)
    # small-integer logits, rounded to bf16: heavy ties at every rank
    x = np.round(rng.standard_normal((1, 3, V)) * 4).astype(np.float32)
    x[0, 1, rng.integers(0, V, 7)] = -0.0
    x[0, 2, rng.integers(0, V, V // 3)] = -np.inf
    h = sv_inputs.bf16_round(x)
    r = oracle_mod.verify(h, None, np.zeros((1, 2), np.int32), None, 0.0, 1)
    xf = sv_inputs.bf16_to_f32(h)
    for i in range(3):
        row = xf[0, i].astype(np.float64) + 0.0       # -0.0 + 0.0 == +0.0: ties by index
        order = np.lexsort((np.arange(V), -row))[:32]
        n = min(32, V)
        assert r.topk_idx[0, i, :n].tolist() == order[:n].tolist()
        assert np.array_equal(r.topk_val[0, i, :n].view(np.uint32), xf[0, i, order[:n]].view(np.uint32))


def test_oracle_is_deterministic(oracle_mod):
    w = sv_inputs.tiny(seed=61, B=8)
    a = oracle_mod.verify_workload(w)
    b = oracle_mod.verify_workload(w)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_acceptance_statistics_match_closed_form(oracle_mod):
    """2048 sequences of the steady-state value distribution (V cut to 4096,
    drafts drawn from q): for each position i the number of sequences that
    reach it, and the total accepted length, against the closed forms
    P(accepted_len >= i) = prod_{l<i} beta_l with beta_l = sum_x min(p_l, q_l)
    on each sequence's own rows (Leviathan et al.'s acceptance rate, which the
    ReSpec notes' Eq.1 test implies), as z-scores with exact variances."""
    w = sv_inputs.steady(B=2048, V=4096, seed=71)
    r = oracle_mod.verify_workload(w, aux=False)
    assert (r.status == 0).all()
    k, T = w.k, w.temperature
    p = softmax(w.target_f32()[:, :k].astype(np.float64) / T, axis=2)
    q = softmax(w.draft_f32().astype(np.float64) / T, axis=2)
    beta = np.minimum(p, q).sum(axis=2)                                   # [B, k]
    reach = np.concatenate([np.ones((w.B, 1)), np.cumprod(beta, axis=1)], axis=1)   # P(acc >= i), i = 0..k
    acc = r.accepted_len
    for i in range(1, k + 1):
        P = reach[:, i]
        z = ((acc >= i).sum() - P.sum()) / math.sqrt((P * (1 - P)).sum())
        assert abs(z) < 5.0, (i, z)
    pm = reach[:, :k + 1] - np.concatenate([reach[:, 1:], np.zeros((w.B, 1))], axis=1)   # P(acc = m)
    m = np.arange(k + 1)
    mean = (pm * m).sum(axis=1)
    var = (pm * m * m).sum(axis=1) - mean ** 2
    z = (acc.sum() - mean.sum()) / math.sqrt(var.sum())
    assert abs(z) < 5.0, z
    assert 0.5 < mean.mean() < k - 0.5                      # the test has power: chains of every length
