"""Pins of the distillation oracle (oracle/kd_oracle.c) against what the pages
and the mathematics fix: the pages' two worked examples (tests/golden), KL(pt || q)
against scipy's relative-entropy routine on the zero-padded soft target, the
gradient against central differences of an independent loss, the invariants
(KL >= 0, KL = 0 when q equals the soft target, gradient rows summing to 0),
clipping, and the data-error rows."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import sv_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "kd_worked_examples.json")


def _row_with_kl(kl, V=64):
    """Stored ids 0..31 with equal values (uniform soft target) and drafter
    logits a on them, 0 elsewhere: KL = -ln M with M = e^a / (e^a + 1), the
    drafter mass on the stored ids.  KL = 0 takes -inf elsewhere instead."""
    z = np.zeros(V, np.float32)
    if kl == 0:
        z[32:] = -np.inf
    else:
        M = math.exp(-kl)
        z[:32] = np.float32(math.log(M / (1 - M)))
    return z, np.zeros(32, np.float32), np.arange(32, dtype=np.int32)


def test_single_sample_worked_example(oracle_mod):
    g = json.load(open(GOLD))["single_sample"]
    rows = [_row_with_kl(k) for k in g["kl_terms"]]
    z = np.stack([r[0] for r in rows])
    tv = np.stack([r[1] for r in rows])
    ti = np.stack([r[2] for r in rows])
    # a group whose rewards sum to 1 leaves the reward itself as the weight
    rewards = np.array([g["reward"], 1 - g["reward"]], np.float32)
    r = oracle_mod.kd(z, tv, ti, np.zeros(3, np.int32), rewards, group=2)
    np.testing.assert_allclose(r.kl, g["kl_terms"], atol=1e-7)
    assert abs(r.weight[0] - g["reward"]) < 1e-7
    assert abs(r.loss - g["loss"]) < 1e-7


def test_grpo_group_worked_example(oracle_mod):
    g = json.load(open(GOLD))["grpo_group"]
    rw = np.array(g["rewards"], np.float32)
    z, tv, ti = _row_with_kl(0.4)                    # the example's KL of about 0.4 per completion
    n = len(rw)
    r = oracle_mod.kd(np.stack([z] * n), np.stack([tv] * n), np.stack([ti] * n), np.arange(n, dtype=np.int32), rw,
                      group=n)
    for i, w in g["weights_rounded"].items():
        assert round(float(r.weight[int(i)]), 2) == w
    np.testing.assert_allclose(r.weight, rw.astype(np.float64) / rw.astype(np.float64).sum(), rtol=1e-15)
    for i in g["zero_weight"]:
        assert r.weight[i] == 0 and not r.grad[i].any()
    np.testing.assert_allclose(r.loss, (r.weight * r.kl).sum(), rtol=1e-14)


def _scipy_kl(z, tv, ti):
    q = scipy.special.softmax(z.astype(np.float64))
    pt = np.zeros_like(q)
    pt[ti] = scipy.special.softmax(tv.astype(np.float64))
    return scipy.stats.entropy(pt, q)


@pytest.mark.parametrize("dtype", [sv_inputs.F32, sv_inputs.BF16])
def test_kl_matches_scipy_relative_entropy(oracle_mod, dtype):
    w = sv_inputs.kd_workload("pin", 6, 3, 2, 300, dtype, 7)
    r = oracle_mod.kd_workload(w)
    zf = w.logits if dtype == sv_inputs.F32 else sv_inputs.bf16_to_f32(w.logits)
    for n in range(w.N):
        assert abs(r.kl[n] - _scipy_kl(zf[n], w.topk_val[n], w.topk_idx[n])) < 1e-12
        assert r.kl[n] > 0


def test_gradient_is_the_derivative_of_the_loss(oracle_mod):
    """Central differences of an independent fp64 loss (scipy softmax and
    relative entropy) at fp64 points: the oracle's gradient formula must match."""
    rng = np.random.default_rng(3)
    V = 40
    z = (rng.standard_normal(V) * 2).astype(np.float32)
    ids = rng.choice(V, 32, replace=False).astype(np.int32)
    tv = (rng.standard_normal(32) + 2).astype(np.float32)
    rewards = np.array([0.8, 0.2], np.float32)
    r = oracle_mod.kd(z[None], tv[None], ids[None], np.zeros(1, np.int32), rewards, group=2)
    w = 0.8
    h = 1e-5
    for x in range(V):
        zp = z.astype(np.float64).copy()
        zm = zp.copy()
        zp[x] += h
        zm[x] -= h
        fd = w * (_scipy_kl(zp, tv, ids) - _scipy_kl(zm, tv, ids)) / (2 * h)
        assert abs(fd - r.grad[0, x]) < 1e-8, x
    assert abs(r.grad.sum()) < 1e-15 * V * 10


def test_zero_kl_when_drafter_matches(oracle_mod):
    z, tv, ti = _row_with_kl(0)
    r = oracle_mod.kd(z[None], tv[None], ti[None], np.zeros(1, np.int32), np.ones(1, np.float32), group=1)
    assert r.kl[0] == 0.0 and r.loss == 0.0
    assert np.all(r.grad == 0)


def test_clip_and_empty_group(oracle_mod):
    z, tv, ti = _row_with_kl(0.5)
    rw = np.array([1.0, 0.0, 0.0, 0.0], np.float32)     # group 0: weights 1, 0; group 1: sum 0
    r = oracle_mod.kd(np.stack([z] * 4), np.stack([tv] * 4), np.stack([ti] * 4), np.arange(4, dtype=np.int32), rw,
                      group=2, w_max=0.25)
    np.testing.assert_array_equal(r.weight, [0.25, 0.0, 0.0, 0.0])
    np.testing.assert_allclose(r.loss, 0.25 * 0.5, rtol=1e-6)


def test_error_rows(oracle_mod):
    z, tv, ti = _row_with_kl(0.3)
    Z = np.stack([z] * 7)
    TV = np.stack([tv] * 7)
    TI = np.stack([ti] * 7)
    Z[0, 5] = np.nan                              # NaN drafter logit
    TI[1, 3] = 64                                 # stored id out of range
    Z[2, :] = -np.inf                             # empty drafter row
    TV[3, :] = -np.inf                            # no stored entry
    TV[4, 3] = np.inf                             # +inf stored value
    rs = np.array([0, 0, 0, 0, 0, 7, 0], np.int32)   # row 5: sample id out of range
    TI[6, 20] = TI[6, 4]                          # row 6: one id in two stored entries
    r = oracle_mod.kd(Z, TV, TI, rs, np.ones(2, np.float32), group=2)
    K = oracle_mod
    np.testing.assert_array_equal(r.status, [K.KD_NAN, K.KD_BAD_INDEX, K.KD_EMPTY, K.KD_EMPTY, K.KD_POSINF,
                                             K.KD_BAD_INDEX, K.KD_DUP_INDEX])
    assert np.all(np.isnan(r.kl)) and r.loss == 0.0 and not r.grad.any()
    # padding entries (value -inf or id -1) carry no weight and are no error
    TV2 = tv.copy()
    TI2 = ti.copy()
    TV2[5] = -np.inf
    TI2[6] = -1
    TI2[5] = TI2[7]                               # a padding entry may repeat a used id
    r2 = oracle_mod.kd(z[None], TV2[None], TI2[None], np.zeros(1, np.int32), np.ones(1, np.float32), group=1)
    used = np.ones(32, bool)
    used[[5, 6]] = False
    assert r2.status[0] == 0
    assert abs(r2.kl[0] - _scipy_kl(z, tv[used], ti[used])) < 1e-12
