"""The GPU-vs-oracle comparator itself (tests/compare.py), on hand-made
results: a difference at an unflagged decision fails, one at a flagged
decision is an exception counted by position, and relative errors treat any
disagreement in finiteness as infinite."""
import math

import numpy as np

from compare import compare_decisions, compare_topk, rel_err


def _orc(acc, out, margin_accept, margin_cdf, status=None):
    B = len(acc)
    return dict(accepted_len=np.array(acc), out_tokens=np.array(out), margin_accept=np.array(margin_accept, float),
                margin_cdf=np.array(margin_cdf, float), status=np.zeros(B, int) if status is None else np.array(status))


def _gpu(acc, out, status=None):
    B = len(acc)
    return dict(accepted_len=np.array(acc), out_tokens=np.array(out),
                status=np.zeros(B, int) if status is None else np.array(status))


def test_identical_results_pass():
    o = _orc([1, 0], [[5, 7], [3, -1]], [[-0.5], [0.2]], [0.3, 0.1])
    rep = compare_decisions(o, _gpu([1, 0], [[5, 7], [3, -1]]), 1)
    assert rep == dict(fails=[], exc_seq=0, exc_pos=0, positions=4)


def test_acceptance_difference_flagged_or_not():
    o = _orc([1], [[5, 7]], [[-3e-6]], [0.3])                 # the oracle accepted draft 0 by 3e-6
    g = _gpu([0], [[9, -1]])
    rep = compare_decisions(o, g, 1)
    assert not rep["fails"] and rep["exc_seq"] == 1 and rep["exc_pos"] == 2
    o = _orc([1], [[5, 7]], [[-3e-4]], [0.3])                 # by 3e-4: a real disagreement
    assert len(compare_decisions(o, g, 1)["fails"]) == 1


def test_draw_difference_flagged_or_not():
    o = _orc([0], [[4, -1]], [[0.5]], [2e-6])
    g = _gpu([0], [[5, -1]])
    rep = compare_decisions(o, g, 1)
    assert not rep["fails"] and rep["exc_pos"] == 1
    o = _orc([0], [[4, -1]], [[0.5]], [0.2])
    assert len(compare_decisions(o, g, 1)["fails"]) == 1


def test_status_difference_fails():
    o = _orc([-1], [[-1, -1]], [[math.nan]], [math.nan], status=[2])
    assert compare_decisions(o, _gpu([-1], [[-1, -1]], status=[0]), 1)["fails"]


def test_topk_bits():
    v = np.array([[[1.0, -0.0]]], np.float32)
    i = np.array([[[3, 4]]], np.int32)
    bad, ok = compare_topk(dict(topk_val=v, topk_idx=i), dict(topk_val=v.copy(), topk_idx=i.copy()))
    assert len(bad) == 0 and ok
    v2 = v.copy()
    v2[0, 0, 1] = 0.0                                           # +0 for -0: different bits
    assert not compare_topk(dict(topk_val=v, topk_idx=i), dict(topk_val=v2, topk_idx=i))[1]


def test_rel_err_finiteness():
    nan, inf = np.nan, np.inf
    assert rel_err([1.0, nan], [1.0, nan]) == 0.0
    assert rel_err([1.0, inf], [1.0, inf]) == 0.0
    assert rel_err([1.0, 2.0], [1.0, nan]) == inf
    assert rel_err([1.0, nan], [1.0, 2.0]) == inf
    assert rel_err([1.0, inf], [1.0, -inf]) == inf
    assert rel_err([1.0, inf], [1.0, nan]) == inf
    assert abs(rel_err([2.0, 4.0], [2.002, 4.0]) - 1e-3) < 1e-12
