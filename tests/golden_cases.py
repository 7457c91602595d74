"""Loader for the hand-derived cases in tests/golden/hand_exact.json."""
import json
import os

import numpy as np

from sv_inputs import F32, Workload

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_exact.json")
_SPECIAL = {"-inf": -np.inf, "inf": np.inf, "nan": np.nan, "-0.0": -0.0, "0.0": 0.0}


def fval(v):
    return _SPECIAL[v] if isinstance(v, str) else float(v)


def farr(rows):
    return np.array([[fval(v) for v in r] for r in rows], dtype=np.float32)


def load():
    with open(_PATH) as f:
        return json.load(f)["cases"]


def workload(case) -> Workload:
    """The case as a B=1 fp32 Workload (draft/uniforms zero-filled when greedy)."""
    k, V, T = case["k"], case["V"], float(case["T"])
    target = farr(case["target"]).reshape(1, k + 1, V)
    draft = farr(case["draft"]).reshape(1, k, V) if "draft" in case else np.zeros((1, k, V), np.float32)
    tokens = np.array(case["draft_tokens"], np.int32).reshape(1, k)
    u = np.array(case.get("uniforms", [0.0] * (k + 2)), np.float32).reshape(1, k + 2)
    return Workload(case["name"], 1, k, V, F32, T, target, draft, tokens, u)


def check(case, got, sampling_aux=True):
    """Compare a result dict (numpy arrays, B=1) with the case's expectations."""
    e = case["expect"]
    name = case["name"]
    assert int(got["accepted_len"][0]) == e["accepted_len"], name
    assert got["out_tokens"][0].tolist() == e["out_tokens"], name
    assert int(got["status"][0]) == e["status"], name
    for r in range(case["k"] + 1):
        if f"topk_idx_row{r}" in e:
            want_i = e[f"topk_idx_row{r}"]
            want_v = np.array([fval(v) for v in e[f"topk_val_row{r}"]], np.float32)
            n = len(want_i)
            assert got["topk_idx"][0, r, :n].tolist() == want_i, name
            gv = got["topk_val"][0, r, :n]
            assert np.array_equal(np.isnan(gv), np.isnan(want_v)), name
            ok = ~np.isnan(want_v)
            # compare bit patterns so that -0.0 and +0.0 are told apart
            assert np.array_equal(gv[ok].view(np.uint32), want_v[ok].view(np.uint32)), name
    if not sampling_aux:
        return
    for key in ("p_tok", "q_tok", "margin_accept", "lse_target", "lse_draft"):
        if key in e and key in got:
            np.testing.assert_allclose(got[key][0][: len(e[key])], e[key], rtol=1e-15, atol=0, err_msg=name)
    if "margin_cdf" in e and "margin_cdf" in got:
        assert float(got["margin_cdf"][0]) == e["margin_cdf"], name
