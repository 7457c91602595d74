"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: accepted_len, out_tokens and top-32 indices identical except decisions the
oracle flags within 1e-5 of their boundary (under 0.1% of positions); top-32
values bit-exact; p_tok/q_tok/lse within 1e-5 relative for fp32 inputs and 2e-3
for bf16 inputs; greedy bit-exact.
"""
import os
import sys

import numpy as np
import pytest

import sv_inputs
import golden_cases
from compare import FLAG, compare_decisions, compare_topk, gpu_to_numpy, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def log(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import draft_verification_spec_amd as m
    m.load_library()      # raises when the HIP library was not built
    return m


@pytest.fixture(scope="module")
def orc(oracle_mod):
    return oracle_mod


def run_gpu(sv, w, aux=True):
    log(f"spec_verify {w.name} B={w.B} k={w.k} V={w.V} dtype={sv_inputs.DTYPE_NAME[w.dtype]} T={w.temperature}")
    t, d, x, u = sv.to_device(w)
    greedy = w.temperature == 0
    r = sv.verify(t, None if greedy else d, x, None if greedy else u, w.temperature, aux=aux)
    torch.cuda.synchronize()
    return gpu_to_numpy(r)


def check_parity(orc_res, gpu, w):
    k = w.k
    rep = compare_decisions(orc_res, gpu, k)
    assert not rep["fails"], rep["fails"][:5]
    # flagged exceptions: under 0.1% of the call's positions B(k+1)
    assert rep["exc_pos"] <= 0.001 * rep["positions"], rep
    bad_idx, vals_ok = compare_topk(orc_res, gpu)
    assert len(bad_idx) == 0, bad_idx[:5]
    assert vals_ok
    if w.temperature > 0 and gpu.get("p_tok") is not None:
        tol = 1e-5 if w.dtype == sv_inputs.F32 else 2e-3
        ok = orc_res["status"] == 0
        for key in ("p_tok", "q_tok", "lse_target", "lse_draft"):
            e = rel_err(orc_res[key][ok], gpu[key][ok])
            assert e < tol, (key, e)
    return rep


# ------------------------------------------------------------------ hand cases
CASES = golden_cases.load()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_exact_on_gpu(sv, case):
    w = golden_cases.workload(case)
    g = run_gpu(sv, w)
    golden_cases.check(case, g, sampling_aux=False)
    e = case["expect"]
    for key in ("p_tok", "q_tok"):
        if key in e:
            np.testing.assert_allclose(g[key][0][: len(e[key])], e[key], rtol=1e-6, atol=0)


# ------------------------------------------------------------------ workloads
def test_tiny_config(sv, orc):
    w = sv_inputs.tiny()
    check_parity(orc.verify_workload(w), run_gpu(sv, w), w)


@pytest.mark.parametrize("seed", [1101, 1102])
def test_tiny_many_sequences(sv, orc, seed):
    w = sv_inputs.tiny(seed=seed, B=256)
    check_parity(orc.verify_workload(w), run_gpu(sv, w), w)


def test_exception_budget_many_positions(sv, orc):
    """4096 positions at the steady-state value distribution (V cut to 12,345,
    a ragged 4-tile row): mismatches must all be flagged and under 0.1%."""
    w = sv_inputs.steady(seed=1201, B=1024, V=12345)
    rep = check_parity(orc.verify_workload(w), run_gpu(sv, w), w)
    log(f"exceptions {rep['exc_pos']} of {rep['positions']} positions")


def test_steady_small_batch_full_vocab(sv, orc):
    w = sv_inputs.steady(B=4)
    check_parity(orc.verify_workload(w), run_gpu(sv, w), w)


def test_steady_full_size(sv, orc):
    """The whole B=32 headline batch in one launch against the oracle."""
    w = sv_inputs.steady()
    g = run_gpu(sv, w)
    rep = check_parity(orc.verify_workload(w), g, w)
    log(f"steady: exceptions {rep['exc_pos']} of {rep['positions']} positions")
    assert (g["status"] == 0).all()
    assert ((g["accepted_len"] >= 0) & (g["accepted_len"] <= 3)).all()


@pytest.mark.parametrize("B", [1, 2, 4])
def test_longtail(sv, orc, B):
    w = sv_inputs.longtail(B)
    check_parity(orc.verify_workload(w), run_gpu(sv, w), w)


def test_grpo_full_size(sv, orc):
    """All 256 sequences of the GRPO batch against the oracle."""
    w = sv_inputs.grpo()
    g = run_gpu(sv, w)
    rep = check_parity(orc.verify_workload(w), g, w)
    log(f"grpo: exceptions {rep['exc_pos']} of {rep['positions']} positions")
    # rollouts of one prompt share target row 0: identical top-32 there
    assert np.array_equal(g["topk_idx"][0, 0], g["topk_idx"][7, 0])


def test_wide_sampling_full_size(sv, orc):
    """All 32 sequences (512 verified rows, fp32) against the oracle."""
    w = sv_inputs.wide()
    g = run_gpu(sv, w)
    rep = check_parity(orc.verify_workload(w), g, w)
    log(f"wide: exceptions {rep['exc_pos']} of {rep['positions']} positions")


def test_wide_greedy_bit_exact(sv, orc):
    w = sv_inputs.wide(greedy=True)
    g = run_gpu(sv, w)
    o = orc.verify_workload(w)
    np.testing.assert_array_equal(o["accepted_len"], g["accepted_len"])
    np.testing.assert_array_equal(o["out_tokens"], g["out_tokens"])
    np.testing.assert_array_equal(o["status"], g["status"])
    np.testing.assert_array_equal(o["topk_idx"], g["topk_idx"])
    np.testing.assert_array_equal(o["topk_val"].view(np.uint32), g["topk_val"].view(np.uint32))


def test_greedy_bf16_prefix_matches(sv, orc):
    """Greedy on bf16 with drafts equal to the target argmax for a prefix of random length."""
    w = sv_inputs.steady(seed=1301, B=16, V=50000)
    w.temperature = 0.0
    rng = np.random.default_rng(5)
    t = w.target_f32()
    am = t.argmax(axis=2)
    for b in range(w.B):
        n = rng.integers(0, w.k + 1)
        w.draft_tokens[b, :n] = am[b, :n]
    o = orc.verify_workload(w)
    g = run_gpu(sv, w)
    for key in ("accepted_len", "out_tokens", "status", "topk_idx"):
        np.testing.assert_array_equal(o[key], g[key], err_msg=key)
    assert len(set(o["accepted_len"].tolist())) > 1


# ------------------------------------------------------------------ edges
@pytest.mark.parametrize("V", [1, 7, 31, 32, 33, 4096, 4097, 3 * 4096 + 17])
@pytest.mark.parametrize("dtype", [sv_inputs.F32, sv_inputs.BF16])
def test_vocab_edges(sv, orc, V, dtype):
    w = sv_inputs.make_workload("edge", 6, 2, V, dtype, 1.0, 1400 + V, 2.0, 0.7)
    check_parity(orc.verify_workload(w), run_gpu(sv, w), w)
    wg = sv_inputs.make_workload("edge_greedy", 6, 2, V, dtype, 0.0, 1400 + V, 2.0, 0.7, draft_T=0.0)
    o, g = orc.verify_workload(wg), run_gpu(sv, wg)
    for key in ("accepted_len", "out_tokens", "topk_idx"):
        np.testing.assert_array_equal(o[key], g[key], err_msg=key)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_k_zero(sv, orc, T):
    w = sv_inputs.make_workload("k0", 5, 0, 9000, sv_inputs.BF16, T, 1501, 2.0, 0.5)
    check_parity(orc.verify_workload(w), run_gpu(sv, w), w)


@pytest.mark.parametrize("dtype", [sv_inputs.BF16, sv_inputs.F32])
def test_bonus_draw_tile_edges(sv, orc, dtype):
    """Bonus draws (every draft accepted: draft rows equal the target rows)
    whose row k has whole tiles of -inf, mass only in a middle tile, only in
    the ragged last tile, or spread over every tile: the crossing tile comes
    from the streaming statistics, the token from that tile's elements."""
    V, k = 3 * 8192 + 1000, 2
    w = sv_inputs.make_workload("bonus", 4, k, V, dtype, 1.0, 1951, 3.0, 0.5)
    f = (lambda x: x) if dtype == sv_inputs.F32 else sv_inputs.bf16_round
    tk = (w.target.astype(np.float32) if dtype == sv_inputs.F32 else sv_inputs.bf16_to_f32(w.target)).copy()
    tk[0, k, :16384] = -np.inf                    # tiles 0-1 empty, mass in tiles 2-3
    tk[1, k, :3 * 8192] = -np.inf                 # mass only in the ragged last tile
    tk[2, k, 8192:16384] += 6.0                   # most mass in tile 1
    w.target = f(tk)
    w.draft = w.target[:, :k].copy()              # p = q: every draft accepted
    o, g = orc.verify_workload(w), run_gpu(sv, w)
    assert (o["accepted_len"] == k).all()
    check_parity(o, g, w)


@pytest.mark.parametrize("which", ["steady", "greedy"])
def test_layouts_give_identical_results(sv, which):
    """The two item layouts only reorder which workgroup takes which item, and
    the two bf16 builds only differ in how many workgroups are resident: every
    combination gives the same bits."""
    w = sv_inputs.make_workload("lay", 6, 3, 40000, sv_inputs.BF16, 0.0 if which == "greedy" else 1.0, 1801, 3.0, 1.0)
    t, d, x, u = sv.to_device(w)
    greedy = w.temperature == 0
    res = []
    combos = [(lay, var) for lay in (sv.SV_LAYOUT_LAUNCH, sv.SV_LAYOUT_XCD_RUNS, sv.SV_LAYOUT_AUTO)
              for var in (sv.SV_VARIANT_BASE, sv.SV_VARIANT_HIGH_OCC, sv.SV_VARIANT_AUTO)]
    for layout, variant in combos:
        log(f"spec_verify layouts {which} layout={layout} variant={variant}")
        r = sv.verify(t, None if greedy else d, x, None if greedy else u, w.temperature, aux=not greedy,
                      layout=layout, variant=variant)
        torch.cuda.synchronize()
        res.append(gpu_to_numpy(r))
    for other in res[1:]:
        for key, v in res[0].items():
            if v is not None:
                np.testing.assert_array_equal(v, other[key], err_msg=key)


@pytest.mark.parametrize("k", [70, 260])
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_long_drafts(sv, orc, k, T):
    """k = 70: more drafts than a wave has lanes, so the draws learn the drawing
    row from the sequence's assembly; k = 260: k + 2 > 256 entries, so the
    assembly walks the group records in several rounds.  High acceptance
    (draft noise 0.05) so that chains run deep."""
    w = sv_inputs.make_workload("long_k", 3, k, 700, sv_inputs.BF16, T, 2300 + k, 2.0, 0.05,
                                draft_T=0.0 if T == 0 else None)
    o = orc.verify_workload(w)
    g = run_gpu(sv, w, aux=T > 0)
    if T > 0:
        check_parity(o, g, w)
        log(f"long drafts k={k}: accepted {g['accepted_len'].tolist()}")
    else:
        for key in ("accepted_len", "out_tokens", "status", "topk_idx"):
            np.testing.assert_array_equal(o[key], g[key], err_msg=key)


def test_plain_full_vocabulary(sv, orc):
    """k = 0 at the pages' vocabulary: plain temperature sampling (bonus draws
    only) with the top-32, in the plain bench workload's distribution."""
    w = sv_inputs.plain(B=8)
    check_parity(orc.verify_workload(w), run_gpu(sv, w), w)


@pytest.mark.parametrize("dtype,V", [(sv_inputs.BF16, 128 * 4096), (sv_inputs.F32, 128 * 2048)])
def test_largest_vocab(sv, orc, dtype, V):
    """The largest vocabulary the library takes: 64 tiles of 16 KB per row."""
    w = sv_inputs.make_workload("maxV", 1, 1, V, dtype, 1.0, 1601, 3.0, 1.0)
    check_parity(orc.verify_workload(w), run_gpu(sv, w), w)


def test_temperatures(sv, orc):
    for T in (0.25, 0.7, 2.0):
        w = sv_inputs.make_workload("temp", 8, 3, 20000, sv_inputs.F32, T, 1701, 3.0, 1.0)
        check_parity(orc.verify_workload(w), run_gpu(sv, w), w)


def test_top32_ties_and_constant_rows(sv, orc):
    """Heavy bf16 ties at the cut, a constant row (every element tied: exact
    fallback path), a row of -inf but 3 tokens, and -0.0/+0.0 ties."""
    V = 151936
    w = sv_inputs.make_workload("ties", 2, 2, V, sv_inputs.BF16, 0.0, 1801, 1.0, 1.0, draft_T=0.0)
    rng = np.random.default_rng(3)
    x = np.round(rng.standard_normal((2, 3, V)) * 2).astype(np.float32)
    x[0, 1] = 0.0
    x[0, 2] = -np.inf
    x[0, 2, [5, 70000, 151935]] = [1.0, 1.0, -1.0]
    x[1, 0, rng.integers(0, V, 100)] = -0.0
    w.target = sv_inputs.bf16_round(x)
    w.draft_tokens[:] = 0
    o, g = orc.verify_workload(w), run_gpu(sv, w)
    for key in ("accepted_len", "out_tokens", "topk_idx", "status"):
        np.testing.assert_array_equal(o[key], g[key], err_msg=key)
    np.testing.assert_array_equal(o["topk_val"].view(np.uint32), g["topk_val"].view(np.uint32))


def _tile_pos(dtype, c, t, s, w):
    """Row index of element w of vector s of thread t in tile c, in the
    streaming layout (thread t owns vectors at s * 256 * W + t * W)."""
    W = 8 if dtype == sv_inputs.BF16 else 4
    return c * 1024 * W + s * 256 * W + t * W + w


@pytest.mark.parametrize("dtype", [sv_inputs.BF16, sv_inputs.F32])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_top32_crowded_tiles(sv, orc, dtype, T):
    """A tile with 57 elements at or above its candidate threshold (it
    publishes its own 32 largest) and one with over 128 (overflow: the merge
    rescans it), in rows whose top-32 takes about 22 elements from the first
    and 10 from the second."""
    V = 40000
    B, k = 3, 1
    W = 8 if dtype == sv_inputs.BF16 else 4
    w = sv_inputs.make_workload("crowded", B, k, V, dtype, T, 2101, 1.0, 0.5, draft_T=T)
    rng = np.random.default_rng(7)
    x = (-4.0 + 0.25 * rng.standard_normal((B, k + 1, V))).astype(np.float32)

    def crowd(row, c, lanes, per_lane, vals):
        # per wave, lanes 0..lanes-1 (wave 3: lane 0 only) hold per_lane of the
        # values; wave 3's lane 1 holds 0.5, so the tile's threshold (the
        # smallest of the 8 listed lane maxima) is 0.5
        it = iter(vals)
        for wave in range(4):
            for ln in (range(lanes) if wave < 3 else (0,)):
                for e in range(per_lane):
                    row[_tile_pos(dtype, c, wave * 64 + ln, e // W, e % W)] = next(it)
        row[_tile_pos(dtype, c, 3 * 64 + 1, 0, 0)] = 0.5
        return row

    for b in range(B):
        for i in range(k + 1):
            # tile 0: 7 lanes x 8 values in [14, 28], step 1/4 (exact in bf16)
            crowd(x[b, i], 0, 2, 8, 14.0 + np.arange(56) / 4.0 + 0.25 * b)
            # tile 1: over 128 values in [3, 24], step 1/8
            n1 = 10 * 4 * W if W == 4 else 7 * 24
            lanes1, per1 = (3, 4 * W) if W == 4 else (2, 24)
            crowd(x[b, i], 1, lanes1, per1, 3.0 + np.arange(n1) / 8.0)
    if dtype == sv_inputs.BF16:
        w.target = sv_inputs.bf16_round(x)
        w.draft = sv_inputs.bf16_round(x[:, :k] + 0.1)
    else:
        w.target = x
        w.draft = (x[:, :k] + np.float32(0.1)).astype(np.float32)
    o, g = orc.verify_workload(w), run_gpu(sv, w)
    for key in ("topk_idx", "status"):
        np.testing.assert_array_equal(o[key], g[key], err_msg=key)
    np.testing.assert_array_equal(o["topk_val"].view(np.uint32), g["topk_val"].view(np.uint32))
    # both tiles contribute to every row's top-32
    tile_of_idx = o["topk_idx"] // (1024 * W)
    assert ((tile_of_idx == 0).sum(axis=-1) > 0).all() and ((tile_of_idx == 1).sum(axis=-1) > 0).all()
    if T == 0:
        for key in ("accepted_len", "out_tokens"):
            np.testing.assert_array_equal(o[key], g[key], err_msg=key)
    else:
        check_parity(o, g, w)


def test_data_errors(sv, orc):
    V = 5000
    w = sv_inputs.make_workload("errors", 8, 2, V, sv_inputs.F32, 1.0, 1901, 2.0, 0.5)
    w.draft_tokens[1, 1] = V             # bad token
    w.draft[2, 0, 17] = np.nan           # NaN in a draft row
    w.target[3, 2, 4000] = np.inf        # +inf in the bonus row
    w.draft[4, 1, :] = -np.inf           # empty draft row
    w.uniforms[5, 3] = 1.0               # bad uniform
    w.target[6, 0, 9] = np.nan           # NaN in a target row (top-32 slot NaN)
    w.target[6, 0, 10] = np.inf
    o, g = orc.verify_workload(w), run_gpu(sv, w)
    for key in ("status", "accepted_len", "out_tokens", "topk_idx"):
        np.testing.assert_array_equal(o[key], g[key], err_msg=key)
    assert g["status"].tolist() == [0, 1, 2, 4, 8, 16, 2, 0]


# ------------------------------------------------------------------ layout
def test_strided_and_unaligned_rows(sv, orc):
    w = sv_inputs.make_workload("stride", 3, 2, 10001, sv_inputs.BF16, 1.0, 2001, 2.0, 0.6)
    base = run_gpu(sv, w)
    t, d, x, u = sv.to_device(w)
    pad = 64
    tb = torch.zeros(3, 3, 10001 + pad, dtype=t.dtype, device=t.device)
    db = torch.zeros(3, 2, 10001 + pad, dtype=t.dtype, device=t.device)
    tb[..., :10001] = t
    db[..., :10001] = d
    r = sv.verify(tb[..., :10001], db[..., :10001], x, u, 1.0, aux=True)
    g = gpu_to_numpy(r)
    for key in ("accepted_len", "out_tokens", "topk_idx", "topk_val", "p_tok", "lse_target"):
        np.testing.assert_array_equal(base[key], g[key], err_msg=key)
    # V=10001 bf16 rows start at odd 16-byte phases: the element-wise load path
    check_parity(orc.verify_workload(w), base, w)


# ------------------------------------------------------------------ determinism
def test_deterministic_across_runs_and_workspaces(sv):
    w = sv_inputs.steady(seed=2101, B=3)
    a = run_gpu(sv, w)
    b = run_gpu(sv, w)
    t, d, x, u = sv.to_device(w)
    ws = torch.zeros(32 << 20, dtype=torch.uint8, device="cuda")
    c = gpu_to_numpy(sv.verify(t, d, x, u, w.temperature, aux=True, workspace=ws))
    for key in a:
        if a[key] is not None:
            np.testing.assert_array_equal(a[key].view(np.uint8), b[key].view(np.uint8), err_msg=key)
            np.testing.assert_array_equal(a[key].view(np.uint8), c[key].view(np.uint8), err_msg=key)


def test_batch_invariance(sv):
    w = sv_inputs.longtail(4)
    full = run_gpu(sv, w)
    for b in range(4):
        one = run_gpu(sv, w.subset([b]))
        for key in full:
            if full[key] is not None:
                np.testing.assert_array_equal(full[key][b:b + 1].view(np.uint8), one[key].view(np.uint8),
                                              err_msg=key)


def test_workspace_left_zero_for_any_next_shape(sv, orc):
    """Regression: one workspace serves calls of growing and shrinking shapes;
    each call must leave every byte zero, or the next layout would read stale
    records as counters."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    for w in (sv_inputs.steady(seed=2201, B=2, V=20000), sv_inputs.steady(seed=2204, B=12, V=20000),
              sv_inputs.tiny(seed=2202, B=9), sv_inputs.steady(seed=2203, B=1)):
        t, d, x, u = sv.to_device(w)
        r = sv.verify(t, d, x, u, w.temperature, aux=True, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0
        check_parity(orc.verify_workload(w), gpu_to_numpy(r), w)
    wg = sv_inputs.wide(seed=2205, B=3, k=4, V=30000, greedy=True)
    t, _, x, _ = sv.to_device(wg)
    sv.verify(t, None, x, None, 0.0, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero().item()) == 0


# ------------------------------------------------------------------ distribution
def test_gpu_lossless_marginal_chi_square(sv, orc):
    """The GPU as a sampler over 10^6 sequences at V=8: every emitted token
    follows the target distribution, and decisions match the oracle."""
    from scipy import stats
    from scipy.special import softmax
    V, k, N, T = 8, 3, 10 ** 6, 1.0
    rng = np.random.default_rng(11)
    t = rng.standard_normal((k + 1, V)).astype(np.float32)
    d = (t[:k] + 0.8 * rng.standard_normal((k, V))).astype(np.float32)
    w = sv_inputs.fixed_rows(N, t, d, T, 11)
    g = run_gpu(sv, w, aux=False)
    p = softmax(t.astype(np.float64) / T, axis=1)
    acc = g["accepted_len"]
    for i in range(k + 1):
        reach = acc >= i
        counts = np.bincount(g["out_tokens"][reach, i], minlength=V)
        _, pv = stats.chisquare(counts, p[i] * reach.sum())
        assert pv > 1e-4 / (k + 1), (i, pv)
    o = orc.verify_workload(w)
    rep = compare_decisions(o, g, k)
    assert not rep["fails"]
    assert rep["exc_pos"] <= 0.001 * rep["positions"]
