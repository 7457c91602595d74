"""HIP graph capture of both entry points.

The library allocates nothing, synchronises nothing, records no memset and
leaves its workspace zero-filled, so one captured call can be replayed: each
replay below runs on fresh inputs copied into the captured buffers, with eager
work and a synchronisation between replays, and must give the bits of an eager
call on the same inputs (both paths are deterministic).
"""
import sys

import numpy as np
import pytest

import sv_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def log(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import draft_verification_spec_amd as m
    m.load_library()
    return m


def bits(t):
    return None if t is None else t.detach().cpu().numpy().view(np.uint8).copy()


def warm_then_capture(fn):
    """One eager call on a side stream, then the capture of fn."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_verify_graph_replays(sv, T):
    B, V = 4, 20000
    w0 = sv_inputs.steady(seed=3101, B=B, V=V)
    shape = sv.make_shape(B, w0.k, V, w0.dtype, T)
    ws = torch.zeros(sv.spec_verify_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    ws_eager = torch.zeros_like(ws)
    t, d, x, u = sv.to_device(w0)
    greedy = T == 0.0

    def call(tt, dd, xx, uu, wsp):
        return sv.verify(tt, None if greedy else dd, xx, None if greedy else uu, T, aux=not greedy, workspace=wsp)

    log(f"graph capture of spec_verify B={B} V={V} T={T}")
    g, out = warm_then_capture(lambda: call(t, d, x, u, ws))
    for seed in (3102, 3103, 3104):
        wi = sv_inputs.steady(seed=seed, B=B, V=V)
        ti, di, xi, ui = sv.to_device(wi)
        t.copy_(ti), d.copy_(di), x.copy_(xi), u.copy_(ui)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: bits(v) for k, v in out._asdict().items()}
        ref = call(ti, di, xi, ui, ws_eager)             # eager work between replays
        torch.cuda.synchronize()
        for k, v in ref._asdict().items():
            if v is not None:
                np.testing.assert_array_equal(got[k], bits(v), err_msg=f"{k} seed {seed}")
        assert int(ws.count_nonzero().item()) == 0
        assert int(ws_eager.count_nonzero().item()) == 0


def test_kd_graph_replays(sv):
    w0 = sv_inputs.kd_small()
    shape = sv.make_kd_shape(w0.N, w0.V, w0.dtype, sv.SV_F32, w0.S, w0.group, w0.w_max)
    ws = torch.zeros(sv.sv_kd_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    ws_eager = torch.zeros_like(ws)
    z, tv, ti, rs, rw = sv.kd_to_device(w0)

    def call(zz, vv, ii, ss, rr, wsp):
        return sv.kd(zz, vv, ii, ss, rr, w0.group, w_max=w0.w_max, grad=True, grad_dtype=torch.float32,
                     workspace=wsp)

    log(f"graph capture of sv_kd N={w0.N} V={w0.V}")
    g, out = warm_then_capture(lambda: call(z, tv, ti, rs, rw, ws))
    for seed in (3201, 3202, 3203):
        wi = sv_inputs.kd_small(seed=seed)
        zi, tvi, tii, rsi, rwi = sv.kd_to_device(wi)
        z.copy_(zi), tv.copy_(tvi), ti.copy_(tii), rs.copy_(rsi), rw.copy_(rwi)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: bits(v) for k, v in out._asdict().items()}
        ref = call(zi, tvi, tii, rsi, rwi, ws_eager)
        torch.cuda.synchronize()
        for k, v in ref._asdict().items():
            if v is not None:
                np.testing.assert_array_equal(got[k], bits(v), err_msg=f"{k} seed {seed}")
        assert int(ws.count_nonzero().item()) == 0
