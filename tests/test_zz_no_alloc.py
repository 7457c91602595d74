"""spec_verify_noalloc, the entry point that allocates nothing, called through
the C ABI.  Its workspace is the library's static scratch array, which keeps
the last call's contents between calls; its outputs must equal those of
spec_verify with a freshly zeroed caller workspace, bit for bit, on calls in a
row whose later inputs are smaller than the first."""
import sys

import numpy as np
import pytest

import sv_inputs

torch = pytest.importorskip("torch")


def log(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sv():
    import draft_verification_spec_amd as m
    m.load_library()
    return m


def _outputs(B, k, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    return dict(acc=torch.full((B,), -7, **i32), out=torch.full((B, k + 1), -7, **i32),
                tv=torch.full((B, k + 1, 32), 7.0, **f32), ti=torch.full((B, k + 1, 32), -7, **i32),
                st=torch.full((B,), -7, **i32), lt=torch.full((B, k + 1), 7.0, **f32),
                ld=torch.full((B, max(k, 1)), 7.0, **f32), pt=torch.full((B, max(k, 1)), 7.0, **f32),
                qt=torch.full((B, max(k, 1)), 7.0, **f32))


def _run(sv, w, noalloc):
    t, d, x, u = sv.to_device(w)
    greedy = w.temperature == 0
    o = _outputs(w.B, w.k, t.device)
    aux = sv.sv_aux_t(o["st"].data_ptr(), o["lt"].data_ptr(), o["ld"].data_ptr(), o["pt"].data_ptr(),
                      o["qt"].data_ptr(), sv.SV_LAYOUT_AUTO)
    shape = sv.make_shape(w.B, w.k, w.V, w.dtype, w.temperature)
    args = (shape, t.data_ptr(), None if greedy else d.data_ptr(), x.data_ptr() if w.k > 0 else None,
            None if greedy else u.data_ptr(), o["acc"].data_ptr(), o["out"].data_ptr(), o["tv"].data_ptr(),
            o["ti"].data_ptr(), aux)
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        rc = sv.spec_verify_noalloc(*args, stream)
    else:
        ws = torch.zeros(sv.spec_verify_workspace_bytes(shape), dtype=torch.uint8, device=t.device)
        rc = sv.spec_verify(*args, ws.data_ptr(), ws.numel(), stream)
    assert rc == sv.SV_OK, sv.spec_verify_error_string(rc)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in o.items()}


def _same(a, b, name):
    for key in a:
        np.testing.assert_array_equal(a[key].view(np.uint8), b[key].view(np.uint8), err_msg=f"{name}: {key}")


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_on_shrinking_calls(sv):
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    calls = [sv_inputs.steady(seed=4101, B=8),                     # 8 x 4 rows of V = 151936, bf16
             sv_inputs.tiny(seed=4102, B=3),                        # then a smaller fp32 batch
             sv_inputs.wide(seed=4103, B=2, k=5, V=30000, greedy=True)]   # then greedy, smaller still
    for w in calls:
        log(f"spec_verify_noalloc {w.name} B={w.B} k={w.k} V={w.V} T={w.temperature}")
        got = _run(sv, w, noalloc=True)
        want = _run(sv, w, noalloc=False)
        _same(got, want, w.name)
        if w.temperature > 0:
            assert (got["st"] == 0).all() and (got["acc"] >= 0).all()


def test_noalloc_rejects_shapes_beyond_its_scratch(sv):
    """A shape whose workspace exceeds the static scratch is refused on the host
    before any device work (the pointers below are never used)."""
    big = sv.make_shape(512, 3, 128256, sv.SV_BF16, 0.7)
    assert sv.spec_verify_workspace_bytes(big) > sv.SV_NOALLOC_MAX_BYTES
    fake = 0x1000
    rc = sv.spec_verify_noalloc(big, fake, fake, fake, fake, fake, fake, fake, fake, None, None)
    assert rc == sv.SV_ERR_SCRATCH
    assert "static scratch" in sv.spec_verify_error_string(rc)
    fits = sv.make_shape(256, 3, 128256, sv.SV_BF16, 0.7)
    assert sv.spec_verify_workspace_bytes(fits) <= sv.SV_NOALLOC_MAX_BYTES
