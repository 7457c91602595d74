"""C-ABI boundary checks that need no GPU: the library loads, exports every
function the header declares, sizes its workspace, describes its error codes
and rejects bad arguments on the host before anything is enqueued."""
import ctypes
import os

import pytest

import draft_verification_spec_amd as sv


@pytest.fixture(scope="module")
def lib():
    return sv.load_library()


def test_exports_every_declared_function(lib):
    names = sv.declared_functions()
    assert set(names) == {"spec_verify", "spec_verify_workspace_bytes", "spec_verify_error_string",
                          "spec_verify_layout_choice", "spec_verify_variant_choice", "spec_verify_noalloc", "sv_kd",
                          "sv_kd_workspace_bytes"}
    for n in names:
        assert hasattr(lib, n), n


def test_error_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        s = sv.spec_verify_error_string(code)
        assert s and "unknown" not in s
    assert "unknown" in sv.spec_verify_error_string(-99)


def test_workspace_bytes():
    f = sv.spec_verify_workspace_bytes
    small = f(sv.make_shape(2, 3, 1000, sv.SV_F32, 1.0))
    big = f(sv.make_shape(32, 3, 151936, sv.SV_BF16, 1.0))
    assert 0 < small < big
    assert big < 64 << 20                      # a few MB at the steady-state shape
    assert f(sv.make_shape(-1, 3, 10, 0, 1.0)) == 0
    assert f(sv.make_shape(1, 3, 0, 0, 1.0)) == 0
    assert f(sv.make_shape(1, 3, 262144, sv.SV_F32, 1.0)) > 0
    assert f(sv.make_shape(1, 3, 262145, sv.SV_F32, 1.0)) == 0
    assert f(sv.make_shape(1, 3, 524288, sv.SV_BF16, 1.0)) > 0
    assert f(sv.make_shape(1, 3, 524289, sv.SV_BF16, 1.0)) == 0
    assert f(sv.make_shape(0, 3, 100, 0, 1.0)) > 0


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _call(shape, aux=None, **over):
    a = dict(t=FAKE, d=FAKE, x=FAKE, u=FAKE, acc=FAKE, out=FAKE, tv=FAKE, ti=FAKE, ws=FAKE * 16,
             wsb=1 << 30)
    a.update(over)
    return sv.spec_verify(shape, a["t"], a["d"], a["x"], a["u"], a["acc"], a["out"], a["tv"], a["ti"], aux,
                          a["ws"], a["wsb"], None)


def test_layout_choice():
    f = sv.spec_verify_layout_choice
    for B in (1, 4, 32, 256):
        for k in (0, 3, 15):
            for dt in (sv.SV_F32, sv.SV_BF16):
                for T in (0.0, 1.0):
                    assert f(sv.make_shape(B, k, 151936, dt, T)) in (sv.SV_LAYOUT_LAUNCH, sv.SV_LAYOUT_XCD_RUNS)
    assert f(sv.make_shape(-1, 3, 1000, 0, 1.0)) == 0
    assert f(sv.make_shape(2, 3, 1000, 0, -1.0)) == 0
    bad = sv.sv_aux_t(None, None, None, None, None, 3)
    assert _call(sv.make_shape(2, 3, 1000, 0, 1.0), aux=bad) == sv.SV_ERR_SHAPE


def test_variant_choice():
    f = sv.spec_verify_variant_choice
    for B in (1, 4, 32, 256):
        for k in (0, 3, 15):
            for T in (0.0, 1.0):
                assert f(sv.make_shape(B, k, 151936, sv.SV_BF16, T)) in (sv.SV_VARIANT_BASE, sv.SV_VARIANT_HIGH_OCC)
                assert f(sv.make_shape(B, k, 151936, sv.SV_F32, T)) == sv.SV_VARIANT_BASE   # one fp32 build
    assert f(sv.make_shape(-1, 3, 1000, 1, 1.0)) == 0
    for v in (-1, 3):
        bad = sv.sv_aux_t(None, None, None, None, None, sv.SV_LAYOUT_AUTO, v)
        assert _call(sv.make_shape(2, 3, 1000, 1, 1.0), aux=bad) == sv.SV_ERR_SHAPE


def test_host_validation_codes():
    good = sv.make_shape(2, 3, 1000, sv.SV_F32, 1.0)
    assert sv.spec_verify(None, 0, 0, 0, 0, 0, 0, 0, 0, None, 0, 0, None) == sv.SV_ERR_NULL
    assert _call(sv.make_shape(2, 3, 1000, 7, 1.0)) == sv.SV_ERR_DTYPE
    assert _call(sv.make_shape(-1, 3, 1000, 0, 1.0)) == sv.SV_ERR_SHAPE
    assert _call(sv.make_shape(2, -1, 1000, 0, 1.0)) == sv.SV_ERR_SHAPE
    assert _call(sv.make_shape(2, 3, 0, 0, 1.0)) == sv.SV_ERR_SHAPE
    assert _call(sv.make_shape(2, 3, 262145, sv.SV_F32, 1.0)) == sv.SV_ERR_SHAPE
    assert _call(sv.make_shape(2, 3, 524289, sv.SV_BF16, 1.0)) == sv.SV_ERR_SHAPE
    assert _call(sv.make_shape(2, 3, 1000, 0, 1.0, target_row_stride=999)) == sv.SV_ERR_SHAPE
    assert _call(sv.make_shape(2, 3, 1000, 0, 1.0, draft_row_stride=10)) == sv.SV_ERR_SHAPE
    assert _call(sv.make_shape(2, 3, 1000, 0, -1.0)) == sv.SV_ERR_TEMPERATURE
    assert _call(sv.make_shape(2, 3, 1000, 0, float("nan"))) == sv.SV_ERR_TEMPERATURE
    assert _call(sv.make_shape(2, 3, 1000, 0, float("inf"))) == sv.SV_ERR_TEMPERATURE
    assert _call(good, t=None) == sv.SV_ERR_NULL
    assert _call(good, d=None) == sv.SV_ERR_NULL          # sampling needs draft logits
    assert _call(good, u=None) == sv.SV_ERR_NULL          # and uniforms
    assert _call(good, x=None) == sv.SV_ERR_NULL
    assert _call(good, tv=None) == sv.SV_ERR_NULL
    assert _call(good, ws=None) == sv.SV_ERR_WORKSPACE
    need = sv.spec_verify_workspace_bytes(good)
    assert _call(good, wsb=need - 1) == sv.SV_ERR_WORKSPACE
    assert _call(good, ws=FAKE * 16 + 8) == sv.SV_ERR_WORKSPACE   # 256-byte alignment
    # B == 0 is a valid empty call: nothing to enqueue
    assert _call(sv.make_shape(0, 3, 1000, 0, 1.0)) == sv.SV_OK


def test_kd_workspace_bytes():
    f = sv.sv_kd_workspace_bytes
    small = f(sv.make_kd_shape(24, 20000, sv.SV_BF16, sv.SV_F32, 12, 4))
    big = f(sv.make_kd_shape(4096, 151936, sv.SV_BF16, sv.SV_BF16, 256, 8))
    assert 0 < small < big < 16 << 20
    assert f(sv.make_kd_shape(-1, 100, 0, 0, 1, 1)) == 0
    assert f(sv.make_kd_shape(1, 0, 0, 0, 1, 1)) == 0
    assert f(sv.make_kd_shape(1, 100, 0, 0, 3, 2)) == 0          # group must divide S
    assert f(sv.make_kd_shape(1, 100, 0, 0, 2, 2, w_max=0.0)) == 0
    assert f(sv.make_kd_shape(1, 262144, sv.SV_F32, 0, 1, 1)) > 0
    assert f(sv.make_kd_shape(1, 262145, sv.SV_F32, 0, 1, 1)) == 0
    assert f(sv.make_kd_shape(1, 524288, sv.SV_BF16, 0, 1, 1)) > 0
    assert f(sv.make_kd_shape(1, 524289, sv.SV_BF16, 0, 1, 1)) == 0


def _kd_call(shape, **over):
    a = dict(z=FAKE, tv=FAKE, ti=FAKE, rs=FAKE, rw=FAKE, kl=FAKE, w=None, st=None, loss=FAKE, g=None,
             ws=FAKE * 16, wsb=1 << 30)
    a.update(over)
    return sv.sv_kd(shape, a["z"], a["tv"], a["ti"], a["rs"], a["rw"], a["kl"], a["w"], a["st"], a["loss"], a["g"],
                    a["ws"], a["wsb"], None)


def test_kd_host_validation_codes():
    good = sv.make_kd_shape(24, 20000, sv.SV_BF16, sv.SV_F32, 12, 4)
    assert sv.sv_kd(None, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, None) == sv.SV_ERR_NULL
    assert _kd_call(sv.make_kd_shape(24, 20000, 5, 0, 12, 4)) == sv.SV_ERR_DTYPE
    assert _kd_call(sv.make_kd_shape(24, 20000, 0, 9, 12, 4)) == sv.SV_ERR_DTYPE
    assert _kd_call(sv.make_kd_shape(-1, 20000, 0, 0, 12, 4)) == sv.SV_ERR_SHAPE
    assert _kd_call(sv.make_kd_shape(24, 0, 0, 0, 12, 4)) == sv.SV_ERR_SHAPE
    assert _kd_call(sv.make_kd_shape(24, 20000, 0, 0, 12, 5)) == sv.SV_ERR_SHAPE
    assert _kd_call(sv.make_kd_shape(24, 20000, 0, 0, 0, 1)) == sv.SV_ERR_SHAPE
    assert _kd_call(sv.make_kd_shape(24, 20000, 0, 0, 12, 4, w_max=float("nan"))) == sv.SV_ERR_SHAPE
    assert _kd_call(sv.make_kd_shape(24, 20000, 0, 0, 12, 4, row_stride=19999)) == sv.SV_ERR_SHAPE
    for k in ("z", "tv", "ti", "rs", "rw", "kl", "loss"):
        assert _kd_call(good, **{k: None}) == sv.SV_ERR_NULL, k
    assert _kd_call(good, ws=None) == sv.SV_ERR_WORKSPACE
    need = sv.sv_kd_workspace_bytes(good)
    assert _kd_call(good, wsb=need - 1) == sv.SV_ERR_WORKSPACE
    assert _kd_call(good, ws=FAKE * 16 + 8) == sv.SV_ERR_WORKSPACE
    assert _kd_call(sv.make_kd_shape(0, 20000, 0, 0, 12, 4)) == sv.SV_OK


def test_product_path_never_touches_the_oracle():
    """Neither the binding nor the HIP source names the oracle package."""
    import glob
    import os
    pkg = os.path.dirname(sv.__file__)
    for f in glob.glob(os.path.join(pkg, "*.py")) + glob.glob(os.path.join(pkg, "csrc", "*")):
        text = open(f).read()
        assert "import oracle" not in text and "sv_oracle" not in text and "orc_verify" not in text, f
        assert "kd_oracle" not in text, f


def test_dispatch_table_matches_its_measurement():
    """The table compiled into the library is the one its committed measurement
    chose: every row of the timing table (the fastest item layout and, for
    bf16, kernel build per dtype, mode, B, k) has the same entry in
    sv_dispatch.h, in the same order."""
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    hdr = open(os.path.join(root, "draft_verification_spec_amd", "csrc", "sv_dispatch.h")).read()
    entries = [tuple(int(v) for v in m) for m in
               re.findall(r"\{(-?\d+), (-?\d+), (-?\d+), (-?\d+), (-?\d+), (-?\d+)\}", hdr)]
    assert entries[-1] == (0, 0, -1, -1, 0, 0)                 # end marker
    L, X = sv.SV_LAYOUT_LAUNCH, sv.SV_LAYOUT_XCD_RUNS
    B_, H_ = sv.SV_VARIANT_BASE, sv.SV_VARIANT_HIGH_OCC
    rows = []
    for line in open(os.path.join(root, "profiles", "dispatch_layout_V151936.md")):
        p = [x.strip() for x in line.strip().strip("|").split("|")]
        if len(p) != 9 or p[0] not in ("bf16", "f32"):
            continue
        times = {(L, B_): p[4], (X, B_): p[5], (L, H_): p[6], (X, H_): p[7]}
        times = {c: float(v) for c, v in times.items() if v != "-"}
        if p[0] == "f32":
            assert set(times) == {(L, B_), (X, B_)}, line   # fp32 has one build
        lay_s, var_s = [x.strip() for x in p[8].split(",")]
        combo = (L if lay_s == "launch" else X, B_ if var_s == "base" else H_)
        # the fastest (the timings are printed to 0.01 us: equal ones are a tie)
        assert times[combo] <= min(times.values()), line
        rows.append((int(p[2]), int(p[3]), 1 if p[0] == "bf16" else 0, 1 if p[1] == "greedy" else 0) + combo)
    assert rows and rows == entries[:-1]
