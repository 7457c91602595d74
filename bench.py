"""Benchmark of the speculative-sampling verification step on one MI355X.

One step = one spec_verify call (acceptance chain, residual/bonus draw and
top-32 for every verified position) over one batch of the steady-state rollout
workload: B=32, k=3, V=151936, bf16 logits, T=1.  The inputs are synthetic and
seeded; 16 copies of the batch (1.09 GB, over four times the 256 MB Infinity
Cache) rotate so every step reads its logits from HBM.

Prints one JSON line.  value = algorithmic logit bytes (each logit read once,
B(2k+1)V * 2 bytes) / wall time per step over K back-to-back steps, inputs
resident in HBM.  By default the K calls are replayed from a HIP graph (one
capture of one call per input copy), so the host's per-call cost stays out of
the number, as in a serving loop that captures its step; --eager times K
direct calls instead.  roofline = the same bytes / the mean duration of the
kernel launch, against the 8 TB/s HBM peak: torch events recorded on the
launch stream before and after the K timed steps (a step is that one launch),
elapsed / K.  Events around each single call add about 2 us of their own (a
plain 11.5 us read reads 14.2 us that way); their distribution is reported
beside it.  cpu_baseline = the plain C oracle on the host over a bounded number
of whole batches.

  python bench.py [--steps K] [--warmup W] [--eager] [--workload steady|longtail1|longtail2|longtail4|grpo|wide|wide_greedy|plain|tiny]
  python bench.py --workload kd   # the drafter distillation step over the stored top-32 (its own metric)
  python bench.py --stream-read   # a plain HBM read of the steady batch's bytes: the achievable read rate
  python bench.py --copy-calib    # a plain 1 GiB device copy, for HBM counter calibration
  python bench.py --source-hash sv_verify|sv_kd_kernel   # the source hash a profile summary records
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "spec-verify logits GB/s (% HBM peak) + rows/s at B=32 k=3 V=151936 bf16"
MALL_BYTES = 256 << 20


def make_workload(name):
    import sv_inputs
    if name == "steady":
        return sv_inputs.steady()
    if name.startswith("longtail"):
        return sv_inputs.longtail(int(name[len("longtail"):]))
    if name == "grpo":
        return sv_inputs.grpo()
    if name == "wide":
        return sv_inputs.wide()
    if name == "wide_greedy":
        return sv_inputs.wide(greedy=True)
    if name == "tiny":
        return sv_inputs.tiny()
    if name == "plain":
        return sv_inputs.plain()
    raise SystemExit(f"unknown workload {name}")


def describe(w):
    return f"{w.name} B={w.B} k={w.k} V={w.V} {'bf16' if w.dtype else 'f32'} T={w.temperature:g}"


KERNEL_SOURCES = {
    "sv_verify": ["draft_verification_spec_amd/csrc/spec_verify.hip", "draft_verification_spec_amd/csrc/sv_device.h"],
    "sv_kd_kernel": ["draft_verification_spec_amd/csrc/sv_kd.hip", "draft_verification_spec_amd/csrc/sv_device.h"],
}


def source_hash(kernel):
    """sha256 over the kernel's source files, in order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def counted_traffic(kernel, profile_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    profiles/<profile_name>.md (fetched + written, copy-calibrated), or None
    when there is none or the kernel's sources changed since the counters were
    taken."""
    import re
    path = os.path.join(ROOT, "profiles", profile_name + ".md")
    if not os.path.exists(path):
        return None
    m = re.search(r"traffic_per_launch: source_sha256=([0-9a-f]{64}) fetch_bytes=(\d+) write_bytes=(\d+)",
                  open(path).read())
    if not m or source_hash(kernel) != m.group(1):
        return None
    return int(m.group(2)) + int(m.group(3))


def cpu_baseline(w, budget_s=10.0):
    """The oracle as it stands, single-threaded, over whole batches until about
    budget_s seconds have passed (at least one batch)."""
    import oracle
    oracle.build()
    t0 = time.perf_counter()
    n = 0
    res = None
    while True:
        res = oracle.verify_workload(w)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    return dt, n, res


def copy_calib():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_per_launch_read": n, "write": n, "launches": 3}))


KD_METRIC = "kd drafter-logit read + gradient write GB/s (% HBM peak) at N=4096 V=151936 bf16"


def bench_kd(args):
    """The reward-weighted distillation step: one sv_kd launch over the rollout
    batch's stored positions (N=4096 rows of V=151936 bf16 drafter logits),
    loss and bf16 gradient.  value = (logits read once + gradient written once)
    / wall time per step."""
    import torch
    import draft_verification_spec_amd as sv
    import sv_inputs

    w = sv_inputs.kd_rollout() if args.workload == "kd" else sv_inputs.kd_small()
    print(f"[bench] workload {w.name} N={w.N} V={w.V} bf16, grad bf16", file=sys.stderr, flush=True)
    z, tv, ti, rs, rw = sv.kd_to_device(w)
    alg = w.alg_bytes(grad_bytes=2)
    copies = args.copies or max(1, -(-4 * MALL_BYTES // (w.N * w.V * w.elem_bytes)))
    zs = [z] + [z.clone() for _ in range(copies - 1)]
    shape = sv.make_kd_shape(w.N, w.V, sv.SV_BF16, sv.SV_BF16, w.S, w.group, w.w_max)
    ws = sv.workspace_for(z.device, sv.sv_kd_workspace_bytes(shape))
    dev = z.device
    kl = torch.empty(w.N, dtype=torch.float32, device=dev)
    wt = torch.empty_like(kl)
    st = torch.empty(w.N, dtype=torch.int32, device=dev)
    loss = torch.zeros(1, dtype=torch.float64, device=dev)
    grad = torch.empty(w.N, w.V, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        rc = sv.sv_kd(shape, zs[i % copies].data_ptr(), tv.data_ptr(), ti.data_ptr(), rs.data_ptr(), rw.data_ptr(),
                      kl.data_ptr(), wt.data_ptr(), st.data_ptr(), loss.data_ptr(), grad.data_ptr(), ws.data_ptr(),
                      ws.numel(), stream.cuda_stream)
        if rc != sv.SV_OK:
            raise sv.SpecVerifyError(rc)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps over {copies} input copies",
          file=sys.stderr, flush=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(args.warmup + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kern_ms = np.array([a.elapsed_time(b) for a, b in ev])
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
    r1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    value = alg / (ms_per_step * 1e-3) / 1e9
    kern_avg = r0.elapsed_time(r1) / args.steps       # ms per launch over the timed region
    achieved = alg / (kern_avg * 1e-3) / 1e9
    line = {
        "metric": KD_METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Philox drafter logits and stored top-32 entries of the workload's shape)",
        "config": {"workload": f"{w.name} N={w.N} V={w.V} bf16 grad bf16", "N": w.N, "V": w.V, "S": w.S,
                   "group": w.group, "alg_bytes_per_step": alg, "input_copies_rotated": copies},
        "rows_per_s": round(w.N / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counted_traffic("sv_kd_kernel", f"sv_kd_kernel_{w.name}_N{w.N}_V{w.V}_bf16"),
                     "kernel": "sv_kd_kernel",
                     "kernel_us_mean": round(kern_avg * 1e3, 3),
                     "kernel_us_source": "events around the K timed launches on the launch stream, / K",
                     "per_call_events_us_p10_p50_p90": [round(float(np.percentile(kern_ms, q)) * 1e3, 3)
                                                        for q in (10, 50, 90)]},
        "loss": float(loss.cpu()[0]),
    }
    if not args.no_cpu:
        import oracle
        oracle.build()
        rows = np.arange(w.N)                   # the whole batch, 256 rows at a time (bounded memory)
        t1 = time.perf_counter()
        o_kl, o_status = [], []
        for i in range(0, w.N, 256):
            q = oracle.kd_workload(w, grad=True, rows=rows[i:i + 256])
            o_kl.append(q.kl)
            o_status.append(q.status)
            del q
        dt = time.perf_counter() - t1
        o_kl, o_status = np.concatenate(o_kl), np.concatenate(o_status)
        sample_bytes = len(rows) * w.V * (w.elem_bytes + 2)
        g_kl = kl.cpu().numpy()[rows]
        ok = o_status == 0
        model, nthreads, usable = host_cpu()
        line["cpu_baseline"] = {
            "value": round(sample_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"all {len(rows)} rows of the batch (loss and fp64 gradient), {dt:.2f} s, one thread",
            "cpu_model": model, "host_threads": nthreads, "usable_threads": usable,
            "rows_per_s": round(len(rows) / dt, 2)}
        line["parity_vs_oracle"] = {"rows": int(len(rows)), "max_abs_kl_err": float(np.max(np.abs(g_kl[ok] - o_kl[ok]))),
                                    "status_equal": bool(np.array_equal(st.cpu().numpy()[rows], o_status))}
    print(json.dumps(line), flush=True)


def host_cpu():
    """CPU model and thread counts of this host, for the baseline's context."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return model, os.cpu_count(), usable


def bench_stream_read(args):
    """The achievable HBM read rate: a kernel that only reads (16-byte loads,
    256 threads, each workgroup issuing all its loads at once, chunks of 32 KB
    as a pair tile of the verification kernel), over the steady batch's 68 MB
    per launch, 16 rotating copies (over 4x the Infinity Cache)."""
    import ctypes
    import torch
    from draft_verification_spec_amd import _build
    lib = ctypes.CDLL(_build.STREAM_LIB)
    lib.sv_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.sv_stream_read.restype = ctypes.c_int
    vecs = 8
    chunk = 256 * 16 * vecs
    nbytes = (68067328 // chunk) * chunk
    copies = args.copies or max(1, -(-4 * MALL_BYTES // nbytes))
    bufs = [torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(nbytes // chunk, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        rc = lib.sv_stream_read(bufs[i % copies].data_ptr(), nbytes, vecs, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"sv_stream_read failed: {rc}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(args.warmup + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
    r1.record(stream)
    torch.cuda.synchronize()
    region_us = r0.elapsed_time(r1) * 1e3 / args.steps
    print(json.dumps({
        "metric": "stream-read GB/s (achievable HBM read rate)", "value": round(nbytes / (region_us * 1e-6) / 1e9, 1),
        "unit": "GB/s", "bytes_per_launch": nbytes, "chunk_bytes": chunk, "workgroups": nbytes // chunk,
        "input_copies_rotated": copies, "steps": args.steps, "kernel_us_mean": round(region_us, 3),
        "kernel_us_source": "events around the K timed launches on the launch stream, / K",
        "per_call_events_us_p10_p50_p90": [round(float(np.percentile(us, q)), 3) for q in (10, 50, 90)],
        "frac_of_8TBs": round(nbytes / (region_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="steady")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0: enough for 4x the MALL)")
    ap.add_argument("--eager", action="store_true", help="time K direct calls instead of HIP-graph replays")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--stream-read", action="store_true")
    ap.add_argument("--source-hash", default=None)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the verification step runs on a single MI355X "
              "(sharding over B or V is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.source_hash:
        print(source_hash(args.source_hash))
        return
    if args.copy_calib:
        return copy_calib()
    if args.stream_read:
        return bench_stream_read(args)
    if args.workload in ("kd", "kd_small"):
        return bench_kd(args)

    import torch
    import draft_verification_spec_amd as sv

    w = make_workload(args.workload)
    print(f"[bench] workload {describe(w)}", file=sys.stderr, flush=True)
    t, d, x, u = sv.to_device(w)
    greedy = w.temperature == 0
    alg = w.alg_bytes()
    copies = args.copies or max(1, -(-4 * MALL_BYTES // alg))
    sets = [(t, d, x, u)] + [(t.clone(), d.clone(), x.clone(), u.clone()) for _ in range(copies - 1)]
    shape = sv.make_shape(w.B, w.k, w.V, w.dtype, w.temperature)
    dev = t.device
    ws = torch.zeros(max(sv.spec_verify_workspace_bytes(shape), 256), dtype=torch.uint8, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    acc = torch.empty(w.B, **i32)
    out = torch.empty(w.B, w.k + 1, **i32)
    tv = torch.empty(w.B, w.k + 1, sv.TOPK, dtype=torch.float32, device=dev)
    ti = torch.empty(w.B, w.k + 1, sv.TOPK, **i32)
    st = torch.empty(w.B, **i32)
    aux = sv.sv_aux_t(st.data_ptr(), None, None, None, None, sv.SV_LAYOUT_AUTO)
    torch.cuda.synchronize()

    def call(i, stream):
        tt, dd, xx, uu = sets[i % copies]
        rc = sv.spec_verify(shape, tt.data_ptr(), None if greedy else dd.data_ptr(),
                            xx.data_ptr() if w.k > 0 else None, None if greedy else uu.data_ptr(),
                            acc.data_ptr(), out.data_ptr(), tv.data_ptr(), ti.data_ptr(), aux,
                            ws.data_ptr(), ws.numel(), stream)
        if rc != sv.SV_OK:
            raise sv.SpecVerifyError(rc)

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        call(i, stream.cuda_stream)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps over {copies} input copies",
          file=sys.stderr, flush=True)

    # events on the launch stream right before and after each of K direct
    # calls: a per-call distribution, each pair adding about 2 us of its own
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        call(args.warmup + i, stream.cuda_stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kern_ms = np.array([a.elapsed_time(b) for a, b in ev])

    # the timed region: K back-to-back steps, one launch each, bracketed by
    # events on the launch stream (the average launch duration) and by the
    # host clock (the whole-job rate)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.eager:
        timing = "eager: K direct calls back to back"
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        r0.record(stream)
        for i in range(args.steps):
            call(args.warmup + args.steps + i, stream.cuda_stream)
        r1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        # one graph of one call per input copy (and one for the remainder), captured on a side stream
        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream().cuda_stream
                for i in range(n):
                    call(i, cs)
            return g
        full, rest = divmod(args.steps, copies)
        g_full = capture(copies) if full else None
        g_rest = capture(rest) if rest else None
        torch.cuda.synchronize()
        if g_full is not None:
            g_full.replay()                # one untimed replay
        torch.cuda.synchronize()
        timing = f"HIP graph: {copies} calls per replay, {full} replays + {rest} calls"
        t0 = time.perf_counter()
        r0.record(stream)
        for _ in range(full):
            g_full.replay()
        if g_rest is not None:
            g_rest.replay()
        r1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    rows = w.B * (w.k + 1)
    value = alg / (ms_per_step * 1e-3) / 1e9
    kern_avg = r0.elapsed_time(r1) / args.steps       # ms per launch over the timed region
    achieved = alg / (kern_avg * 1e-3) / 1e9
    # the last step's outputs, from the last input copy used
    call(copies - 1, stream.cuda_stream)
    torch.cuda.synchronize()
    g = dict(accepted_len=acc.cpu().numpy(), out_tokens=out.cpu().numpy(), topk_val=tv.cpu().numpy(),
             topk_idx=ti.cpu().numpy(), status=st.cpu().numpy())
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype else "f32",
        "data": "synthetic (seeded Philox logits of the workload's shape and distribution)",
        "config": {"workload": describe(w), "B": w.B, "k": w.k, "V": w.V, "verified_rows": rows,
                   "alg_bytes_per_step": alg, "input_copies_rotated": copies, "timing": timing},
        "rows_per_s": round(rows / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counted_traffic("sv_verify", f"sv_verify_{w.name}_B{w.B}_k{w.k}_V{w.V}_"
                                                             f"{'bf16' if w.dtype else 'f32'}"),
                     "kernel": "sv_verify", "kernel_us_mean": round(kern_avg * 1e3, 3),
                     "kernel_us_source": "events around the K timed launches on the launch stream, / K",
                     "per_call_events_us_p10_p50_p90": [round(float(np.percentile(kern_ms, q)) * 1e3, 3)
                                                        for q in (10, 50, 90)]},
        "mean_accepted_len": float(np.mean(g["accepted_len"])),
        "mean_accepted_len_plus1": float(np.mean(g["accepted_len"]) + 1),
    }
    if not args.no_cpu:
        dt, n, o = cpu_baseline(w)
        from tests.compare import compare_decisions   # same comparator as the parity tests
        model, nthreads, usable = host_cpu()
        line["cpu_baseline"] = {
            "value": round(alg / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the full {describe(w)} batch, {n} pass(es), {dt:.2f} s per batch, one thread",
            "cpu_model": model, "host_threads": nthreads, "usable_threads": usable,
            "rows_per_s": round(rows / dt, 2)}
        if not greedy:
            rep = compare_decisions(o, g, w.k)
            line["parity_vs_oracle"] = {"fails": len(rep["fails"]), "exception_positions": rep["exc_pos"],
                                        "positions": rep["positions"]}
        else:
            line["parity_vs_oracle"] = {"bit_exact": bool(np.array_equal(o["out_tokens"], g["out_tokens"]))}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
