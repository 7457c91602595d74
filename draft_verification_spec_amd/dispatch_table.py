"""Measure the verification kernel's two item layouts over batch sizes and
draft lengths on the GPU, and write the table the library's SV_LAYOUT_AUTO
uses (csrc/sv_dispatch.h) with a summary (profiles/dispatch_layout_V151936.md).

    python -m draft_verification_spec_amd.dispatch_table     # on an MI355X; rebuild afterwards

Inputs are timing inputs only, generated on the device (seeded): target logits
N(0, 3^2), draft = target + N(0, 1), drafted tokens drawn from the draft
softmax by the Gumbel-max trick, uniforms U[0, 1).  Each configuration runs
both layouts back to back (several input copies rotate, up to 1 GB), 60 steps
each, five times in alternation; the table keeps the layout with the lower
best time.  The layouts give identical
results; only the order in which streaming workgroups take the (group, tile)
items differs.
"""
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
V = 151936

GRID = ([("bf16", False, B, k) for B in (1, 2, 4, 8, 16, 32, 64, 128, 256) for k in (0, 1, 2, 3, 4, 8, 15)]
        + [("f32", False, B, k) for B in (1, 8, 32, 128) for k in (0, 3, 15)]
        + [(dt, True, B, k) for dt in ("bf16", "f32") for B in (1, 8, 32, 128) for k in (3, 15)])


def make_inputs(torch, dt, greedy, B, k, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    t = torch.randn(B, k + 1, V, generator=g, device="cuda") * 3
    d = t[:, :k] + torch.randn(B, k, V, generator=g, device="cuda")
    gum = -torch.log(-torch.log(torch.rand(B, k, V, generator=g, device="cuda").clamp_min(1e-20)))
    x = (d + gum).argmax(dim=2).to(torch.int32) if not greedy else d.argmax(dim=2).to(torch.int32)
    u = torch.rand(B, k + 2, generator=g, device="cuda")
    tt = torch.bfloat16 if dt == "bf16" else torch.float32
    return t.to(tt), d.to(tt), x, u


def measure(torch, sv, dt, greedy, B, k, steps=60, rounds=5):
    t, d, x, u = make_inputs(torch, dt, greedy, B, k, 7000 + B * 31 + k)
    size = t.numel() * t.element_size() + (0 if greedy else d.numel() * d.element_size())
    copies = max(1, min(64, -(-(1 << 30) // size)))
    sets = [(t, d)] + [(t.clone(), d.clone()) for _ in range(copies - 1)]
    T = 0.0 if greedy else 1.0
    best = {}
    for rnd in range(rounds):
        for layout in (sv.SV_LAYOUT_LAUNCH, sv.SV_LAYOUT_XCD_RUNS):
            def step(i):
                a, b = sets[i % copies]
                sv.verify(a, None if greedy else b, x, None if greedy else u, T, layout=layout)
            for i in range(5):
                step(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                step(i)
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) / steps * 1e6
            best[layout] = min(best.get(layout, 1e30), us)
    del sets, t, d
    torch.cuda.empty_cache()
    return best


def main():
    import torch
    sys.path.insert(0, ROOT)
    import draft_verification_spec_amd as sv
    rows = []
    for dt, greedy, B, k in GRID:
        best = measure(torch, sv, dt, greedy, B, k)
        lay = min(best, key=best.get)
        rows.append((dt, greedy, B, k, best[sv.SV_LAYOUT_LAUNCH], best[sv.SV_LAYOUT_XCD_RUNS], lay))
        print(f"[dispatch] {dt} {'greedy' if greedy else 'sampling'} B={B} k={k}: launch "
              f"{best[sv.SV_LAYOUT_LAUNCH]:.2f} us, xcd runs {best[sv.SV_LAYOUT_XCD_RUNS]:.2f} us", flush=True)
    entries = ",\n".join(f"    {{{B}, {k}, {1 if dt == 'bf16' else 0}, {1 if greedy else 0}, {lay}}}"
                         for dt, greedy, B, k, _, _, lay in rows)
    header = f'''// sv_dispatch.h -- item layout per shape for the verification kernel, measured
// on MI355X by draft_verification_spec_amd/dispatch_table.py (V = {V}): for
// each (B, k, dtype, mode) the faster of launch order (1) and one run of items
// per XCD (2).  Timings: profiles/dispatch_layout_V{V}.md.
#pragma once
#include <stdint.h>

struct SvLayoutEntry {{
  int32_t B, k, dtype, greedy, layout;
}};
static const SvLayoutEntry kSvLayoutTable[] = {{
{entries},
    {{0, 0, -1, -1, 0}},  // (end marker)
}};
'''
    out_dir = os.environ.get("SV_DISPATCH_OUT", os.path.join(ROOT, "gpurun_out"))
    os.makedirs(out_dir, exist_ok=True)
    open(os.path.join(out_dir, "sv_dispatch.h"), "w").write(header)
    lines = ["| dtype | mode | B | k | launch order (us/step) | XCD runs (us/step) | table |",
             "|---|---|---|---|---|---|---|"]
    for dt, greedy, B, k, a, b, lay in rows:
        lines.append(f"| {dt} | {'greedy' if greedy else 'sampling'} | {B} | {k} | {a:.2f} | {b:.2f} | "
                     f"{'launch' if lay == sv.SV_LAYOUT_LAUNCH else 'xcd runs'} |")
    open(os.path.join(out_dir, f"dispatch_layout_V{V}.md"), "w").write("\n".join(lines) + "\n")
    print(f"[dispatch] wrote {out_dir}/sv_dispatch.h and dispatch_layout_V{V}.md", flush=True)


if __name__ == "__main__":
    main()
