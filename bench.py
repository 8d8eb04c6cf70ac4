#!/usr/bin/env python3
"""Benchmark of the MSDeformAttn hot path on one MI355X.

One step = one pass of the whole hot path over one batch of the encoder
workload (B=2, M=8, D=32, L=4 levels 76x106/38x53/19x27/8x13, S=Nq=10687, K=4,
fp32): reference points -> sampling locations -> L*K softmax -> core forward ->
grad_value zero fill -> core backward, every kernel from libmsda.so, inputs
(seeded synthetic draws) resident in HBM before the timed region.

Prints ONE JSON line. ``value`` is queries/s of that fwd+bwd step; the
``roofline`` object is for the kernel with the largest share of the step, with
its algorithmic bytes divided by its average duration measured here with HIP
events on the stream it runs on; ``cpu_baseline`` is the fp64 oracle on the
host. Per-kernel and forward-only figures are included as extra keys.

    python bench.py [--steps K] [--warmup W] [--workload encoder]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published peak
METRIC = "MSDeformAttn fwd/bwd queries/s and effective HBM GB/s (% of peak), encoder shape"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="encoder_backward",
                   help="workload name (the step always runs fwd+bwd)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph replay")
    p.add_argument("--only", default=None, help="time only this kernel in a loop (for profiling runs)")
    return p.parse_args()


def unique_value_bytes(loc, shapes, B, M, row_bytes):
    """Bytes of the distinct value rows (b, s, m) -- D channels each -- that
    at least one in-map corner touches: what an ideal kernel must read of
    value."""
    import torch
    touched = torch.zeros(B, int((shapes[:, 0] * shapes[:, 1]).sum()), M, dtype=torch.bool, device=loc.device)
    _, Nq, _, L, K, _ = loc.shape
    start = 0
    for l in range(L):
        H, W = int(shapes[l, 0]), int(shapes[l, 1])
        x = loc[:, :, :, l, :, 0].double() * W - 0.5
        y = loc[:, :, :, l, :, 1].double() * H - 0.5
        x0 = torch.floor(x)
        y0 = torch.floor(y)
        for dy in (0, 1):
            for dx in (0, 1):
                xi = x0 + dx
                yi = y0 + dy
                ok = (xi >= 0) & (xi < W) & (yi >= 0) & (yi < H)
                row = (start + yi.clamp(0, H - 1) * W + xi.clamp(0, W - 1)).long()
                bidx = torch.arange(B, device=loc.device).view(B, 1, 1, 1).expand_as(row)
                midx = torch.arange(M, device=loc.device).view(1, 1, M, 1).expand_as(row)
                touched[bidx[ok], row[ok], midx[ok]] = True
        start += H * W
    return int(touched.sum().item()) * row_bytes


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scale_deformable_attention_msdeformattn_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, only if they
    were taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(wl_name, min_seconds=10.0):
    """The fp64 oracle, as it stands (single-threaded C), on the same step:
    reference points, locations, softmax, forward and backward of the whole
    workload once."""
    import numpy as np
    import oracle
    from scale_deformable_attention_msdeformattn_amd import workloads
    d = workloads.draw(wl_name, 0)
    w = d.workload
    shapes = d.spatial_shapes.numpy()
    # host-side input upcasts are not timed
    vr, off, logits, G, value = (oracle._f64(x) for x in (d.valid_ratios, d.offsets_px, d.logits,
                                                          d.grad_output, d.value))
    passes = 0
    t0 = time.perf_counter()
    while True:  # whole passes until at least min_seconds of CPU work
        lsi, _ = oracle.level_start_index(shapes)
        ref = oracle.reference_points_encoder(shapes, vr)
        loc = oracle.sampling_locations(shapes, ref, off)
        A = oracle.softmax(logits, w.levels * w.points).reshape(w.batch, w.nq, w.heads, w.levels, w.points)
        oracle.forward(value, shapes, lsi, loc, A)
        oracle.backward(value, shapes, lsi, loc, A, G)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    q = w.batch * w.nq
    return {"value": passes * q / dt, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} whole passes of the {w.name} workload ({q} queries each: reference points, "
                      f"locations, softmax, forward, backward), single-threaded fp64 C, {dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by batch or head without any exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import scale_deformable_attention_msdeformattn_amd as msda
    from scale_deformable_attention_msdeformattn_amd import workloads

    msda.load()
    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.device("cuda:0")
    d = workloads.draw(args.workload, 0)
    w = d.workload
    assert w.encoder, "the step computes encoder reference points"
    B, M, D, L, K, S, Nq = w.batch, w.heads, w.channels, w.levels, w.points, w.num_value, w.nq
    shapes = d.spatial_shapes
    lsi, _ = msda.level_start_index_host(shapes)
    value = d.value.to(dev)
    vr = d.valid_ratios.to(dev)
    off = d.offsets_px.to(dev)
    logits = d.logits.to(dev)
    G = (d.grad_output if d.grad_output is not None else torch.randn(B, Nq, M * D)).to(dev)
    elem = value.element_size()
    stream = torch.cuda.current_stream(dev)

    state = {}

    def k_ref():
        state["ref"] = msda.msda_reference_points(shapes, valid_ratios=vr)

    def k_loc():
        state["loc"] = msda.msda_sampling_locations(shapes, state["ref"], off)

    def k_softmax():
        state["A"] = msda.msda_attention_softmax(shapes, logits, K)

    def k_fwd():
        state["out"] = msda.msda_forward(value, shapes, lsi, state["loc"], state["A"])

    def k_bwd():  # grad_value zero fill (a small kernel of its own) + backward
        state["grads"] = msda.msda_backward(value, shapes, lsi, state["loc"], state["A"], G)

    kernels = [("reference_points", k_ref), ("sampling_locations", k_loc), ("attention_softmax", k_softmax),
               ("forward", k_fwd), ("backward", k_bwd)]

    def step():
        for _, f in kernels:
            f()

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()

    if args.only:
        f = dict(kernels)[args.only]
        for _ in range(args.steps):
            f()
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "steps": args.steps}))
        return

    # algorithmic bytes per launch
    loc = state["loc"]
    vbytes = unique_value_bytes(loc, shapes.to(dev), B, M, D * elem)
    f32 = 4
    alg = {
        "reference_points": B * L * 2 * f32 + B * Nq * L * 2 * f32,
        "sampling_locations": B * Nq * L * 2 * f32 + 2 * B * Nq * M * L * K * 2 * f32,
        "attention_softmax": 2 * B * Nq * M * L * K * f32,
        "forward": vbytes + B * Nq * M * L * K * 3 * f32 + B * Nq * M * D * f32,
        # reads value, loc, A, G; writes grad_value (fp32), grad_loc, grad_A
        "backward": vbytes + B * Nq * M * L * K * 3 * f32 + B * Nq * M * D * f32
                    + B * S * M * D * f32 + B * Nq * M * L * K * 3 * f32,
    }

    # ---- timed region 1: whole steps (graph replay unless --eager) ----
    graph = None
    if not args.eager:
        try:
            s = torch.cuda.Stream(dev)
            s.wait_stream(stream)
            with torch.cuda.stream(s):
                step()
            stream.wait_stream(s)
            torch.cuda.synchronize()
            eager_out = state["out"].clone()
            eager_gv = state["grads"][0].clone()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            for _ in range(3):  # every replay must match eager (fill kernels, no memset nodes)
                graph.replay()
                torch.cuda.synchronize()
                if not (torch.equal(state["out"], eager_out) and
                        torch.allclose(state["grads"][0], eager_gv, rtol=0, atol=1e-4)):
                    raise RuntimeError("graph replay differs from eager")
        except Exception as e:  # fall back to eager timing, and say so
            print(f"[bench] graph capture unavailable ({e}); timing eager launches", file=sys.stderr)
            graph = None
    run = graph.replay if graph is not None else step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        run()
    t1.record(stream)
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / args.steps

    # ---- timed region 2: per-kernel durations, events between the kernels of
    # eager steps on the same stream ----
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[i][0].record(stream)
        for j, (_, f) in enumerate(kernels):
            f()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    per = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)])) * 1e3
           for j, (name, _) in enumerate(kernels)}  # microseconds
    eager_step_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][-1]) for i in range(args.steps)]))

    # ---- timed region 3: the backward kernel alone (accumulate mode, so the
    # zero fill that msda_backward otherwise enqueues first is left out) ----
    acc = torch.zeros(B, S, M, D, dtype=torch.float32, device=dev)
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for _ in range(args.steps):
        msda.msda_backward(value, shapes, lsi, state["loc"], state["A"], G, grad_value=acc)
    b1.record(stream)
    torch.cuda.synchronize()
    bwd_kernel_us = b0.elapsed_time(b1) / args.steps * 1e3
    per["grad_value_zero_fill"] = max(per["backward"] - bwd_kernel_us, 0.0)
    per["backward"] = bwd_kernel_us
    alg["grad_value_zero_fill"] = B * S * M * D * f32

    kstats = {}
    for name, us in per.items():
        gbps = alg[name] / (us * 1e-6) / 1e9
        kstats[name] = {"avg_us": round(us, 3), "algorithmic_bytes": alg[name], "gbps": round(gbps, 1),
                        "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    dominant = max(per, key=per.get)
    dom_gbps = alg[dominant] / (per[dominant] * 1e-6) / 1e9
    traffic = measured_traffic(dominant)
    queries = B * Nq
    result = {
        "metric": METRIC,
        "value": queries / (step_ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if value.dtype == torch.float32 else "bf16 value, f32 compute",
        "data": "synthetic (seeded draws with the pages' shapes and distributions; no dataset)",
        "config": {"workload": w.description, "step": "reference points + locations + softmax + forward + "
                   "grad_value zero fill + backward", "graph_replay": graph is not None},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "kernels": kstats,
        "eager_ms_per_step": eager_step_ms,
        "forward": {"queries_per_s": queries / (per["forward"] * 1e-6),
                    "effective_gbps": kstats["forward"]["gbps"],
                    "frac_of_hbm_peak": kstats["forward"]["frac_of_hbm_peak"]},
        "backward": {"queries_per_s": queries / (per["backward"] * 1e-6),
                     "effective_gbps": kstats["backward"]["gbps"],
                     "frac_of_hbm_peak": kstats["backward"]["frac_of_hbm_peak"]},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
