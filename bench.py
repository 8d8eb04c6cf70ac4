#!/usr/bin/env python3
"""Benchmark of the MSDeformAttn hot path on one MI355X.

One step = one pass of the whole hot path over one batch of the encoder
workload (B=2, M=8, D=32, L=4 levels 76x106/38x53/19x27/8x13, S=Nq=10687, K=4,
fp32): reference points -> sampling locations -> L*K softmax -> core forward ->
core backward (grad_value, grad_sampling_locations, grad_attention_weights),
every kernel from libmsda.so, inputs
(seeded synthetic draws) resident in HBM before the timed region.

Prints ONE JSON line. ``value`` is queries/s of that fwd+bwd step (a HIP graph
of the step replayed K times). ``kernels`` gives every GPU kernel's average
duration, timed live with HIP event pairs that the library records around each
launch on the launch's own stream (msda_timing_*), and its algorithmic bytes
per launch; ``roofline`` is for the kernel with the largest share of the step.
``cpu_baseline`` is the fp64 oracle on the host.

    python bench.py [--steps K] [--warmup W] [--workload encoder_backward]

Counter runs for the HBM traffic of the kernels (rocprofv3 --pmc, one counter
per run) use ``--eager``; ``--copy-mib N`` runs only a plain elementwise copy
of N MiB (the calibration kernel for FETCH_SIZE / WRITE_SIZE), and
``--ingest-counters DIR [--copy-mib N]`` turns the four counter runs under DIR
(fetch/, write/, copy_fetch/, copy_write/) into profiles/traffic.json.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published peak
METRIC = "MSDeformAttn fwd/bwd queries/s and effective HBM GB/s (% of peak), encoder shape"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_MIB_DEFAULT = 256


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="encoder_backward",
                   help="workload name (the step always runs fwd+bwd)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-encoder-stack", action="store_true",
                   help="skip the 6-layer encoder stack measurement (projections + FFN around the core)")
    p.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph replay")
    p.add_argument("--no-extra-configs", action="store_true",
                   help="skip the decoder and large-batch bf16 forward timings")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="only run a plain copy of this many MiB, 5 times (counter calibration)")
    p.add_argument("--ingest-counters", default=None, metavar="DIR",
                   help="write profiles/traffic.json from rocprofv3 --pmc runs under DIR and exit")
    return p.parse_args()


def unique_value_bytes(loc, shapes, B, M, row_bytes):
    """(Bytes of the distinct value rows (b, s, m) -- D channels each -- that
    at least one in-map corner touches: what an ideal kernel must read of
    value; and the number of in-map corner reads, each one such row, that the
    forward's gathers serve from the caches.)"""
    import torch
    touched = torch.zeros(B, int((shapes[:, 0] * shapes[:, 1]).sum()), M, dtype=torch.bool, device=loc.device)
    _, Nq, _, L, K, _ = loc.shape
    start = 0
    corners = 0
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
                corners += int(ok.sum().item())
                row = (start + yi.clamp(0, H - 1) * W + xi.clamp(0, W - 1)).long()
                bidx = torch.arange(B, device=loc.device).view(B, 1, 1, 1).expand_as(row)
                midx = torch.arange(M, device=loc.device).view(1, 1, M, 1).expand_as(row)
                touched[bidx[ok], row[ok], midx[ok]] = True
        start += H * W
    return int(touched.sum().item()) * row_bytes, corners


def dense_levels(shapes, Nq, K):
    """The levels the backward treats as dense (no tile records): at least 24
    samples per pixel per batch and head, and at most 8 x 256 pixels. This
    mirrors the library's tile planner so that each backward kernel is
    charged for the levels it handles."""
    return [l for l, (H, W) in enumerate(shapes) if Nq * K >= 24 * H * W and H * W <= 8 * 256]


def algorithmic_bytes(B, M, D, Nq, shapes, K, vbytes):
    """Bytes each kernel must move at the least (read + write, fp32), per
    launch. `vbytes` = the distinct value rows the samples touch. Kernels that
    only touch workspace (clears) count the op's
    own arrays they read or write, and scratch-only ones count 0."""
    f32 = 4
    L = len(shapes)
    S = sum(H * W for H, W in shapes)
    samples = B * Nq * M * L * K
    per_level = B * Nq * M * K              # samples of one level
    rows = B * Nq * M * D * f32             # output / grad_output
    dense = dense_levels(shapes, Nq, K)
    dense_pix = sum(shapes[l][0] * shapes[l][1] for l in dense)
    # a dense level is split over queries when it has over 3072 samples
    split_pix = sum(shapes[l][0] * shapes[l][1] for l in dense if Nq * K > 3072)
    sparse_samples = per_level * (L - len(dense))
    dense_samples = per_level * len(dense)
    gv_row = B * M * D * f32                 # grad_value bytes per pixel
    return {
        "reference_points_kernel": B * L * 2 * f32 + B * Nq * L * 2 * f32,
        "sampling_locations_kernel": B * Nq * L * 2 * f32 + 2 * samples * 2 * f32,
        "softmax_vec_kernel": 2 * samples * f32,
        "forward_c256_kernel": vbytes + samples * 3 * f32 + rows,
        # the same op with the coarse levels staged in LDS (same algorithmic bytes)
        "forward_staged_kernel": vbytes + samples * 3 * f32 + rows,
        "zero_fill_kernel": S * gv_row,
        "clear_totals_kernel": 0,
        "bin_count_kernel": sparse_samples * 2 * f32,
        # value rows, loc, A, grad_output in; grad_loc, grad_A out
        "backward_c256_kernel": vbytes + samples * 3 * f32 + rows + samples * 3 * f32,
        # sparse levels: grad_output, their loc and A in, their grad_value rows
        # out; the sums of split dense levels ride along as extra items
        "tile_accum_kernel": rows + sparse_samples * 3 * f32 + (S - dense_pix + split_pix) * gv_row,
        # dense levels: grad_output, their loc and A in; grad_value rows out
        # for levels with one query split (the others park sums in workspace)
        "dense_accum_kernel": rows + dense_samples * 3 * f32 + (dense_pix - split_pix) * gv_row,
    }


def kernel_source_hash():
    """Hash of the kernel sources with comments and whitespace removed, so
    that counter figures stay attached to the code they were measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scale_deformable_attention_msdeformattn_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(f.encode() + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, only if they
    were taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    e = t.get("kernels", {}).get(kernel)
    return None if e is None else e.get("hbm_bytes_per_launch")


def _counter_rows(d, counter):
    """(kernel name, value in KiB) per dispatch from a rocprofv3 csv run."""
    out = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not out:
        raise SystemExit(f"no {counter} rows under {d}")
    return out


def _short_kernel_name(full):
    """'void ns::(anonymous namespace)::name<T, 8>(args)' -> 'name'. The fused
    instantiations of the c256 and staged kernels (last template argument
    true) get the names the library's own timing uses for them,
    forward_fused_c256_kernel, backward_fused_c256_kernel and
    forward_fused_staged_kernel, so their counters are kept apart."""
    head = full.replace("(anonymous namespace)", "")
    tmpl = head.split("(")[0]
    name = tmpl.split("<")[0]
    name = name.split("::")[-1].split()[-1] if name.strip() else name
    if name in ("forward_c256_kernel", "backward_c256_kernel") and tmpl.rstrip().endswith("true>"):
        name = name.replace("_c256", "_fused_c256")
    if name == "forward_staged_kernel" and tmpl.rstrip().endswith("true>"):
        name = "forward_fused_staged_kernel"
    return name


def ingest_counters(d, copy_mib, workload):
    """profiles/traffic.json from four rocprofv3 --pmc runs (csv output):
    d/fetch and d/write of `bench.py --eager`, d/copy_fetch and d/copy_write
    of `bench.py --copy-mib N`. Each kernel's per-dispatch KiB is averaged and
    scaled by the copy kernel's known bytes over its counter reading."""
    copy_kib = copy_mib * 1024.0

    def copy_avg(sub, counter):
        vals = [v for n, v in _counter_rows(os.path.join(d, sub), counter) if "vectorized_elementwise_kernel" in n]
        return sum(vals) / len(vals)

    fetch_scale = copy_kib / copy_avg("copy_fetch", "FETCH_SIZE")
    write_scale = copy_kib / copy_avg("copy_write", "WRITE_SIZE")
    names = list(algorithmic_bytes(1, 1, 1, 1, [(1, 1)], 1, 0))
    kernels = {}
    for counter, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        for full, v in _counter_rows(os.path.join(d, sub), counter):
            short = _short_kernel_name(full)
            if short not in names:
                continue
            e = kernels.setdefault(short, {"FETCH_SIZE": [], "WRITE_SIZE": []})
            e[counter].append(v)
    table = {}
    for k, e in kernels.items():
        if not e["FETCH_SIZE"] or not e["WRITE_SIZE"]:
            continue
        fk = sum(e["FETCH_SIZE"]) / len(e["FETCH_SIZE"])
        wk = sum(e["WRITE_SIZE"]) / len(e["WRITE_SIZE"])
        table[k] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                    "hbm_bytes_per_launch": int(round((fk * fetch_scale + wk * write_scale) * 1024)),
                    "dispatches": len(e["FETCH_SIZE"])}
    out = {"source_hash": kernel_source_hash(), "workload": workload,
           "calibration": {"kernel": "torch elementwise copy (mul by 1) fp32", "copy_mib": copy_mib,
                           "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4)},
           "kernels": table}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def copy_calibration(mib):
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "dispatches": 5}))


def encoder_stack(msda, shapes, lsi, vr, B, S, M, L, K, dev, args, n_layers=6):
    """Six Deformable-DETR encoder layers (MSDeformAttn with its four
    projections + FFN 1024 + layer norms, random init) forward and backward at
    the workload's shapes, fp32: time per step (eager, HIP events) and the
    share of it spent in libmsda's kernels."""
    import torch
    from scale_deformable_attention_msdeformattn_amd.layer import Encoder
    torch.manual_seed(0)
    enc = Encoder(n_layers=n_layers, d_model=256, d_ffn=1024, n_levels=L, n_heads=M, n_points=K).to(dev)
    src = torch.randn(B, S, 256, device=dev, requires_grad=True)
    pos = torch.randn(B, S, 256, device=dev)
    ref = msda.msda_reference_points(shapes, valid_ratios=vr)
    R = torch.randn(B, S, 256, device=dev)

    def step():
        enc.zero_grad(set_to_none=True)
        src.grad = None
        (enc(src, pos, ref, shapes, lsi) * R).sum().backward()

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    steps = max(3, min(args.steps, 10))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    step()
    torch.cuda.synchronize()
    msda.msda_timing_enable(False)
    core_ms = sum(v[0] for v in msda.msda_timing_read().values())
    msda.msda_timing_reset()
    return {"layers": n_layers, "ms_per_step": ms, "queries_per_s": B * S / (ms * 1e-3),
            "core_ms_per_step": core_ms, "core_share": core_ms / ms,
            "note": "fwd+bwd of the stack; core = libmsda kernels (fused forward/backward), the rest torch "
                    "GEMMs (fp32), layer norms and elementwise ops"}


def cpu_baseline(wl_name, min_seconds=10.0):
    """The fp64 oracle, as it stands (single-threaded C), on the same step:
    reference points, locations, softmax, forward and backward of the whole
    workload once."""
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


def forward_configs(msda, workloads, dev, args, names=("decoder", "encoder_bf16_large")):
    """The forward alone on the other forward workloads of the pages' shapes
    (the decoder's 300 object queries; the large batch with bf16 value):
    average kernel duration from the library's event pairs over 20 calls,
    queries/s and effective HBM GB/s over the algorithmic bytes (the distinct
    value rows touched, loc, A and the output)."""
    import torch
    out = {}
    for name in names:
        d = workloads.draw(name, 0)
        w = d.workload
        shapes = d.spatial_shapes
        lsi, _ = msda.level_start_index_host(shapes)
        vr = d.valid_ratios.to(dev)
        if w.encoder:
            ref = msda.msda_reference_points(shapes, valid_ratios=vr)
        else:
            ref = msda.msda_reference_points(shapes, valid_ratios=vr, query_ref=d.query_ref.to(dev))
        loc = msda.msda_sampling_locations(shapes, ref, d.offsets_px.to(dev))
        A = msda.msda_attention_softmax(shapes, d.logits.to(dev), w.points)
        value = d.value.to(dev)
        B, M, D, L, K, Nq = w.batch, w.heads, w.channels, w.levels, w.points, w.nq
        elem = value.element_size()
        vbytes, _ = unique_value_bytes(loc, shapes.to(dev), B, M, D * elem)
        alg = vbytes + B * Nq * M * L * K * 3 * 4 + B * Nq * M * D * 4
        for _ in range(5):
            msda.msda_forward(value, shapes, lsi, loc, A)
        torch.cuda.synchronize()
        msda.msda_timing_reset()
        msda.msda_timing_enable(True)
        n = 20
        for _ in range(n):
            msda.msda_forward(value, shapes, lsi, loc, A)
        torch.cuda.synchronize()
        msda.msda_timing_enable(False)
        t = msda.msda_timing_read()
        msda.msda_timing_reset()
        kernel, (ms, cnt) = max(t.items(), key=lambda kv: kv[1][0])
        us = ms * 1e3 / cnt
        gbps = alg / (us * 1e-6) / 1e9
        out[name] = {"workload": w.description, "kernel": kernel, "avg_us": round(us, 3),
                     "queries_per_s": B * Nq / (us * 1e-6), "algorithmic_bytes": alg,
                     "effective_gbps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        del value, loc, A, ref
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: this build runs on a "
              "single GPU (the op shards by batch or by head with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.ingest_counters:
        ingest_counters(args.ingest_counters, args.copy_mib or COPY_MIB_DEFAULT, args.workload)
        return
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return

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

    def k_bwd():
        state["grads"] = msda.msda_backward(value, shapes, lsi, state["loc"], state["A"], G)

    calls = [("msda_reference_points", k_ref), ("msda_sampling_locations", k_loc),
             ("msda_attention_softmax", k_softmax), ("msda_forward", k_fwd), ("msda_backward", k_bwd)]

    def step():
        for _, f in calls:
            f()

    # the fused path: reference points -> fused forward (locations and softmax
    # formed in the core, written out for the backward) -> fused backward
    # (gradients carried to the offsets, logits and reference points)
    logits_flat = logits.reshape(B, Nq, M, L * K)

    def fused_step():
        ref = msda.msda_reference_points(shapes, valid_ratios=vr)
        out, loc, A = msda.msda_forward_fused(value, shapes, lsi, ref, off, logits_flat)
        state["fused"] = (out, msda.msda_backward_fused(value, shapes, lsi, loc, A, G))

    # the same with 4-d box references (cx, cy, w, h): the encoder points with
    # a fixed box of 8 level-0 pixels, offsets relative to the box size
    box_ref = torch.cat([msda.msda_reference_points(shapes, valid_ratios=vr),
                         torch.full((B, Nq, L, 2), 8.0 / float(shapes[0, 1]), device=dev)], dim=-1).contiguous()

    def box_step():
        out, loc, A = msda.msda_forward_fused(value, shapes, lsi, box_ref, off, logits_flat)
        state["box"] = (out, msda.msda_backward_fused(value, shapes, lsi, loc, A, G, box_references=box_ref,
                                                      sampling_offsets=off))

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()

    vbytes, corner_reads = unique_value_bytes(state["loc"], shapes.to(dev), B, M, D * elem)
    alg = algorithmic_bytes(B, M, D, Nq, [tuple(int(v) for v in hw) for hw in shapes.tolist()], K, vbytes)

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

    # ---- timed region 1b: the fused steps, graph replay like region 1 ----
    def graph_time(fn, key):
        try:
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            s2 = torch.cuda.Stream(dev)
            s2.wait_stream(stream)
            with torch.cuda.stream(s2):
                fn()
            stream.wait_stream(s2)
            torch.cuda.synchronize()
            eager = state[key][0].clone()
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2):
                fn()
            g2.replay()
            torch.cuda.synchronize()
            if not torch.equal(state[key][0], eager):
                raise RuntimeError(f"{key} graph replay differs from eager")
            for _ in range(args.warmup):
                g2.replay()
            torch.cuda.synchronize()
            f0 = torch.cuda.Event(enable_timing=True)
            f1 = torch.cuda.Event(enable_timing=True)
            f0.record(stream)
            for _ in range(args.steps):
                g2.replay()
            f1.record(stream)
            torch.cuda.synchronize()
            return f0.elapsed_time(f1) / args.steps
        except Exception as e:  # report, do not hide
            print(f"[bench] {key} step not timed ({e})", file=sys.stderr)
            return None

    fused_ms = graph_time(fused_step, "fused")
    box_ms = graph_time(box_step, "box")

    # ---- timed region 2: per entry point, events between the calls of eager
    # steps on the same stream ----
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[i][0].record(stream)
        for j, (_, f) in enumerate(calls):
            f()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    per_call = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)])) * 1e3
                for j, (name, _) in enumerate(calls)}  # microseconds
    eager_step_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][-1]) for i in range(args.steps)]))

    # ---- timed region 3: every GPU kernel, event pairs recorded by the
    # library around each launch on its stream ----
    torch.cuda.synchronize()
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    msda.msda_timing_enable(False)
    timing = msda.msda_timing_read()
    msda.msda_timing_reset()
    # the fused step's kernels, in a session of their own
    msda.msda_timing_enable(True)
    for _ in range(args.steps):
        fused_step()
    torch.cuda.synchronize()
    msda.msda_timing_enable(False)
    timing_fused = msda.msda_timing_read()
    msda.msda_timing_reset()

    kstats = {}
    for name, (ms, n) in timing.items():
        us = ms * 1e3 / n
        e = {"avg_us": round(us, 3), "launches_per_step": n / args.steps}
        if name in alg:
            gbps = alg[name] / (us * 1e-6) / 1e9
            e.update({"algorithmic_bytes": alg[name], "gbps": round(gbps, 1),
                      "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)})
        kstats[name] = e
    dominant = max((k for k in kstats if k in alg), key=lambda k: kstats[k]["avg_us"])
    dom_us = kstats[dominant]["avg_us"]
    dom_gbps = alg[dominant] / (dom_us * 1e-6) / 1e9
    queries = B * Nq
    # the forward kernel this shape takes (coarse levels staged in LDS, or one wave per query)
    fwd_name = next((k for k in ("forward_staged_kernel", "forward_c256_kernel") if k in kstats), None)
    fwd = kstats.get(fwd_name, {}) if fwd_name else {}
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
        "data": "synthetic (seeded draws with Deformable DETR's encoder shapes and distributions; no dataset)",
        "config": {"workload": w.description, "step": "reference points + locations + softmax + forward + "
                   "backward", "graph_replay": graph is not None},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dominant), "avg_us": dom_us,
                     "algorithmic_bytes": alg[dominant]},
        "kernels": kstats,
        "entry_points_us": {k: round(v, 3) for k, v in per_call.items()},
        "eager_ms_per_step": eager_step_ms,
        "forward": {"kernel": fwd_name, "queries_per_s": queries / (fwd["avg_us"] * 1e-6) if fwd else None,
                    "effective_gbps": fwd.get("gbps"), "frac_of_hbm_peak": fwd.get("frac_of_hbm_peak"),
                    "traffic": measured_traffic(fwd_name) if fwd_name else None,
                    "gather": None if not fwd else {
                        "corner_reads": corner_reads, "bytes": corner_reads * D * elem,
                        "tbps": round(corner_reads * D * elem / (fwd["avg_us"] * 1e-6) / 1e12, 2),
                        "note": "in-map corner reads of one head's value row each; the fine levels' are served by "
                                "L1/L2 (we measured 50-58 B/clk/CU for 16-byte lane gathers on that path, 31-36 TB/s "
                                "on 256 CUs at 2.4 GHz), the coarse levels' from LDS when they are staged"}},
        "backward": {"queries_per_s": queries / (per_call["msda_backward"] * 1e-6),
                     "note": "the whole msda_backward call, all its kernels",
                     "main_kernel_gather": None if "backward_c256_kernel" not in kstats else {
                         "corner_reads": corner_reads, "bytes": corner_reads * D * elem,
                         "tbps": round(corner_reads * D * elem / (kstats["backward_c256_kernel"]["avg_us"] * 1e-6)
                                       / 1e12, 2),
                         "note": "backward_c256 gathers the same in-map corner rows as the forward, all through "
                                 "the L1/L2 path (31-36 TB/s measured ceiling on 256 CUs)"}},
        "fused_step": None if fused_ms is None else {
            "ms_per_step": fused_ms, "queries_per_s": queries / (fused_ms * 1e-3),
            "kernels_avg_us": {k: round(v[0] * 1e3 / v[1], 3) for k, v in timing_fused.items()},
            "step": "reference points + msda_forward_fused + msda_backward_fused (gradients to value, offsets, "
                    "logits and reference points)"},
        "fused_box_step": None if box_ms is None else {
            "ms_per_step": box_ms, "queries_per_s": queries / (box_ms * 1e-3),
            "step": "msda_forward_fused + msda_backward_fused with 4-d box references (gradients to value, "
                    "offsets, logits and boxes)"},
    }
    if not args.no_encoder_stack:
        result["encoder_stack"] = encoder_stack(msda, shapes, lsi, vr, B, S, M, L, K, dev, args)
    if not args.no_extra_configs:
        result["other_forward_configs"] = forward_configs(msda, workloads, dev, args)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
