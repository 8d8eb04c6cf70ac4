#!/usr/bin/env python3
"""Benchmark of the MSDeformAttn hot path on one MI355X.

One step = one pass of the whole hot path over one batch of the encoder
workload (B=2, M=8, D=32, L=4 levels 76x106/38x53/19x27/8x13, S=Nq=10687, K=4,
fp32): reference points -> sampling locations -> L*K softmax -> core forward ->
core backward (grad_value, grad_sampling_locations, grad_attention_weights),
every kernel from libmsda.so, inputs
(seeded synthetic draws) resident in HBM before the timed region.

Prints ONE JSON line. ``value`` is queries/s of that fwd+bwd step (a HIP graph
of the step replayed K times back to back: warm, the step's ~100 MB stay in
the 256 MB Infinity Cache). ``kernels`` gives every GPU kernel's average
duration, timed live with HIP event pairs that the library records around each
launch on the launch's own stream (msda_timing_*), and its algorithmic bytes
per launch; ``roofline`` is for the kernel with the largest share of the step
(warm event timing). ``cold`` times every entry point again with L2 and the
Infinity Cache evicted before each call (a 1 GiB read in between), and
``copy_ceiling`` is a plain device copy's rate, beside the 8 TB/s peak.
``cpu_baseline`` is the fp64 oracle on the host's cores (and on one core).

    python bench.py [--steps K] [--warmup W] [--workload encoder_backward]

Counter runs (rocprofv3 --pmc, one pass of COUNTER_PASSES per run) use
``--eager --profile-run``; ``--copy-mib N`` runs only a plain elementwise copy
of N MiB (a check of the byte counting: it must read and write N MiB), and
``--ingest-counters DIR`` turns the passes under DIR/<pass> into
profiles/traffic.json and profiles/counters_encoder_step.md, and
``--trace-summary DIR`` turns a ``rocprofv3 --kernel-trace --stats`` run of
this script (csv output under DIR) into profiles/kernel_trace_encoder_step.md.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published peak
METRIC = "MSDeformAttn fwd/bwd queries/s and effective HBM GB/s (% of peak), encoder shape"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COUNTERS_MD = os.path.join(ROOT, "profiles", "counters_encoder_step.md")
TRACE_MD = os.path.join(ROOT, "profiles", "kernel_trace_encoder_step.md")
FLUSH_BYTES = 1 << 30   # read between cold calls: 4x the 256 MB Infinity Cache, 32x all L2

# rocprofv3 --pmc passes read by --ingest-counters, one run each on
# `bench.py --eager --profile-run` (rocprofv3 does not split counters over
# runs: at most 8 SQ, 4 TCC, 4 TCP, 2 TA, 2 TD and 2 GRBM counters per pass).
COUNTER_PASSES = {
    # L2 -> fabric reads by request size (exact bytes) and writes (64 B or 32 B)
    "tcc_read": ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum"],
    "tcc_write_hit": ["TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum"],
    "sq_time": ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY",
                "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_LDS"],
    "sq_insts": ["SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
                 "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS_ATOMIC", "SQ_ACTIVE_INST_ANY"],
    "units": ["TA_TA_BUSY_sum", "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TD_TC_STALL_sum", "TD_TD_BUSY_sum",
              "TCP_TOTAL_CACHE_ACCESSES_sum", "TCP_TCC_READ_REQ_sum", "TCP_TCC_ATOMIC_WITHOUT_RET_REQ_sum",
              "TCP_TCC_ATOMIC_WITH_RET_REQ_sum", "GRBM_GUI_ACTIVE", "GRBM_COUNT"],
}


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
    p.add_argument("--profile-run", action="store_true",
                   help="only the plain step, eager, for counter passes (no fused steps, timing loops or extras)")
    p.add_argument("--cold-iters", type=int, default=20,
                   help="calls per entry point in the cold-cache timing (0 skips it)")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="only run a plain copy of this many MiB, 5 times (a check of the counters' byte counts)")
    p.add_argument("--trace-summary", default=None, metavar="DIR",
                   help="write profiles/kernel_trace_encoder_step.md from a rocprofv3 --kernel-trace --stats run "
                        "of this script with the same --steps and --warmup (csv output under DIR)")
    p.add_argument("--ingest-counters", default=None, metavar="DIR",
                   help="write profiles/traffic.json and the counter summary from rocprofv3 --pmc passes under "
                        "DIR/<pass> and exit")
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
    """The levels the backward treats as dense (no tile records): the last
    run of adjacent levels with at least 24 samples per pixel per batch and
    head and at most 2048 pixels. This mirrors the library's tile planner so
    that each backward kernel is charged for the levels it handles."""
    out = []
    for l, (H, W) in enumerate(shapes):
        if Nq * K >= 24 * H * W and H * W <= 2048:
            out.append(l)
        elif out:
            out = []
    return out


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
    # the dense levels are split over queries when they have over 3072 samples
    split_pix = dense_pix if Nq * K * len(dense) > 3072 else 0
    sparse_samples = per_level * (L - len(dense))
    dense_samples = per_level * len(dense)
    gv_row = B * M * D * f32                 # grad_value bytes per pixel
    return {
        "reference_points_kernel": B * L * 2 * f32 + B * Nq * L * 2 * f32,
        "sampling_locations_kernel": B * Nq * L * 2 * f32 + 2 * samples * 2 * f32,
        "softmax_vec_kernel": 2 * samples * f32,
        # the three above in one launch: the reference points are not read back
        "prologue_kernel": B * L * 2 * f32 + B * Nq * L * 2 * f32 + 2 * samples * 2 * f32 + 2 * samples * f32,
        "forward_c256_kernel": vbytes + samples * 3 * f32 + rows,
        # the same op with the coarse levels staged in LDS (same algorithmic bytes)
        "forward_staged_kernel": vbytes + samples * 3 * f32 + rows,
        "zero_fill_kernel": S * gv_row,
        "clear_totals_kernel": 0,
        "bin_count_kernel": sparse_samples * 2 * f32,
        # the same binning grouped per (batch, head, query range)
        "bin_count_head_kernel": sparse_samples * 2 * f32,
        # value rows, loc, A, grad_output in; grad_loc, grad_A out
        "backward_c256_kernel": vbytes + samples * 3 * f32 + rows + samples * 3 * f32,
        # the same outputs per (batch, head, query range), coarse levels staged in LDS
        "backward_head_kernel": vbytes + samples * 3 * f32 + rows + samples * 3 * f32,
        # sparse levels: grad_output in, their grad_value rows out (each
        # sample's cell and weights come from its records, in the workspace)
        "tile_accum_kernel": rows + (S - dense_pix) * gv_row,
        # the dense levels split over queries: their grad_value rows out (the
        # split sums come from the workspace)
        "dense_reduce_kernel": split_pix * gv_row,
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


def _counter_rows(d):
    """{(kernel name, counter): [values per dispatch]} from rocprofv3 csv runs under d."""
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                key = (_short_kernel_name(r["Kernel_Name"]), r["Counter_Name"])
                out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


def _short_kernel_name(full):
    """'void ns::(anonymous namespace)::name<T, 8>(args)' -> 'name'. The fused
    instantiations of the c256 and staged kernels (last template argument
    true) get the names the library's own timing uses for them,
    forward_fused_c256_kernel, backward_fused_c256_kernel,
    forward_fused_staged_kernel and backward_fused_head_kernel, so their
    counters are kept apart."""
    head = full.replace("(anonymous namespace)", "")
    tmpl = head.split("(")[0]
    name = tmpl.split("<")[0]
    name = name.split("::")[-1].split()[-1] if name.strip() else name
    if name in ("forward_c256_kernel", "backward_c256_kernel") and tmpl.rstrip().endswith("true>"):
        name = name.replace("_c256", "_fused_c256")
    if name == "forward_staged_kernel" and tmpl.rstrip().endswith("true>"):
        name = "forward_fused_staged_kernel"
    if name == "backward_head_kernel" and tmpl.rstrip().endswith("true>"):
        name = "backward_fused_head_kernel"
    return name


def ingest_counters(d, workload):
    """profiles/traffic.json and profiles/counters_encoder_step.md from the
    COUNTER_PASSES runs under d/<pass> (csv output of rocprofv3 --pmc on
    `bench.py --eager --profile-run`). Per kernel the counters are averaged
    over its dispatches. L2 -> fabric bytes are exact: reads are counted by
    request size (32, 64 and 128 B) and writes as 64 B or 32 B requests.
    These bytes include what the 256 MB Infinity Cache (memory-side) serves,
    so they bound the DRAM bytes from above."""
    rows = {}
    hashes = set()
    for name in COUNTER_PASSES:
        sub = os.path.join(d, name)
        if not os.path.isdir(sub):
            raise SystemExit(f"missing counter pass {sub}")
        rows.update(_counter_rows(sub))
        # the profiled run's own line names the kernel sources it ran on
        for log in glob.glob(os.path.join(sub, "*.log")):
            for ln in open(log):
                if ln.startswith("{") and "profile_run" in ln:
                    hashes.add(json.loads(ln)["source_hash"])
    if len(hashes) != 1:
        raise SystemExit(f"the passes under {d} do not name one kernel-source hash: {sorted(hashes)}")
    source_hash = hashes.pop()
    names = sorted({k for k, _ in rows})
    w = __import__("scale_deformable_attention_msdeformattn_amd.workloads", fromlist=["WORKLOADS"]).WORKLOADS[workload]
    shapes = [tuple(hw) for hw in w.spatial_shapes]
    # every value row is touched at this workload (the bench line's unique-bytes count says 100%)
    vbytes = w.batch * w.num_value * w.heads * w.channels * 4
    alg = algorithmic_bytes(w.batch, w.heads, w.channels, w.nq, shapes, w.points, vbytes)
    table = {}
    for k in names:
        c = {cn: sum(v) / len(v) for (kn, cn), v in rows.items() if kn == k}
        if "TCC_EA0_RDREQ_sum" not in c or "TCC_EA0_WRREQ_sum" not in c:
            continue
        n32, n64, n128 = (c.get(f"TCC_EA0_RDREQ_{b}B_sum", 0.0) for b in (32, 64, 128))
        rd = 32 * n32 + 64 * n64 + 128 * n128
        wr = 64 * c["TCC_EA0_WRREQ_64B_sum"] + 32 * (c["TCC_EA0_WRREQ_sum"] - c["TCC_EA0_WRREQ_64B_sum"])
        hit, miss = c.get("TCC_HIT_sum", 0.0), c.get("TCC_MISS_sum", 0.0)
        e = {"dispatches": len(rows[(k, "TCC_EA0_RDREQ_sum")]),
             "read_bytes": int(round(rd)), "write_bytes": int(round(wr)),
             "hbm_bytes_per_launch": int(round(rd + wr)),
             "read_requests_other_sizes": int(round(c["TCC_EA0_RDREQ_sum"] - n32 - n64 - n128)),
             "l2_hit_rate": round(hit / (hit + miss), 4) if hit + miss else None}
        if k in alg and alg[k]:
            e["algorithmic_bytes"] = alg[k]
            e["hbm_over_algorithmic"] = round((rd + wr) / alg[k], 3)
        for cn in ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR", "SQ_INSTS_LDS",
                   "SQ_INSTS_SALU", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS_ATOMIC", "TCP_TCC_ATOMIC_WITHOUT_RET_REQ_sum",
                   "TCP_TCC_ATOMIC_WITH_RET_REQ_sum", "GRBM_GUI_ACTIVE"):
            if cn in c:
                e[cn] = int(round(c[cn]))
        if c.get("SQ_WAVE_CYCLES"):
            e["wait_inst_share"] = round(c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"], 3)
            e["wait_any_share"] = round(c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"], 3)
        if c.get("GRBM_GUI_ACTIVE"):
            # GRBM_GUI_ACTIVE sums the 8 XCDs' busy cycles; SQ_INSTS_VALU counts
            # wave instructions, each 4 cycles of a 16-lane SIMD (1024 SIMDs)
            busy = c["GRBM_GUI_ACTIVE"] / 8
            e["valu_share_of_busy"] = round(c.get("SQ_INSTS_VALU", 0.0) * 4 / 1024 / busy, 3)
            e["ta_busy_share"] = round(c.get("TA_TA_BUSY_sum", 0.0) / (256 * busy), 3)
        table[k] = e
    out = {"source_hash": source_hash, "workload": workload,
           "command": "rocprofv3 --pmc <pass counters> --output-format csv -d DIR/<pass> -o run -- "
                      "python3 bench.py --eager --profile-run --steps 3 --warmup 1 > DIR/<pass>/bench.log",
           "passes": COUNTER_PASSES,
           "bytes": "L2 -> fabric (Infinity Cache included): reads by request size, writes 64 B or 32 B",
           "kernels": table}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    _counter_summary(out)
    print(json.dumps(out))


def _counter_summary(t):
    lines = [f"# Counters per kernel — {t['workload']} step (plain path), one MI355X", "",
             "Generated by `python bench.py --ingest-counters DIR` from the rocprofv3 passes below, each run as",
             "", "```", "cd /tmp && export TMPDIR=/tmp",
             "rocprofv3 --pmc <counters of the pass> --output-format csv -d <out>/pmc/<pass> -o run \\",
             "    -- python3 <repo>/bench.py --eager --profile-run --steps 3 --warmup 1 \\",
             "    > <out>/pmc/<pass>/bench.log", "```", ""]
    for k, v in t["passes"].items():
        lines.append(f"- `{k}`: {', '.join(v)}")
    lines += ["", f"Kernel sources hash `{t['source_hash']}`. Bytes are L2 -> fabric traffic, exact by request "
              "size; the Infinity Cache serves part of it, so DRAM bytes are at most these.", "",
              "| kernel | disp. | read MB | write MB | / algorithmic | L2 hit | VALU share of busy | TA busy | "
              "wait (inst) | LDS bank conflicts / LDS inst |",
              "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for k, e in sorted(t["kernels"].items(), key=lambda kv: -kv[1]["hbm_bytes_per_launch"]):
        conf = "" if not e.get("SQ_INSTS_LDS") else f"{e.get('SQ_LDS_BANK_CONFLICT', 0) / e['SQ_INSTS_LDS']:.2f}"
        hit = "" if e["l2_hit_rate"] is None else f"{100 * e['l2_hit_rate']:.1f}%"
        ratio = f"{e['hbm_over_algorithmic']:.2f}x" if "hbm_over_algorithmic" in e else ""
        lines.append(
            f"| `{k}` | {e['dispatches']} | {e['read_bytes'] / 1e6:.1f} | {e['write_bytes'] / 1e6:.1f} | {ratio} | "
            f"{hit} | {e.get('valu_share_of_busy', float('nan')):.2f} | {e.get('ta_busy_share', float('nan')):.2f} | "
            f"{e.get('wait_inst_share', float('nan')):.2f} | {conf} |")
    with open(COUNTERS_MD, "w") as f:
        f.write("\n".join(lines) + "\n")


LIB_KERNELS = ("prologue_kernel", "reference_points_kernel", "sampling_locations_kernel", "softmax_vec_kernel", "forward_",
               "bin_count", "backward_", "clear_totals_kernel", "tile_accum_kernel", "dense_accum_kernel",
               "dense_reduce_kernel", "zero_", "ref_grad_sum_kernel", "fused_grads_kernel")


def trace_summary(d, steps, warmup):
    """profiles/kernel_trace_encoder_step.md from the kernel trace of
    `bench.py --steps K --warmup W` under rocprofv3 --kernel-trace --stats.
    The run's plain steps (the prologue kernel, then the forward, ...) come
    in this order: max(1, W) warm-up steps and one captured step
    (eager), 3 + W + K graph replays, then K eager steps timed per entry
    point and K eager steps timed per kernel by the library's event pairs
    (the figures of the bench line). Per kernel: rocprofv3's average over
    every launch of the run, and the medians over the graph replays and over
    the library-timed eager steps; then the timeline of the median graph
    replay."""
    import statistics as st
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        raise SystemExit(f"no kernel_stats/kernel_trace csv under {d}")
    all_avg = {}
    for r in csv.DictReader(open(stats[0])):
        n = _short_kernel_name(r["Name"])
        if n.startswith(LIB_KERNELS):
            c, t = all_avg.get(n, (0, 0.0))
            all_avg[n] = (c + int(r["Calls"]), t + float(r["TotalDurationNs"]))
    rows = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short_kernel_name(r["Kernel_Name"]))
                  for r in csv.DictReader(open(trace[0])))
    # a plain step opens with the prologue kernel; it runs until the next
    # step of any kind (the fused and box steps open with the reference points)
    starts = [i for i, r in enumerate(rows) if r[2] == "prologue_kernel"]
    plain = []
    for si in starts:
        j = si + 1
        while j < len(rows) and rows[j][2] not in ("prologue_kernel", "reference_points_kernel"):
            j += 1
        plain.append(rows[si:j])
    w0 = max(1, warmup) + 1
    nrep = 3 + warmup + steps
    want = w0 + nrep + 2 * steps
    if len(plain) < want:
        raise SystemExit(f"{len(plain)} plain steps in the trace, expected at least {want} for "
                         f"--steps {steps} --warmup {warmup}")
    # the replays after the three that are checked against eager (those are
    # followed by torch's comparison kernels); library kernels only
    graph = [[r for r in seg if r[2].startswith(LIB_KERNELS)] for seg in plain[w0 + 3:w0 + nrep]]
    timed = [[r for r in seg if r[2].startswith(LIB_KERNELS)] for seg in plain[w0 + nrep + steps:w0 + nrep + 2 * steps]]

    def per_kernel(group):
        k = {}
        for seg in group:
            for s0, e0, n in seg:
                k.setdefault(n, []).append((e0 - s0) / 1e3)
        return {n: st.median(v) for n, v in k.items()}

    kg, kt = per_kernel(graph), per_kernel(timed)
    # the kernel sources the profiled run used (its bench line names them)
    src_hash = kernel_source_hash()
    blog = os.path.join(d, "bench.log")
    bline = None
    if os.path.exists(blog):
        bl = [ln for ln in open(blog) if ln.startswith('{"metric"')]
        if bl:
            bline = json.loads(bl[-1])
            src_hash = bline.get("source_hash", src_hash)
    spans = sorted(((max(r[1] for r in seg) - seg[0][0]) / 1e3, i) for i, seg in enumerate(graph))
    med = graph[spans[len(spans) // 2][1]]
    flags = "" if (steps, warmup) == (50, 10) else f" --steps {steps} --warmup {warmup}"  # the defaults, or not
    cmd = (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/"
           f"trace -o run -- python3 <repo>/bench.py{flags} > <out>/trace/bench.log")
    lines = ["# Kernel trace — encoder_backward step (B=2, M=8, D=32, L=4 76x106..8x13, S=Nq=10687, K=4, fp32)", "",
             "Generated by `python bench.py --trace-summary DIR --steps {0} --warmup {1}` from the csv output of".format(
                 steps, warmup), "", "```", cmd, "```", "",
             f"Kernel sources hash `{src_hash}`. The library's kernels only (torch's own kernels omitted). "
             "`all launches` is rocprofv3's average over every launch of the run (plain, fused and box steps, "
             "graph replays and eager loops, the cold loop); the medians are per launch over the "
             f"{len(graph)} graph replays of the plain step (warm-up and timed) and over the {len(timed)} eager plain steps whose "
             "kernels the library times with HIP event pairs (the `kernels` figures of the bench line).", "",
             "| kernel | launches | avg µs, all launches | median µs, graph replays | median µs, event-timed eager steps |",
             "|---|---:|---:|---:|---:|"]
    for n, (c, t) in sorted(all_avg.items(), key=lambda kv: -kv[1][1]):
        g_ = f"{kg[n]:.1f}" if n in kg else ""
        t_ = f"{kt[n]:.1f}" if n in kt else ""
        lines.append(f"| `{n}` | {c} | {t / c / 1e3:.1f} | {g_} | {t_} |")
    if bline is not None:
        if True:
            b = bline
            lines += ["", f"The bench line this profiled run printed: {b['ms_per_step'] * 1e3:.1f} µs per graph-replayed "
                      f"step; per kernel (library event pairs, eager): " +
                      ", ".join(f"{k} {v['avg_us']:.1f}" for k, v in b["kernels"].items()) + " µs; roofline kernel "
                      f"`{b['roofline']['kernel']}` at {b['roofline']['avg_us']:.1f} µs."]
    lines += ["", f"Graph-replay step spans (first kernel start to last kernel end): median "
              f"{spans[len(spans) // 2][0]:.1f} µs, min {spans[0][0]:.1f} µs, max {spans[-1][0]:.1f} µs. "
              "The timeline of the median replay (µs from its first kernel's start; kernels on two HW queues "
              "overlap):", "", "| start | end | µs | kernel |", "|---:|---:|---:|---|"]
    t0 = med[0][0]
    for s0, e0, n in med:
        lines.append(f"| {(s0 - t0) / 1e3:.1f} | {(e0 - t0) / 1e3:.1f} | {(e0 - s0) / 1e3:.1f} | `{n}` |")
    with open(TRACE_MD, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


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


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_threads():
    """Host threads for the oracle baseline: the cores this process may run
    on, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl_name, min_seconds=10.0):
    """The fp64 oracle, as it stands, on the same step (reference points,
    locations, softmax, forward and backward of the whole workload): whole
    passes until min_seconds of wall time, once on all the host threads
    (the forward split over queries, the backward over (image, head) pairs,
    results bit-identical to one thread) and once on one thread."""
    import oracle
    from scale_deformable_attention_msdeformattn_amd import workloads
    d = workloads.draw(wl_name, 0)
    w = d.workload
    shapes = d.spatial_shapes.numpy()
    # host-side input upcasts are not timed
    vr, off, logits, G, value = (oracle._f64(x) for x in (d.valid_ratios, d.offsets_px, d.logits,
                                                          d.grad_output, d.value))

    def run(threads):
        passes = 0
        with oracle.threads(threads):
            t0 = time.perf_counter()
            while True:
                lsi, _ = oracle.level_start_index(shapes)
                ref = oracle.reference_points_encoder(shapes, vr)
                loc = oracle.sampling_locations(shapes, ref, off)
                A = oracle.softmax(logits, w.levels * w.points).reshape(w.batch, w.nq, w.heads, w.levels,
                                                                        w.points)
                oracle.forward(value, shapes, lsi, loc, A)
                oracle.backward(value, shapes, lsi, loc, A, G)
                passes += 1
                dt = time.perf_counter() - t0
                if dt >= min_seconds:
                    return passes, dt

    q = w.batch * w.nq
    n = host_threads()
    p_all, t_all = run(n)
    p_one, t_one = run(1)
    return {"value": p_all * q / t_all, "unit": "queries/s", "cores": n, "kind": "oracle",
            "sample": f"{p_all} whole passes of the {w.name} workload ({q} queries each: reference points, "
                      f"locations, softmax, forward, backward), fp64 C on {n} threads, {t_all:.2f} s",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_core": {"value": p_one * q / t_one, "unit": "queries/s", "cores": 1,
                            "sample": f"{p_one} whole passes on one thread, {t_one:.2f} s"}}


def copy_ceiling(dev, nbytes=FLUSH_BYTES, reps=10):
    """A plain device copy of nbytes (torch's copy kernel) timed with events:
    (read + write bytes) / time, the rate a streaming kernel reaches here."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"gbps": round(2 * nbytes / s / 1e9, 1), "bytes_copied": nbytes, "kernel": "torch copy_ (fp32)",
            "frac_of_8tbps": round(2 * nbytes / s / 1e9 / HBM_PEAK_GBPS, 4)}


def cold_timing(msda, calls, dev, iters):
    """Every entry point of the step timed with L2 and the 256 MB Infinity
    Cache evicted before it: a 1 GiB read (a reduction over a buffer that no
    call touches) runs between the calls, outside the timed pairs. Two rounds:
    per call with HIP events around it (the library's timing off, so the
    backward runs as in the step), then per kernel with the library's event
    pairs. Returns both, averaged."""
    import torch
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    per_call = {name: 0.0 for name, _ in calls}
    torch.cuda.synchronize()
    for _ in range(iters):
        for name, f in calls:
            torch.sum(flush, dim=0, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            f()
            e1.record(stream)
            e1.synchronize()
            per_call[name] += e0.elapsed_time(e1) * 1e3 / iters
    msda.msda_timing_reset()
    for _ in range(iters):
        for name, f in calls:
            torch.sum(flush, dim=0, out=sink)
            msda.msda_timing_enable(True)
            f()
            msda.msda_timing_enable(False)
            torch.cuda.synchronize()
    timing = msda.msda_timing_read()
    msda.msda_timing_reset()
    del flush
    torch.cuda.empty_cache()
    return {k: ms * 1e3 / n for k, (ms, n) in timing.items()}, per_call


def forward_configs(msda, workloads, dev, args, names=("decoder", "encoder_bf16_large")):
    """The forward alone on the other forward workloads of the pages' shapes
    (the decoder's 300 object queries; the large batch with bf16 value): the
    time per call of a HIP graph of 20 back-to-back calls (the library's
    event pairs name the kernel, and their own figure, which overstates a
    kernel of a few microseconds, is kept as event_us), queries/s and
    effective HBM GB/s over the algorithmic bytes (the distinct value rows
    touched, loc, A and the output)."""
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
        event_us = ms * 1e3 / cnt
        s2 = torch.cuda.Stream(dev)
        s2.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(s2):
            msda.msda_forward(value, shapes, lsi, loc, A)
        torch.cuda.current_stream(dev).wait_stream(s2)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(n):
                msda.msda_forward(value, shapes, lsi, loc, A)
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        g0.record()
        for _ in range(reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        us = g0.elapsed_time(g1) * 1e3 / (reps * n)
        del graph
        gbps = alg / (us * 1e-6) / 1e9
        out[name] = {"workload": w.description, "kernel": kernel, "avg_us": round(us, 3),
                     "event_us": round(event_us, 3), "timing": f"graph of {n} calls, replayed {reps} times",
                     "queries_per_s": B * Nq / (us * 1e-6), "algorithmic_bytes": alg,
                     "effective_gbps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        del value, loc, A, ref
        torch.cuda.empty_cache()
    return out


def generic_path(msda, workloads, dev, shapes):
    """The paths for shapes without compiled kernels, timed on the encoder
    maps with 8 heads of 16 channels (C = 128): the generic 4-channel
    forward (a graph of 20 calls) and the generic backward (grad_value by
    float atomics; HIP events around 10 calls). Effective GB/s over the same kind
    of algorithmic bytes as the fast path's."""
    import torch
    wl = workloads.custom(name="generic_c128", batch=2, heads=8, channels=16, points=4,
                          spatial_shapes=[tuple(int(v) for v in hw) for hw in shapes.tolist()], num_query=None,
                          offset_sigma_px=2.0, random_valid_ratios=True, backward=True)
    d = workloads.draw(wl, 0)
    w = d.workload
    B, M, D, L, K, Nq = w.batch, w.heads, w.channels, w.levels, w.points, w.nq
    lsi, _ = msda.level_start_index_host(d.spatial_shapes)
    vr = d.valid_ratios.to(dev)
    ref = msda.msda_reference_points(d.spatial_shapes, valid_ratios=vr)
    loc = msda.msda_sampling_locations(d.spatial_shapes, ref, d.offsets_px.to(dev))
    A = msda.msda_attention_softmax(d.spatial_shapes, d.logits.to(dev), K)
    value = d.value.to(dev)
    G = d.grad_output.to(dev)
    vbytes, _ = unique_value_bytes(loc, d.spatial_shapes.to(dev), B, M, D * 4)
    samples = B * Nq * M * L * K
    fwd_alg = vbytes + samples * 3 * 4 + B * Nq * M * D * 4
    bwd_alg = 2 * vbytes + samples * 6 * 4 + B * Nq * M * D * 4
    f = lambda: msda.msda_forward(value, d.spatial_shapes, lsi, loc, A)
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    f()
    torch.cuda.synchronize()
    msda.msda_timing_enable(False)
    fwd_kernel = max(msda.msda_timing_read().items(), key=lambda kv: kv[1][0])[0]
    msda.msda_timing_reset()
    s2 = torch.cuda.Stream(dev)
    s2.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s2):
        f()
    torch.cuda.current_stream(dev).wait_stream(s2)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    n = 20
    with torch.cuda.graph(graph):
        for _ in range(n):
            f()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    fwd_us = e0.elapsed_time(e1) * 1e3 / (5 * n)
    del graph
    bwd = lambda: msda.msda_backward(value, d.spatial_shapes, lsi, loc, A, G)
    for _ in range(2):
        bwd()
    torch.cuda.synchronize()
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    bwd()
    torch.cuda.synchronize()
    msda.msda_timing_enable(False)
    bwd_kernel = max(msda.msda_timing_read().items(), key=lambda kv: kv[1][0])[0]
    msda.msda_timing_reset()
    e0.record()
    for _ in range(10):
        bwd()
    e1.record()
    torch.cuda.synchronize()
    bwd_us = e0.elapsed_time(e1) * 1e3 / 10
    out = {"workload": f"encoder maps, B={B} M={M} D={D} (C={M * D}) L={L} K={K} S=Nq={Nq} fp32",
           "forward": {"kernel": fwd_kernel, "avg_us": round(fwd_us, 2),
                       "effective_gbps": round(fwd_alg / (fwd_us * 1e-6) / 1e9, 1)},
           "backward": {"kernel": bwd_kernel + " (grad_value by float atomics)", "call_us": round(bwd_us, 2),
                        "effective_gbps": round(bwd_alg / (bwd_us * 1e-6) / 1e9, 1)}}
    del value, loc, A, ref, G
    torch.cuda.empty_cache()
    return out


def decoder_backward(msda, workloads, dev):
    """The backward of the decoder's 300 object queries per image (the tiled
    per-query path: binning, the per-query main kernel, tile_accum and the
    dense levels): HIP events around 20 back-to-back calls, and the kernels
    each timed alone by the library's event pairs."""
    import torch
    base = workloads.WORKLOADS["decoder"]
    wl = workloads.custom(name="decoder_backward", batch=base.batch, heads=base.heads, channels=base.channels,
                          points=base.points, spatial_shapes=base.spatial_shapes, num_query=base.num_query,
                          offset_sigma_px=base.offset_sigma_px, random_valid_ratios=True, backward=True)
    d = workloads.draw(wl, 0)
    shapes = d.spatial_shapes
    lsi, _ = msda.level_start_index_host(shapes)
    ref = msda.msda_reference_points(shapes, valid_ratios=d.valid_ratios.to(dev), query_ref=d.query_ref.to(dev))
    loc = msda.msda_sampling_locations(shapes, ref, d.offsets_px.to(dev))
    A = msda.msda_attention_softmax(shapes, d.logits.to(dev), wl.points)
    value, G = d.value.to(dev), d.grad_output.to(dev)
    f = lambda: msda.msda_backward(value, shapes, lsi, loc, A, G)
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        f()
    e1.record()
    torch.cuda.synchronize()
    call_us = e0.elapsed_time(e1) * 1e3 / 20
    msda.msda_timing_reset()
    msda.msda_timing_enable(True)
    for _ in range(5):
        f()
    torch.cuda.synchronize()
    msda.msda_timing_enable(False)
    kernels = {k: round(v[0] * 1e3 / v[1], 2) for k, v in msda.msda_timing_read().items()}
    msda.msda_timing_reset()
    queries = wl.batch * wl.nq
    return {"workload": f"decoder backward fp32: B={wl.batch} M={wl.heads} D={wl.channels} L={wl.levels} "
                        f"Nq={wl.nq} K={wl.points}", "call_us": round(call_us, 2),
            "queries_per_s": queries / (call_us * 1e-6), "kernels_alone_us": kernels}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the figure is one GPU's "
              "share (the op shards by batch or by head with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.ingest_counters:
        ingest_counters(args.ingest_counters, args.workload)
        return
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.steps, args.warmup)
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

    def k_prologue():  # reference points, sampling locations and softmax, one launch
        state["ref"], state["loc"], state["A"] = msda.msda_prologue(shapes, off, logits, valid_ratios=vr)

    def k_fwd():
        state["out"] = msda.msda_forward(value, shapes, lsi, state["loc"], state["A"])

    def k_bwd():
        state["grads"] = msda.msda_backward(value, shapes, lsi, state["loc"], state["A"], G)

    calls = [("msda_prologue", k_prologue), ("msda_forward", k_fwd), ("msda_backward", k_bwd)]

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
    if args.profile_run:  # counter passes: the plain step's kernels only, eager
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": w.name, "steps": args.steps, "source_hash": kernel_source_hash()}),
              flush=True)
        return

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

    # ---- timed region 4: every entry point again with the caches evicted
    # before each call (cold), and a plain copy's rate ----
    cold = None
    if args.cold_iters > 0:
        cold_kernels, cold_calls = cold_timing(msda, calls, dev, args.cold_iters)
        cold = {"protocol": f"{args.cold_iters} calls per entry point; before each, a 1 GiB read (4x the 256 MB "
                            "Infinity Cache) outside the timed pairs, so every input starts in HBM; one round "
                            "timed per call (as in the step), one per kernel (library event pairs, the backward's "
                            "kernels in turn on one stream)",
                "entry_points_us": {k: round(v, 3) for k, v in cold_calls.items()},
                "step_us_sum": round(sum(cold_calls.values()), 3),
                "kernels": {k: {"avg_us": round(us, 3), **({} if k not in alg else {
                    "gbps": round(alg[k] / (us * 1e-6) / 1e9, 1),
                    "frac_of_hbm_peak": round(alg[k] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})}
                            for k, us in cold_kernels.items()}}
    copy = copy_ceiling(dev)

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
    # the backward's main kernel on this shape (per head with staged levels, or per query)
    bwd_main = next((k for k in ("backward_head_kernel", "backward_c256_kernel") if k in kstats), None)
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
        "config": {"workload": w.description, "step": "reference points + locations + softmax (one launch) + forward + "
                   "backward", "graph_replay": graph is not None},
        "source_hash": kernel_source_hash(),
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dominant), "avg_us": dom_us,
                     "algorithmic_bytes": alg[dominant],
                     "timing": "warm: library event pairs around each launch over back-to-back eager steps",
                     "cold_frac": None if cold is None or dominant not in cold["kernels"]
                     else cold["kernels"][dominant].get("frac_of_hbm_peak"),
                     "frac_of_copy_ceiling": round(dom_gbps / copy["gbps"], 4)},
        "kernels": kstats,
        "entry_points_us": {k: round(v, 3) for k, v in per_call.items()},
        "cold": cold,
        "copy_ceiling": copy,
        "eager_ms_per_step": eager_step_ms,
        "forward": {"kernel": fwd_name, "queries_per_s": queries / (fwd["avg_us"] * 1e-6) if fwd else None,
                    "effective_gbps": fwd.get("gbps"), "frac_of_hbm_peak": fwd.get("frac_of_hbm_peak"),
                    "cold": None if cold is None or fwd_name not in cold["kernels"] else {
                        "avg_us": cold["kernels"][fwd_name]["avg_us"],
                        "queries_per_s": queries / (cold["kernels"][fwd_name]["avg_us"] * 1e-6),
                        "effective_gbps": cold["kernels"][fwd_name].get("gbps"),
                        "frac_of_hbm_peak": cold["kernels"][fwd_name].get("frac_of_hbm_peak")},
                    "traffic": measured_traffic(fwd_name) if fwd_name else None,
                    "gather": None if not fwd else {
                        "corner_reads": corner_reads, "bytes": corner_reads * D * elem,
                        "tbps": round(corner_reads * D * elem / (fwd["avg_us"] * 1e-6) / 1e12, 2),
                        "note": "in-map corner reads of one head's value row each; the fine levels' are served by "
                                "L1/L2 (we measured 50-58 B/clk/CU for 16-byte lane gathers on that path, 31-36 TB/s "
                                "on 256 CUs at 2.4 GHz), the coarse levels' from LDS when they are staged"}},
        "backward": {"queries_per_s": queries / (per_call["msda_backward"] * 1e-6),
                     "cold_queries_per_s": None if cold is None else
                     queries / (cold["entry_points_us"]["msda_backward"] * 1e-6),
                     "note": "the whole msda_backward call, all its kernels",
                     "main_kernel_gather": None if bwd_main is None else {
                         "kernel": bwd_main, "corner_reads": corner_reads, "bytes": corner_reads * D * elem,
                         "tbps": round(corner_reads * D * elem / (kstats[bwd_main]["avg_us"] * 1e-6)
                                       / 1e12, 2),
                         "note": "the main backward kernel gathers the same in-map corner rows as the forward "
                                 "(the per-head kernel serves the coarse levels' from LDS, the per-query kernel all "
                                 "through the L1/L2 path, 31-36 TB/s measured ceiling on 256 CUs)"}},
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
        result["generic_path"] = generic_path(msda, workloads, dev, shapes)
        result["decoder_backward"] = decoder_backward(msda, workloads, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
