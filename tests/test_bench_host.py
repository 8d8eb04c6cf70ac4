"""Host logic of bench.py that needs no GPU: the single-GPU guard, the kernel
names it groups counters by, the exact L2 byte arithmetic of the counter
ingestion, the kernel-source hash that keeps counter figures attached to the
code they were measured on, its mirror of the library's dense-level rule
(checked against the library's own planner through the C ABI), and the trace
summary's segmentation of a kernel trace into plain steps."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from scale_deformable_attention_msdeformattn_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no bench line


@pytest.mark.parametrize("full,short", [
    ("void msda::(anonymous namespace)::tile_accum_kernel<8, 4, 4>(msda::Geometry, msda::TilePlan)", "tile_accum_kernel"),
    ("void msda::(anonymous namespace)::forward_staged_kernel<float, 8, 4, 4, 2, false>(msda::Geometry)",
     "forward_staged_kernel"),
    ("void msda::(anonymous namespace)::forward_staged_kernel<float, 8, 4, 4, 2, true>(msda::Geometry)",
     "forward_fused_staged_kernel"),
    ("void msda::(anonymous namespace)::backward_head_kernel<float, 8, 4, 4, 2, true>(msda::Geometry)",
     "backward_fused_head_kernel"),
    ("void msda::(anonymous namespace)::backward_c256_kernel<unsigned short, 8, 4, 4, true>(msda::Geometry)",
     "backward_fused_c256_kernel"),
    ("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>(int, float)",
     "vectorized_elementwise_kernel"),
])
def test_short_kernel_names(full, short):
    assert bench._short_kernel_name(full) == short


def _write_pass(d, name, rows, source_hash):
    os.makedirs(os.path.join(d, name))
    with open(os.path.join(d, name, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, counter, values in rows:
            for v in values:  # one row per dispatch
                w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": v})
    with open(os.path.join(d, name, "bench.log"), "w") as f:
        f.write(json.dumps({"profile_run": "encoder_backward", "steps": 3, "source_hash": source_hash}) + "\n")


def test_counter_ingestion_bytes(tmp_path, monkeypatch):
    kern = "void msda::(anonymous namespace)::tile_accum_kernel<8, 4, 4>(msda::Geometry)"
    # two dispatches per counter; the ingestion averages them
    counters = {
        "tcc_read": {"TCC_EA0_RDREQ_sum": [1000, 1200], "TCC_EA0_RDREQ_32B_sum": [100, 100],
                     "TCC_EA0_RDREQ_64B_sum": [200, 200], "TCC_EA0_RDREQ_128B_sum": [690, 890]},
        "tcc_write_hit": {"TCC_HIT_sum": [300, 300], "TCC_MISS_sum": [100, 100], "TCC_EA0_WRREQ_sum": [50, 50],
                          "TCC_EA0_WRREQ_64B_sum": [40, 40]},
        "sq_time": {"SQ_WAVES": [64, 64], "SQ_WAVE_CYCLES": [1000, 1000], "SQ_WAIT_INST_ANY": [250, 250],
                    "SQ_WAIT_ANY": [500, 500]},
        "sq_insts": {"SQ_INSTS_VALU": [2048, 2048]},
        "units": {"TA_TA_BUSY_sum": [256 * 100, 256 * 100], "GRBM_GUI_ACTIVE": [8 * 400, 8 * 400]},
    }
    d = str(tmp_path / "pmc")
    for name in bench.COUNTER_PASSES:
        rows = [(kern, c, v) for c, v in counters.get(name, {}).items()]
        _write_pass(d, name, rows, "feedfacecafebeef")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(bench, "COUNTERS_MD", str(tmp_path / "counters.md"))
    bench.ingest_counters(d, "encoder_backward")
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["source_hash"] == "feedfacecafebeef"
    e = t["kernels"]["tile_accum_kernel"]
    rd = 32 * 100 + 64 * 200 + 128 * 790            # exact bytes by request size, averaged
    wr = 64 * 40 + 32 * (50 - 40)                    # 64-B writes, the rest 32 B
    assert e["dispatches"] == 2
    assert e["read_bytes"] == rd and e["write_bytes"] == wr and e["hbm_bytes_per_launch"] == rd + wr
    assert e["read_requests_other_sizes"] == 1100 - 100 - 200 - 790
    assert e["l2_hit_rate"] == pytest.approx(0.75)
    assert e["wait_inst_share"] == pytest.approx(0.25) and e["wait_any_share"] == pytest.approx(0.5)
    # busy cycles per XCD = GRBM / 8 = 400; VALU: 2048 wave instructions * 4 cycles / 1024 SIMDs
    assert e["valu_share_of_busy"] == pytest.approx(2048 * 4 / 1024 / 400, abs=1e-3)
    assert e["ta_busy_share"] == pytest.approx(100 / 400, abs=1e-3)
    assert e["hbm_over_algorithmic"] == pytest.approx((rd + wr) / e["algorithmic_bytes"], abs=1e-3)
    assert "tile_accum_kernel" in open(tmp_path / "counters.md").read()


def test_counter_ingestion_needs_one_source_hash(tmp_path, monkeypatch):
    d = str(tmp_path / "pmc")
    for i, name in enumerate(bench.COUNTER_PASSES):
        _write_pass(d, name, [], "aaaa" if i else "bbbb")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(bench, "COUNTERS_MD", str(tmp_path / "counters.md"))
    with pytest.raises(SystemExit):
        bench.ingest_counters(d, "encoder_backward")
    assert not (tmp_path / "traffic.json").exists()


def test_kernel_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    csrc = tmp_path / "scale_deformable_attention_msdeformattn_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("int f(int x) { return x + 1; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / "k.hip").write_text("// a comment\nint f(int x)  {\n  return x + 1; /* why */ }\n")
    assert bench.kernel_source_hash() == h0
    (csrc / "k.hip").write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != h0


@pytest.mark.parametrize("shapes,nq,k", [
    (((76, 106), (38, 53), (19, 27), (8, 13)), 10687, 4),
    (((4, 4), (40, 40), (6, 6)), 3000, 4),
    (((64, 64), (24, 24), (16, 16), (8, 8)), 12000, 4),
    (((100, 167), (50, 84), (25, 42), (13, 21)), 22223, 4),
    (((12, 10), (6, 5), (3, 3), (2, 2), (1, 1)), 164, 4),
    (((46, 46),), 50000, 4),
])
def test_dense_levels_mirror_the_library(shapes, nq, k):
    sh = B.Shape(shapes, 2, 8, 32, k, nq)
    assert bench.dense_levels(shapes, nq, k) == B.msda_backward_plan(sh)["dense"]


def _k(name):
    return f"void msda::(anonymous namespace)::{name}<8, 4, 4>(msda::Geometry)"


# a plain step as the trace shows it: (kernel, start offset, duration) in ns
PLAIN = [("prologue_kernel", 0, 16000), ("forward_staged_kernel", 16000, 38000),
         ("dense_accum_kernel", 60000, 40000), ("bin_count_head_kernel", 66000, 28000),
         ("backward_head_kernel", 94000, 64000), ("dense_reduce_kernel", 101000, 23000),
         ("tile_accum_kernel", 158000, 44000)]
FUSED = [("reference_points_kernel", 0, 5000), ("forward_staged_kernel<float, 8, 4, 4, 2, true>", 5000, 50000)]


def test_trace_summary_segments_plain_steps(tmp_path, monkeypatch):
    """The trace summary finds the plain steps by their opening prologue
    kernel, ends each at the next step of any kind (a fused step opens with
    the reference points), drops torch's kernels, and takes the replays and
    the event-timed eager steps from their places in the run's order."""
    steps, warmup = 4, 2
    w0 = max(1, warmup) + 1
    nrep = 3 + warmup + steps
    n_plain = w0 + nrep + 2 * steps
    rows, t = [], 0
    for i in range(n_plain):
        scale = 1.0 + 0.01 * i  # later steps a little slower: the medians pick the middle
        for name, s0, dur in PLAIN:
            rows.append((_k(name), t + int(s0 * scale), t + int((s0 + dur) * scale)))
        # a torch kernel inside the segment (the replays' comparison kernels)
        rows.append(("void at::native::vectorized_elementwise_kernel<4>(int)", t + 210000, t + 211000))
        t += 300000
    for _ in range(3):  # fused steps after the plain ones
        for name, s0, dur in FUSED:
            full = f"void msda::(anonymous namespace)::{name}(msda::Geometry)" if "<" in name else _k(name)
            rows.append((full, t + s0, t + s0 + dur))
        t += 300000
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        for k, s0, e0 in rows:
            wr.writerow({"Kernel_Name": k, "Start_Timestamp": s0, "End_Timestamp": e0})
    counts = {}
    for k, s0, e0 in rows:
        c, tot = counts.get(k, (0, 0))
        counts[k] = (c + 1, tot + e0 - s0)
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs"])
        wr.writeheader()
        for k, (c, tot) in counts.items():
            wr.writerow({"Name": k, "Calls": c, "TotalDurationNs": tot})
    out = tmp_path / "trace.md"
    monkeypatch.setattr(bench, "TRACE_MD", str(out))
    bench.trace_summary(str(d), steps, warmup)
    md = out.read_text()
    # replays w0+3 .. w0+nrep-1 and eager steps w0+nrep+steps .. end
    assert f"over the {nrep - 3} graph replays" in md and f"over the {steps} eager plain steps" in md
    timeline = md.split("| start | end | µs | kernel |")[1].strip().splitlines()[1:]
    assert [ln.split("`")[1] for ln in timeline] == [n for n, _, _ in PLAIN]
    # the median replay is the middle one of the replays taken
    mid = sorted(range(w0 + 3, w0 + nrep))[(nrep - 3) // 2]
    first = timeline[1].split("|")
    assert abs(float(first[1]) - 16.0 * (1.0 + 0.01 * mid)) < 0.05
    # the fused step's kernels are not in the plain steps' medians
    row = [ln for ln in md.splitlines() if ln.startswith("| `reference_points_kernel`")][0]
    assert row.split("|")[4].strip() == "" and row.split("|")[5].strip() == ""
    assert "vectorized_elementwise_kernel" not in md
