"""Host-side pieces of bench.py: the counter summary's scaling, the step
period of a kernel trace, and the rule that a stored traffic figure is
reported only for unchanged kernel sources."""

import csv
import json

import bench

COPY = "void tpk::shard_copy_kernel(tpk::ShardMap, uint4 const*, uint4*)"
GEMM = "void tpk::skinny_kernel<1, 8, 1, 4, 1>(tpk::GemmArgs, int, long, int, float*, unsigned int*)"
OTHER = "void tpk::reduce_kernel<false, false, 8>(tpk::PartialPtrs, int, long, void*)"


def _csv(path, counter, copy_kib, gemm_kib, steps, gemms_per_step):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i in range(3):
            w.writerow([i, 4096, COPY, counter, copy_kib])
        for s in range(steps):
            for j in range(gemms_per_step):
                w.writerow([10 + s * 9 + j, 49152, GEMM, counter, gemm_kib])
            w.writerow([99, 8192, OTHER, counter, 12345.0])


def test_summarize_counters_scales_by_the_copy(tmp_path):
    copy_bytes = 1 << 20
    # the copy reads as half its bytes on FETCH_SIZE and exactly on WRITE_SIZE
    _csv(tmp_path / "f.csv", "FETCH_SIZE", copy_bytes / 1024 / 2, 100.0, 3, 2)
    _csv(tmp_path / "w.csv", "WRITE_SIZE", copy_bytes / 1024, 10.0, 3, 2)
    run = {"workload": "x", "copy_bytes": copy_bytes, "copy_launches": 3, "steps": 3,
           "gemm_launches_per_step": 2, "gemm_algorithmic_bytes_per_step": 400 * 1024,
           "source_sha256": "s"}
    (tmp_path / "run.log").write_text("banner\n" + json.dumps(run) + "\n")
    d = bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "run.log"),
                                 str(tmp_path / "out.json"))
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    assert d["fetch_bytes_per_step"] == 2 * 2 * 100 * 1024
    assert d["write_bytes_per_step"] == 2 * 10 * 1024
    assert d["traffic_over_algorithmic"] == round((400 + 20) / 400, 4)
    assert json.load(open(tmp_path / "out.json"))["traffic_bytes_per_step"] == 420 * 1024


def test_code_digest_ignores_comments_and_layout_only():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* plain */ }"
    b = "int f(int x)\n{\n    return 2 * x;\n}"
    c = "int f(int x) { return 3 * x; }"
    assert bench.code_digest(a) == bench.code_digest(b)
    assert bench.code_digest(a) != bench.code_digest(c)


def test_stored_traffic_needs_unchanged_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_file", lambda w: str(tmp_path / f"{w}.json"))
    (tmp_path / "a.json").write_text(json.dumps({"source_sha256": bench.gemm_source_sha256(),
                                                 "traffic_bytes_per_step": 7}))
    (tmp_path / "b.json").write_text(json.dumps({"source_sha256": "0" * 64, "traffic_bytes_per_step": 7}))
    assert bench.stored_traffic("a")["traffic_bytes_per_step"] == 7
    assert bench.stored_traffic("b") is None
    assert bench.stored_traffic("missing") is None


def test_step_trace_period_with_identical_layers_and_two_launch_calls(tmp_path):
    """A step of 4 identical layers whose GEMM call launches two kernels:
    the layer's period (3 dispatches) repeats too, so the step's 12
    dispatches are found from the step time the run measured."""
    layer = [("skinny_kernel<1>", 10), ("skinny_split_finish<0>", 5), ("reduce_kernel<0>", 3)]
    K, layers, gap = 3, 4, 2
    rows, t = [], 0
    for name, dur in [("setup_kernel", 7)] * 2:
        rows.append((t, t + dur, name)); t += dur + gap
    for _ in range(K + 2):                       # warm-up passes, then the K timed steps
        for _ in range(layers):
            for name, dur in layer:
                rows.append((t, t + dur, name)); t += dur + gap
    step_ns = layers * sum(d + gap for _, d in layer)
    with open(tmp_path / "trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"])
        for a, b, name in rows:
            w.writerow([f"void tpk::{name}(args)", a, b, 256, 256])
    run = {"workload": "x", "ms_per_step": step_ns / 1e6, "steps": K, "steps_in_trace": K + 2,
           "gemm_launches_per_step": layers, "launches_per_step": 2 * layers,
           "gemm_algorithmic_bytes_per_step": 1000, "gemm_flops_per_step": 2000}
    (tmp_path / "run.log").write_text(json.dumps(run) + "\n")
    bench.summarize_step_trace(str(tmp_path / "trace.csv"), str(tmp_path / "run.log"), str(tmp_path / "out.txt"))
    text = (tmp_path / "out.txt").read_text()
    assert f"{layers * len(layer)} dispatches per step" in text
    assert f"GEMM dispatches per step: {2 * layers}" in text
