"""Host logic of bench.py, on the CPU: the one-GPU guard, the counter
calibration behind `roofline.traffic`, the staleness check of committed
counter summaries, the run-variant names of the summaries, and the rocprofv3
kernel-statistics summary."""
import csv
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _counters(d, counter, rows):
    _write_csv(os.path.join(d, "pass", "x_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [(k, counter, v) for k, v in rows])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""                    # no JSON line


def test_traffic_is_scaled_by_the_copy_probe(tmp_path):
    """A copy of 1 GiB whose FETCH_SIZE reads half the copied KiB gives a fetch
    scale of 2; WRITE_SIZE reading the full size gives 1. Kernel dispatches
    are averaged; other kernels in the same pass are ignored."""
    kern = "void gnn::k_fwd_main<float, 4, 1, 4>(gnn::FwdParams)"
    other = "void gnn::k_fwd_merge<float, 4>(gnn::FwdParams)"
    copy = "__amd_rocclr_copyBuffer"
    _counters(tmp_path / "f", "FETCH_SIZE", [(kern, 1000.0), (kern, 3000.0), (other, 99.0)])
    _counters(tmp_path / "w", "WRITE_SIZE", [(kern, 500.0), (kern, 500.0)])
    _counters(tmp_path / "cf", "FETCH_SIZE", [(copy, 524288.0)])
    _counters(tmp_path / "cw", "WRITE_SIZE", [(copy, 1048576.0)])
    out = tmp_path / "s.txt"
    args = types.SimpleNamespace(traffic=[str(tmp_path / x) for x in ("f", "w", "cf", "cw")], kernel="gatv2_fwd_main",
                                 kernel_regex="k_fwd_main", copy_mib=1024, workload="w", bench_args="", out=str(out))
    assert bench.traffic_summary(args) == 0
    vals = dict(line.split(":", 1) for line in out.read_text().splitlines() if ":" in line and line[0] != "#")
    assert float(vals["fetch_bytes_per_launch"]) == 2000.0 * 1024 * 2
    assert float(vals["write_bytes_per_launch"]) == 500.0 * 1024
    assert float(vals["traffic_bytes_per_launch"]) == 2000.0 * 1024 * 2 + 500.0 * 1024
    assert vals["kernel_symbol"].strip() == kern


def test_missing_kernel_in_a_counter_pass_is_an_error(tmp_path):
    _counters(tmp_path / "f", "FETCH_SIZE", [("void other()", 1.0)])
    with pytest.raises(SystemExit):
        bench._counter_means(str(tmp_path / "f"), "FETCH_SIZE", "k_fwd_main")


def test_committed_traffic_is_ignored_once_sources_change(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    tag = bench.profile_tag("wl", False, False, "none")
    path = tmp_path / f"gt_fwd_main__{tag}__counters.txt"
    good = bench.kernel_source_hash("gt_fwd_main")
    path.write_text(f"# header: with a colon\nsource_sha256: {good}\ntraffic_bytes_per_launch: 1234\n")
    assert bench.read_traffic("gt_fwd_main", tag) == 1234.0
    path.write_text("source_sha256: 0000000000000000\ntraffic_bytes_per_launch: 1234\n")
    assert bench.read_traffic("gt_fwd_main", tag) is None
    assert bench.read_traffic("gt_fwd_main", "no_such_run") is None


def test_source_hash_follows_the_kernel_family():
    attn = bench.kernel_source_hash("gt_fwd_main")
    assert bench.kernel_source_hash("gatv2_bwd_src_main") == attn
    assert bench.kernel_source_hash("reduce_fwd_main") != attn
    assert bench.kernel_source_hash("spmm_t_main") == bench.kernel_source_hash("spmm_main") != attn


def test_profile_tag_names_each_variant():
    assert bench.profile_tag("gt_comm16_n1m_deg27", False, False, "none") == "gt_comm16_n1m_deg27"
    assert bench.profile_tag("gt_comm16_n1m_deg27", True, False, "none") == "gt_comm16_n1m_deg27__tiles"
    assert bench.profile_tag("gatv2_zipf21_n100k", False, True, "none") == "gatv2_zipf21_n100k__bwd"
    assert bench.profile_tag("gatv2_zipf21_n100k", False, False, "degree") == "gatv2_zipf21_n100k__degree"
    assert bench.profile_tag("a", True, True, "rcm") == "a__tiles__bwd__rcm"


def test_every_committed_counter_summary_names_a_known_variant():
    """Each committed counter summary belongs to a workload and variant the
    bench can produce, so the bench finds it by the same name."""
    import inspect

    import workloads
    modelled = inspect.getsource(bench.kernel_bytes)
    tags = {bench.profile_tag(w, t, b, r) for w in workloads.SPECS for t in (False, True) for b in (False, True)
            for r in ("none", "degree", "rcm")}
    for fn in os.listdir(os.path.join(ROOT, "profiles")):
        if fn.endswith("__counters.txt"):
            kernel, tag = fn[: -len("__counters.txt")].split("__", 1)
            assert tag in tags, fn
            assert f'"{kernel}"' in modelled, fn          # a kernel the byte model knows


def test_kernel_stats_summary_sorts_by_total_time(tmp_path):
    hdr = ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs", "Percentage"]
    _write_csv(str(tmp_path / "t" / "x_kernel_stats.csv"), hdr,
               [("small", 2, 2000, 1000, 900, 1100, 10.0), ("big", 3, 18000, 6000, 5000, 7000, 90.0)])
    out = tmp_path / "sum.txt"
    args = types.SimpleNamespace(summarize=str(tmp_path / "t"), command="cmd", kernel="gt_fwd_main", out=str(out))
    assert bench.summarize(args) == 0
    rows = [line.split() for line in out.read_text().splitlines() if line.strip().endswith(("big", "small"))]
    assert [r[-1] for r in rows] == ["big", "small"]
    assert float(rows[0][1]) == 6.0 and float(rows[1][1]) == 1.0      # average in microseconds


def test_source_hash_ignores_comments():
    code = "int f(int x) {\n    return x + 1;   // add one\n}\n"
    commented = "/* a block\n   comment */\n// header\nint f(int x) {\n    return x + 1;   // plus one\n\n}\n"
    changed = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench._code_only(code) == bench._code_only(commented)
    assert bench._code_only(code) != bench._code_only(changed)


def test_gather_ceiling_follows_the_quoted_probe_lines():
    """The ceiling table is the probe note's gather lines, and the lookup
    interpolates between them in log(table size), held at the ends."""
    import re
    quoted = {}
    with open(os.path.join(ROOT, "profiles", "bw_probe__read_copy_gather.txt")) as f:
        for line in f:
            m = re.match(r"gather (\d+)-byte rows from a (\d+) MiB table.*: ([\d.]+) GB/s", line)
            if m:
                quoted.setdefault(int(m.group(1)), []).append((int(m.group(2)), float(m.group(3))))
    assert quoted == bench.GATHER_CEILING_GBPS
    mib = 1 << 20
    assert bench.gather_ceiling(51 * mib, 512) == 8067.2             # below the smallest table: held
    assert bench.gather_ceiling(8192 * mib, 1024) == 6290.9          # above the largest: held
    assert bench.gather_ceiling(256 * mib, 300) == 7692.6            # nearest row size (256 B)
    mid = bench.gather_ceiling(512 * mib, 512)                       # halfway in log size between 256 and 1024 MiB
    assert mid == pytest.approx((7580.3 + 7153.9) / 2)


def test_roofline_context_labels_the_cache_state():
    # GATv2 forward, 100k nodes, H = 8, D = 16, fp32, V = XS: one 51 MB table -> Infinity Cache
    c = bench.roofline_context("gatv2_fwd_main", 8, 16, 4, 100_000, 7926.3, 2.527e9, 345.3)
    assert c["bound"] == "infinity-cache" and c["cache_resident"] and c["gathered_table_bytes"] == 51_200_000
    assert c["model_is_bound"] and c["traffic_frac_of_gather_ceiling"] == pytest.approx(
        2.527e9 / 345.3e-6 / 1e9 / 8067.2, rel=1e-3)
    assert "Infinity Cache" in c["note"]
    # GT forward, 2.45M nodes, H = 4, D = 32, bf16: K and V, 627 MB each -> HBM
    c = bench.roofline_context("gt_fwd_main", 4, 32, 2, 2_450_000, 7804.0, None, 4430.0)
    assert c["bound"] == "hbm" and not c["cache_resident"] and c["traffic_frac_of_gather_ceiling"] is None
    assert c["gathered_table_bytes"] == 2 * 256 * 2_450_000
    # a model rate above the HBM peak is flagged as no bound
    c = bench.roofline_context("gt_bwd_src_main", 8, 64, 2, 1_000_000, 10164.0, 30.34e9, 6020.0)
    assert not c["model_is_bound"] and "not a bound" in c["note"]


@pytest.mark.parametrize("name", ["gt_uniform_n2708", "gatv2_zipf21_n100k", "spmm_chunglu25_n169k",
                                  "maxpool_zipf21_n100k"])
def test_cpu_baseline_checks_the_measured_outputs(name):
    """The baseline leg compares the GPU's outputs on its sampled rows with
    the oracle: the oracle's own outputs pass, a planted error fails."""
    import numpy as np

    import oracle
    import workloads
    wl = workloads.make(name, 600, backward=name != "maxpool_zipf21_n100k")
    n = wl.n_nodes
    rp, rx = oracle.csr_build(wl.src, wl.dst, n)
    f = {k: np.asarray(v) for k, v in wl.feats.items()}
    if wl.kind == "spmm":
        F = wl.heads * wl.dim
        gpu = {"Y": oracle.spmm(rp, rx, f["X"].reshape(n, F))["Y"],
               "dX": oracle.spmm(rp, rx, f["dO"].reshape(n, F), transpose=True)["Y"]}
        key = "Y"
    elif wl.kind == "reduce":
        r = oracle.segment_reduce(rp, rx, f["X"].reshape(n, -1), "max", "src")
        gpu = {"out": np.asarray(r["out"], np.float32), "arg": r["arg"]}
        key = "out"
    elif wl.kind == "gatv2":
        r = oracle.gatv2_fwd(rp, rx, f["XD"], f["XS"], wl.att, slope=0.2)
        b = oracle.gatv2_bwd(rp, rx, f["XD"], f["XS"], wl.att, f["dO"], slope=0.2, want_da=False)
        gpu = {"O": r["O"], "LSE": r["LSE"], "dQ": b["dXD"], "dK": b["dXS"]}
        key = "O"
    else:
        r = oracle.gt_fwd(rp, rx, f["Q"], f["K"], f["V"])
        b = oracle.gt_bwd(rp, rx, f["Q"], f["K"], f["V"], f["dO"])
        gpu = {"O": r["O"], "LSE": r["LSE"], "dQ": b["dQ"], "dK": b["dK"], "dV": b["dV"]}
        key = "O"
    rec = bench.cpu_baseline(wl, rp, rx, 0.05, gpu=gpu)
    par = rec["parity"]
    assert par["within_tolerance"] and par["rows"] > 0, par
    bad = dict(gpu)
    bad[key] = np.array(gpu[key], dtype=np.float64 if key != "out" else np.float32, copy=True)
    bad[key][...] += 0.5 * (np.abs(bad[key]).max() + 1.0)
    assert not bench.cpu_baseline(wl, rp, rx, 0.05, gpu=bad)["parity"]["within_tolerance"]


def test_memory_record_adds_up():
    """The bench line's memory object: library bytes are the plan's structures
    plus workspace; caller bytes count the graph and every tensor of the step."""
    import numpy as np
    import torch

    class Plan:
        pass

    g = types.SimpleNamespace(gnn_plan_export=lambda plan: {"structure_bytes": 1000, "workspace_bytes": 24})
    T = {"Q": torch.zeros(10, 2, 4), "LSE": torch.zeros(10, 2)}
    ip, ix = torch.zeros(11, dtype=torch.int32), torch.zeros(30, dtype=torch.int32)
    wl = types.SimpleNamespace(kind="gt", heads=2)
    rec = bench.memory_record(g, Plan(), T, ip, ix, wl, 30)
    assert rec["library_bytes"] == 1024 and rec["caller_graph_bytes"] == 4 * 41
    assert rec["caller_feature_and_output_bytes"] == 4 * (80 + 20)
    assert rec["per_edge_score_bytes_not_materialised"] == 30 * 2 * 4
