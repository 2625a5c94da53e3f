#!/usr/bin/env python3
"""Benchmark of fused CSR neighbourhood attention on one MI355X.

A step is one pass of the attention hot path over the workload's graph with
inputs resident in HBM: the forward (Graph Transformer or GATv2, light and
heavy kernels plus the heavy merge), and for workloads that carry an upstream
gradient also the LSE-recompute backward (destination and source passes).
Graph preprocessing (CSR build, bucketing, transposed adjacency) runs once
before timing and is reported separately.

Default workload: GATv2 forward on the Zipf(2.1) in-degree graph
(N = 100,000, mean in-degree 50, H = 8, D = 16, fp32).

Output: one JSON line on stdout (metric GEdges/s = edges incl. self-loops per
second of step time), with a roofline object for the dominant kernel and the
fp64 CPU oracle timed on a bounded sample as a baseline. The step time is
taken without per-kernel events; the same steps are then repeated with a
HIP event pair around every kernel for the per-kernel durations.

Other modes:
  --copy-probe          run only a plain device copy of known size (counter
                        calibration runs under rocprofv3 --pmc)
  --summarize DIR ...   turn rocprofv3 CSV output in DIR into a short text
                        summary (see --help)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEdges/s and achieved HBM GB/s (% of peak) for fused CSR attention fwd/bwd"
HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "gatv2_zipf21_n100k"
_CSRC = os.path.join(ROOT, "io_aware_sparse_amd", "csrc")
# sources whose change makes a committed counter summary stale, per kernel family
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in ("attn.hip", "attn_core.h", "attn_tile.hip", "attn_gat.hip",
                                                   "device.h")]
REDUCE_SOURCES = [os.path.join(_CSRC, f) for f in ("reduce.hip", "attn_core.h", "device.h")]
SPMM_SOURCES = [os.path.join(_CSRC, f) for f in ("spmm.hip", "attn_core.h", "device.h")]
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text without comments and blank lines, so that a comment edit
    does not mark a counter summary as stale."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(kernel: str = "") -> str:
    """Hash of the code (comments stripped) of `kernel`'s family's sources
    (reduce_*, spmm_*, else attention)."""
    h = hashlib.sha256()
    for f in (REDUCE_SOURCES if kernel.startswith("reduce_") else SPMM_SOURCES if kernel.startswith("spmm_")
              else KERNEL_SOURCES):
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


# --------------------------------------------------------------- byte model

def step_counts(info, indptr, indices, tiled):
    """Per-kernel unit counts for the byte model."""
    import numpy as np
    ip = indptr.astype(np.int64)
    n = ip.size - 1
    deg = np.diff(ip)
    c = {"N": n, "E": int(ip[-1])}
    light = info["light_nt"] if tiled else info["light"]
    heavy = info["heavy"]
    c["main_rows"] = int(light.size + heavy.size)
    c["main_light"] = int(light.size)
    c["main_heavy"] = int(heavy.size)
    c["main_edges"] = int(deg[light].sum() + deg[heavy].sum())
    if info.get("has_csc"):
        odeg = np.diff(info["cindptr"].astype(np.int64))
        cl = info["c_light_nt"] if tiled else info["c_light"]
        ch = info["c_heavy"]
        c["src_rows"] = int(cl.size + ch.size)
        c["src_light"] = int(cl.size)
        c["src_heavy"] = int(ch.size)
        c["src_edges"] = int(odeg[cl].sum() + odeg[ch].sum())
    if tiled:
        c["tiles"] = int(info["n_tiles"])
        rows = (16 * info["trb"][:, None].astype(np.int64) + np.arange(16)).ravel()
        rows = rows[rows < n]
        rdeg = np.diff(info["rindptr"].astype(np.int64))
        c["tile_rows"] = int(rows.size)
        c["tile_res_edges"] = int(rdeg[rows].sum())
        if info.get("has_csc"):
            srcs = (16 * info["tcb"][:, None].astype(np.int64) + np.arange(16)).ravel()
            srcs = srcs[srcs < n]
            rcdeg = np.diff(info["rcindptr"].astype(np.int64))
            c["tile_srcs"] = int(srcs.size)
            c["tile_res_src_edges"] = int(rcdeg[srcs].sum())
    return c


def kernel_bytes(kind, c, H, D, s, v_alias=True):
    """Algorithmic HBM bytes one launch of kernel `kind` must move.

    R = H*D*s is one node's feature row. Counted: the CSR structure the
    kernel walks, one gathered row per edge per gathered table (a 16x16 tile
    counts its 16 source rows per table once: 32R per tile for two tables),
    per-node rows read or written once, per-node statistics and tile
    metadata (40 B per tile). Not counted: heavy partials (workspace) and any
    re-read a cache would serve."""
    R = H * D * s
    rows, E, nl, nh = c.get("main_rows", 0), c.get("main_edges", 0), c.get("main_light", 0), c.get("main_heavy", 0)
    if kind in ("gt_fwd_main", "gatv2_fwd_main"):
        g = R * E * (1 if (kind == "gatv2_fwd_main" and v_alias) else 2)
        extra = 4 * H * D if kind == "gatv2_fwd_main" else 0
        return 4 * (rows + 1) + 4 * E + g + R * rows + (R + 4 * H) * nl + extra
    if kind in ("gt_fwd_merge", "gatv2_fwd_merge"):
        return (R + 4 * H) * nh
    if kind == "gt_bwd_dst_main":     # reads Q, dO, LSE; gathers K, V; writes dQ and (lse, Delta)
        return 4 * (rows + 1) + 4 * E + 2 * R * E + (2 * R + 4 * H) * rows + (R + 8 * H) * nl
    if kind == "gt_bwd_dst_merge":
        return (R + 8 * H) * nh
    sr, se, sl, sh = c.get("src_rows", 0), c.get("src_edges", 0), c.get("src_light", 0), c.get("src_heavy", 0)
    if kind == "gt_bwd_src_main":     # reads K, V; gathers Q, dO and (lse, Delta); writes dK, dV
        return 4 * (sr + 1) + 4 * se + (2 * R + 8 * H) * se + 2 * R * sr + 2 * R * sl
    if kind == "gt_bwd_src_merge":
        return 2 * R * sh
    if kind == "gatv2_bwd_dst_main":  # reads XD, dO, LSE, att; gathers XS (+V); writes dXD, stats, d_att rows
        return (4 * (rows + 1) + 4 * E + R * E * (1 if v_alias else 2) + (2 * R + 4 * H) * rows + 4 * H * D
                + (R + 8 * H + 4 * H * D) * nl)
    if kind == "gatv2_bwd_dst_merge":
        return (R + 8 * H + 4 * H * D) * nh
    if kind == "gatv2_bwd_src_main":  # reads XS (+V); gathers XD, dO and stats; writes dXS (+dV)
        nv = 1 if v_alias else 2
        return 4 * (sr + 1) + 4 * se + (2 * R + 8 * H) * se + nv * R * sr + nv * R * sl + 4 * H * D
    if kind == "gatv2_bwd_src_merge":
        return (1 if v_alias else 2) * R * sh
    if kind == "gatv2_bwd_datt":      # per-node d_att rows read once
        return 4 * H * D * c.get("N", 0)
    t, tr, te = c.get("tiles", 0), c.get("tile_rows", 0), c.get("tile_res_edges", 0)
    F, rsz = H * D, H * D * s          # reduction layer: F features, rsz bytes per row
    diff = 1 if c.get("msg") == "diff" else 0
    if kind == "spmm_main":             # index + weight per entry, one gathered row; light rows written
        return 4 * (rows + 1) + 8 * E + rsz * E + rsz * nl
    if kind == "spmm_merge":
        return rsz * nh
    if kind == "spmm_t_main":           # the same over the transposed adjacency
        return 4 * (sr + 1) + 8 * se + rsz * se + rsz * sl
    if kind == "spmm_t_merge":
        return rsz * sh
    if kind == "reduce_fwd_init":       # identity keys of the heavy rows
        return 8 * F * nh
    if kind == "reduce_fwd_main":       # gathers a row per edge; light rows write out and arg
        return 4 * (rows + 1) + 4 * E + rsz * E + (rsz + 4 * F + 4) * nl + diff * rsz * rows
    if kind == "reduce_fwd_final":      # heavy rows: keys in, winner's row slice, out and arg
        return 8 * F * nh + (rsz * (1 + diff) + rsz + 4 * F + 4) * nh
    if kind == "reduce_bwd_main":       # gathers dOut and arg rows per transposed edge; writes dX
        return 4 * (sr + 1) + 4 * se + (rsz + 4 * F) * se + (rsz + 4) * sl + diff * (rsz + 8) * sr
    if kind == "reduce_bwd_merge":
        return rsz * sh
    if kind == "gt_tile_fwd":         # tiles: K, V blocks; rows: Q in, O and LSE out; residual gathers
        return 40 * t + 32 * R * t + 4 * (tr + 1) + (4 + 2 * R) * te + R * tr + (R + 4 * H) * tr
    if kind == "gt_tile_bwd_dst":     # tiles: K, V blocks; rows: Q, dO, LSE in, dQ, stats out
        return 40 * t + 32 * R * t + 4 * (tr + 1) + (4 + 2 * R) * te + (2 * R + 4 * H) * tr + (R + 8 * H) * tr
    ts, tse = c.get("tile_srcs", 0), c.get("tile_res_src_edges", 0)
    if kind == "gt_tile_bwd_src":     # tiles: Q, dO blocks + 16 row stats; sources: K, V in, dK, dV out
        return 40 * t + (32 * R + 16 * 8 * H) * t + 4 * (ts + 1) + (4 + 2 * R + 8 * H) * tse + 4 * R * ts
    if kind == "spmm_wsb":            # tiles: mask, X block, 16 degrees; rows: residual range, degree, Y out;
        return 40 * t + (16 * rsz + 128) * t + 4 * (tr + 1) + 8 * tr + (8 + rsz) * te + rsz * tr  # residual entries
    if kind == "spmm_t_wsb":          # the same by column block over the transposed residual
        return 40 * t + (16 * rsz + 128) * t + 4 * (ts + 1) + 8 * ts + (8 + rsz) * tse + rsz * ts
    return 0


# ------------------------------------------------------ what the rate means

INFINITY_CACHE_BYTES = 256 << 20      # MI355X last-level (Infinity) cache
# Random-gather rate (GB/s) of 64 row gathers per destination from one table,
# by row bytes and table MiB, quoted from profiles/bw_probe__read_copy_gather.txt.
GATHER_CEILING_GBPS = {
    256: [(64, 8107.5), (256, 7692.6), (1024, 7245.8), (4096, 6376.6)],
    512: [(64, 8067.2), (256, 7580.3), (1024, 7153.9), (4096, 6311.5)],
    1024: [(64, 8073.7), (256, 7630.7), (1024, 7197.6), (4096, 6290.9)],
}


def gathered_tables(kind, H, D, s, N, v_alias=True):
    """(bytes of the node tables kernel `kind` gathers rows from per edge,
    bytes of one gathered row)."""
    R = H * D * s
    F4 = 4 * H * D
    two = {"gt_fwd_main", "gt_bwd_dst_main", "gt_bwd_src_main", "gatv2_bwd_src_main", "gt_tile_fwd",
           "gt_tile_bwd_dst", "gt_tile_bwd_src"}
    if kind in two:
        return 2 * R * N, R
    if kind in ("gatv2_fwd_main", "gatv2_bwd_dst_main"):
        return (1 if v_alias else 2) * R * N, R
    if kind in ("reduce_fwd_main", "spmm_main", "spmm_t_main", "spmm_wsb", "spmm_t_wsb"):
        return R * N, R
    if kind == "reduce_bwd_main":                 # dOut rows and winner rows (int32 per feature)
        return (R + F4) * N, R
    return 0, R


def gather_ceiling(table_bytes, row_bytes):
    """Measured gather ceiling (GB/s) for a gathered working set of
    table_bytes in rows of row_bytes: the nearest row size, interpolated in
    log(table size) between the measured sizes and held at the ends."""
    import math
    rows = min(GATHER_CEILING_GBPS, key=lambda r: abs(math.log(max(row_bytes, 1) / r)))
    pts = GATHER_CEILING_GBPS[rows]
    mib = max(table_bytes, 1) / (1 << 20)
    if mib <= pts[0][0]:
        return pts[0][1]
    if mib >= pts[-1][0]:
        return pts[-1][1]
    for (m0, c0), (m1, c1) in zip(pts, pts[1:]):
        if m0 <= mib <= m1:
            t = math.log(mib / m0) / math.log(m1 / m0)
            return c0 + t * (c1 - c0)
    return pts[-1][1]


def roofline_context(kind, H, D, s, N, achieved, traffic, avg_us, v_alias=True):
    """Fields that say what the model fraction measures for this kernel: the
    gathered working set, whether it fits the Infinity Cache (then the rate is
    mostly cache bandwidth and the bound is labelled "infinity-cache", else
    "hbm"), the counter rate against the measured gather ceiling for that
    working set, and whether the model is a bound at all (a model fraction
    above 1 means caches served repeated rows)."""
    tb, row = gathered_tables(kind, H, D, s, N, v_alias)
    resident = tb <= INFINITY_CACHE_BYTES
    ceil = gather_ceiling(tb, row)
    out = {
        "bound": "infinity-cache" if resident else "hbm",
        "gathered_table_bytes": int(tb),
        "gathered_row_bytes": int(row),
        "cache_resident": bool(resident),
        "gather_ceiling_GBps": round(ceil, 1),
        "gather_ceiling_source": f"profiles/bw_probe__read_copy_gather.txt ({row}-byte rows, "
                                 f"{tb / (1 << 20):.0f} MiB working set)",
    }
    frac = achieved / HBM_PEAK_GBPS if achieved else None
    out["model_is_bound"] = bool(frac is not None and frac <= 1.0)
    if traffic and avg_us:
        rate = traffic / (avg_us * 1e-6) / 1e9
        out["traffic_frac_of_gather_ceiling"] = round(rate / ceil, 4)
    else:
        out["traffic_frac_of_gather_ceiling"] = None
    notes = []
    if resident:
        notes.append(f"the gathered tables ({tb / 1e6:.0f} MB) fit in the 256 MB Infinity Cache, so the "
                     "gathers are served mostly from it: frac is model bytes over the 8 TB/s HBM peak, not HBM "
                     "utilisation")
    if frac is not None and frac > 1.0:
        notes.append("model fraction above 1: the per-edge model is not a bound here (caches served "
                     "repeated rows)")
    out["note"] = "; ".join(notes) if notes else "gathered tables exceed the Infinity Cache: the gathers reach HBM"
    return out


# ---------------------------------------------------------------- profiles

def profile_tag(workload: str, tiles: bool, extra_backward: bool, reorder: str) -> str:
    """Name of a run variant in the profile summaries: the workload, then
    __tiles (tile path on), __bwd (gradient pass added to a forward-only
    workload) and __<order> (graph relabelled), in that order."""
    return (workload + ("__tiles" if tiles else "") + ("__bwd" if extra_backward else "")
            + (f"__{reorder}" if reorder != "none" else ""))


def read_traffic(kernel: str, tag: str):
    """Scaled HBM bytes per launch from a committed counter summary of the
    same run variant (`profile_tag`), or None if there is none or it was
    taken on different kernel sources."""
    path = os.path.join(PROFILES, f"{kernel}__{tag}__counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _counter_means(d, counter, pattern):
    import re
    vals = {}
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and re.search(pattern, r["Kernel_Name"]):
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for /{pattern}/ under {d}")
    name, v = max(vals.items(), key=lambda kv: sum(kv[1]) / len(kv[1]))
    return name, sum(v) / len(v), len(v)


def traffic_summary(args) -> int:
    """Scaled HBM traffic per launch of one kernel from four counter runs:
    FETCH_SIZE and WRITE_SIZE of the kernel, and of a plain copy of known
    size (--copy-probe) that calibrates each counter (KiB per dispatch)."""
    fdir, wdir, cfdir, cwdir = args.traffic
    kname, fetch_kib, nf = _counter_means(fdir, "FETCH_SIZE", args.kernel_regex)
    _, write_kib, nw = _counter_means(wdir, "WRITE_SIZE", args.kernel_regex)
    _, cfetch, _ = _counter_means(cfdir, "FETCH_SIZE", "copyBuffer")
    _, cwrite, _ = _counter_means(cwdir, "WRITE_SIZE", "copyBuffer")
    known_kib = (args.copy_mib << 20) / 1024.0
    f_fac, w_fac = known_kib / cfetch, known_kib / cwrite
    fetch_b = fetch_kib * 1024 * f_fac
    write_b = write_kib * 1024 * w_fac
    lines = [
        f"# HBM traffic of {args.kernel} on {args.workload}",
        f"# commands (from the repository root, under /tmp as working directory):",
        f"#   rocprofv3 --pmc FETCH_SIZE -d {fdir} -o fetch --output-format csv -- python3 bench.py {args.bench_args}",
        f"#   rocprofv3 --pmc WRITE_SIZE -d {wdir} -o write --output-format csv -- python3 bench.py {args.bench_args}",
        f"#   rocprofv3 --pmc FETCH_SIZE -d {cfdir} -o cf --output-format csv -- python3 bench.py --copy-probe",
        f"#   rocprofv3 --pmc WRITE_SIZE -d {cwdir} -o cw --output-format csv -- python3 bench.py --copy-probe",
        f"#   python3 bench.py --traffic {fdir} {wdir} {cfdir} {cwdir} --kernel {args.kernel} "
        f"--kernel-regex '{args.kernel_regex}' --workload {args.workload} --bench-args '{args.bench_args}'",
        f"kernel_symbol: {kname}",
        f"source_sha256: {kernel_source_hash(args.kernel)}",
        f"fetch_kib_per_dispatch: {fetch_kib:.1f}  (n={nf})",
        f"write_kib_per_dispatch: {write_kib:.1f}  (n={nw})",
        f"copy_probe_kib: {known_kib:.0f}",
        f"copy_fetch_kib: {cfetch:.1f}  -> fetch scale {f_fac:.4f}",
        f"copy_write_kib: {cwrite:.1f}  -> write scale {w_fac:.4f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
    ]
    text = "\n".join(lines) + "\n"
    out = args.out or os.path.join(PROFILES, f"{args.kernel}__{args.workload}__counters.txt")
    with open(out, "w") as f:
        f.write(text)
    print(text)
    return 0


CACHE_TEXT = {"flushed": "flushed: 512 MiB fill before every step, outside the timed events",
              "warm": "warm: steps back to back"}
UNIT_COUNTERS = ["SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
                 "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE",
                 "TCC_HIT_sum", "TCC_MISS_sum"]
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8


def _dispatch_means(d, pattern):
    """Mean per dispatch of every counter for the kernel matching pattern
    (rows of one dispatch and counter are summed first)."""
    import re
    per = {}
    dur = {}
    names = set()
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                if re.search(pattern, r["Kernel_Name"]):
                    names.add(r["Kernel_Name"])
                    key = (fn, r["Dispatch_Id"])
                    per.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
                    per[key][r["Counter_Name"]] += float(r["Counter_Value"])
                    dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    if not per:
        raise SystemExit(f"no counter rows for /{pattern}/ under {d}")
    out = {}
    for c in {c for v in per.values() for c in v}:
        vals = [v[c] for v in per.values() if c in v]
        out[c] = sum(vals) / len(vals)
    out["duration_s"] = sum(dur.values()) / len(dur)
    return sorted(names), out, len(per)


def units_summary(args) -> int:
    """Execution-unit counters of one kernel (one rocprofv3 --pmc pass with
    UNIT_COUNTERS), with rocprof's own derived-metric expressions."""
    names, m, n = _dispatch_means(args.units, args.kernel_regex)
    # GRBM_GUI_ACTIVE comes summed over the XCDs' instances; rocprof's derived
    # metrics take the max over them, i.e. the busy cycles of one XCD
    gui = m.get("GRBM_GUI_ACTIVE", float("nan")) / XCD_NUM
    hit, miss = m.get("TCC_HIT_sum", 0.0), m.get("TCC_MISS_sum", 0.0)
    lds_act, lds_cf = m.get("SQ_LDS_IDX_ACTIVE", 0.0), m.get("SQ_LDS_BANK_CONFLICT", 0.0)
    derived = {
        "VALUBusy_pct (100*SQ_ACTIVE_INST_VALU/CU_NUM/GUI)":
            100 * m.get("SQ_ACTIVE_INST_VALU", 0.0) / CU_NUM / gui,
        "MfmaUtil_pct (100*SQ_VALU_MFMA_BUSY_CYCLES/(GUI*SIMD_NUM))":
            100 * m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * SIMD_NUM),
        "LdsBankConflict_per_access (SQ_LDS_BANK_CONFLICT/(SQ_LDS_IDX_ACTIVE-SQ_LDS_BANK_CONFLICT))":
            lds_cf / (lds_act - lds_cf) if lds_act > lds_cf else 0.0,
        "LDSBankConflict_pct_of_time (100*SQ_LDS_BANK_CONFLICT/GUI/CU_NUM)":
            100 * lds_cf / gui / CU_NUM,
        "OccupancyPercent (400*SQ_WAVE_CYCLES/GUI/CU_NUM/32)":
            400 * m.get("SQ_WAVE_CYCLES", 0.0) / gui / CU_NUM / 32,
        "L2_hit_pct (100*TCC_HIT_sum/(TCC_HIT_sum+TCC_MISS_sum))":
            100 * hit / (hit + miss) if hit + miss > 0 else float("nan"),
    }
    lines = [
        f"# execution-unit counters of {args.kernel} on {args.workload}",
        f"# command (from the repository root, under /tmp as working directory):",
        f"#   rocprofv3 --pmc {' '.join(UNIT_COUNTERS)} -d {args.units} -o units --output-format csv "
        f"-- python3 bench.py {args.bench_args}",
        f"#   python3 bench.py --units {args.units} --kernel {args.kernel} --kernel-regex '{args.kernel_regex}' "
        f"--workload {args.workload} --bench-args '{args.bench_args}'",
        f"# CU_NUM {CU_NUM}, SIMD_NUM {SIMD_NUM}; values are means per dispatch (n={n}); "
        f"GRBM_GUI_ACTIVE below is the sum over {XCD_NUM} XCDs, the formulas use sum/{XCD_NUM}",
        f"dispatch_us: {m['duration_s'] * 1e6:.2f}",
        f"clock_GHz (GRBM_GUI_ACTIVE/{XCD_NUM}/dispatch time): {gui / m['duration_s'] / 1e9:.3f}",
        *[f"kernel_symbol: {k}" for k in names],
        f"source_sha256: {kernel_source_hash(args.kernel)}",
        *[f"{c}: {m[c]:.1f}" for c in UNIT_COUNTERS if c in m],
        f"GUI (GRBM_GUI_ACTIVE/{XCD_NUM}): {gui:.1f}",
        *[f"{k}: {v:.3f}" for k, v in derived.items()],
    ]
    text = "\n".join(lines) + "\n"
    out = args.out or os.path.join(PROFILES, f"{args.kernel}__{args.workload}__units.txt")
    with open(out, "w") as f:
        f.write(text)
    print(text)
    return 0


def summarize(args) -> int:
    """Summarise rocprofv3 output (kernel stats or counters) into text."""
    out = []
    stats = glob.glob(os.path.join(args.summarize, "**", "*kernel_stats.csv"), recursive=True)
    counters = glob.glob(os.path.join(args.summarize, "**", "*counter_collection.csv"), recursive=True)
    out.append(f"# rocprofv3 summary of {args.summarize}")
    if args.command:
        out.append(f"# command: {args.command}")
    out.append(f"source_sha256: {kernel_source_hash(args.kernel or '')}")
    for fn in stats:
        out.append(f"## kernel stats ({os.path.basename(fn)})")
        with open(fn) as f:
            rows = list(csv.DictReader(f))
        rows.sort(key=lambda r: -float(r.get("TotalDurationNs", 0) or 0))
        out.append(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_ms':>10} {'pct':>6}  kernel")
        for r in rows[:25]:
            out.append(f"{r['Calls']:>6} {float(r['AverageNs'])/1e3:10.2f} {float(r['MinNs'])/1e3:10.2f} "
                       f"{float(r['MaxNs'])/1e3:10.2f} {float(r['TotalDurationNs'])/1e6:10.3f} "
                       f"{float(r['Percentage']):6.2f}  {r['Name'][:140]}")
    for fn in counters:
        out.append(f"## counters ({os.path.basename(fn)}), per dispatch")
        with open(fn) as f:
            rows = list(csv.DictReader(f))
        agg = {}
        for r in rows:
            key = (r["Kernel_Name"], r["Counter_Name"])
            agg.setdefault(key, []).append(float(r["Counter_Value"]))
        for (k, c), v in sorted(agg.items()):
            out.append(f"{c:>14} n={len(v):4d} mean={sum(v)/len(v):16.1f} min={min(v):16.1f} max={max(v):16.1f}  {k[:120]}")
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)
    return 0


# ----------------------------------------------------------------- workload

def setup(name, plan_opts, backward=None, reorder="none", spmm_norm="gcn"):
    import numpy as np
    import torch

    import io_aware_sparse_amd as g
    import workloads

    t0 = time.time()
    wl = workloads.make(name, backward=backward)
    t_gen = time.time() - t0
    n, H, D = wl.n_nodes, wl.heads, wl.dim
    dev = torch.device("cuda:0")

    def feat(nm):
        if wl.dtype == "bf16":
            t = torch.from_numpy(wl.bits[nm].view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            t = torch.from_numpy(wl.feats[nm]).to(dev)
        return t if perm is None else g.gnn_permute_rows(t, perm)

    src = torch.from_numpy(wl.src).to(dev)
    dst = torch.from_numpy(wl.dst).to(dev)
    torch.cuda.synchronize()
    t0 = time.time()
    indptr, indices = g.gnn_csr_build(src, dst, n)
    torch.cuda.synchronize()
    t_csr = time.time() - t0
    del src, dst
    perm, t_reorder, t_relabel = None, 0.0, 0.0
    if reorder != "none":
        t0 = time.time()
        perm = g.gnn_reorder(indptr, indices, reorder)
        torch.cuda.synchronize()
        t_reorder = time.time() - t0
        t0 = time.time()
        indptr, indices = g.gnn_permute_graph(indptr, indices, perm)
        torch.cuda.synchronize()
        t_relabel = time.time() - t0
    t0 = time.time()
    plan = g.gnn_plan_create(indptr, indices, want_csc=wl.backward, **plan_opts)
    torch.cuda.synchronize()
    t_plan = time.time() - t0
    tensors = {}
    if wl.kind == "spmm":
        g.gnn_spmm_prepare(plan, spmm_norm)           # cached per graph: outside the timed steps
        F = H * D
        tensors["X"] = feat("X").reshape(n, F)
        tensors["Y"] = torch.empty_like(tensors["X"])
        if wl.backward:
            tensors["dO"] = feat("dO").reshape(n, F)
            tensors["dX"] = torch.empty_like(tensors["X"])
        torch.cuda.synchronize()
        prep = dict(generate_s=round(t_gen, 3), csr_build_ms=round(1e3 * t_csr, 3),
                    plan_create_ms=round(1e3 * t_plan, 3), reorder=reorder, reorder_ms=round(1e3 * t_reorder, 3),
                    relabel_ms=round(1e3 * t_relabel, 3), norm=spmm_norm)
        return wl, indptr, indices, plan, tensors, int(indices.numel()), prep
    if wl.kind == "reduce":
        F = H * D
        tensors["X"] = feat("X").reshape(n, F)
        tensors["out"] = torch.empty_like(tensors["X"])
        tensors["arg"] = torch.empty((n, F), dtype=torch.int32, device=dev)
        if wl.backward:
            tensors["dO"] = feat("dO").reshape(n, F)
            tensors["dX"] = torch.empty_like(tensors["X"])
        torch.cuda.synchronize()
        prep = dict(generate_s=round(t_gen, 3), csr_build_ms=round(1e3 * t_csr, 3),
                    plan_create_ms=round(1e3 * t_plan, 3), reorder=reorder, reorder_ms=round(1e3 * t_reorder, 3),
                    relabel_ms=round(1e3 * t_relabel, 3))
        return wl, indptr, indices, plan, tensors, int(indices.numel()), prep
    if wl.kind == "gt":
        for nm in ("Q", "K", "V"):
            tensors[nm] = feat(nm)
        if wl.backward:
            tensors["dO"] = feat("dO")
    else:
        tensors["XD"], tensors["XS"] = feat("XD"), feat("XS")
        tensors["att"] = torch.from_numpy(wl.att).to(dev)
        if wl.backward:
            tensors["dO"] = feat("dO")
    E = int(indices.numel())
    tensors["O"] = torch.empty_like(tensors["Q"] if wl.kind == "gt" else tensors["XD"])
    tensors["LSE"] = torch.empty((n, H), dtype=torch.float32, device=dev)
    if wl.backward:
        ref = tensors["Q"] if wl.kind == "gt" else tensors["XD"]
        for nm in ("dQ", "dK", "dV"):
            tensors[nm] = torch.empty_like(ref)
        tensors["d_att"] = torch.empty((H, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    prep = dict(generate_s=round(t_gen, 3), csr_build_ms=round(1e3 * t_csr, 3), plan_create_ms=round(1e3 * t_plan, 3),
                reorder=reorder, reorder_ms=round(1e3 * t_reorder, 3), relabel_ms=round(1e3 * t_relabel, 3))
    return wl, indptr, indices, plan, tensors, E, prep


def make_step(g, wl, indptr, indices, plan, T, op="max", msg="src"):
    if wl.kind == "spmm":
        def step():
            g.gnn_spmm(plan, indptr, indices, T["X"], Y=T["Y"])
            if wl.backward:
                g.gnn_spmm(plan, indptr, indices, T["dO"], transpose=True, Y=T["dX"])
        return step
    if wl.kind == "reduce":
        def step():
            g.gnn_reduce_fwd(plan, indptr, indices, T["X"], op, msg, out=T["out"], arg=T["arg"])
            if wl.backward:
                g.gnn_reduce_bwd(plan, indptr, indices, T["dO"], T["arg"], msg, dX=T["dX"])
        return step
    if wl.kind == "gatv2" and not wl.backward:
        def step():
            g.gatv2_attn_fwd(plan, indptr, indices, T["XD"], T["XS"], T["att"], negative_slope=0.2, O=T["O"],
                             LSE=T["LSE"])
    elif wl.kind == "gatv2":
        def step():
            g.gatv2_attn_fwd(plan, indptr, indices, T["XD"], T["XS"], T["att"], negative_slope=0.2, O=T["O"],
                             LSE=T["LSE"])
            g.gatv2_attn_bwd(plan, indptr, indices, T["XD"], T["XS"], T["att"], T["dO"], T["LSE"],
                             negative_slope=0.2, dXD=T["dQ"], dXS=T["dK"], d_att=T["d_att"])
    elif not wl.backward:
        def step():
            g.gnn_attn_fwd(plan, indptr, indices, T["Q"], T["K"], T["V"], O=T["O"], LSE=T["LSE"])
    else:
        def step():
            g.gnn_attn_fwd(plan, indptr, indices, T["Q"], T["K"], T["V"], O=T["O"], LSE=T["LSE"])
            g.gnn_attn_bwd(plan, indptr, indices, T["Q"], T["K"], T["V"], T["O"], T["dO"], T["LSE"],
                           dQ=T["dQ"], dK=T["dK"], dV=T["dV"])
    return step


def graph_replay(g, plan, indptr, indices, T, steps, E):
    """The GT forward through the allocation-free entry point, captured once
    into a HIP graph (torch.cuda.CUDAGraph) and replayed back to back with
    warm caches: the host issues one graph launch per step instead of the
    binding's checks and the kernel launches. Its outputs must equal the
    eager call's bit for bit. None if the heavy rows need more scratch than
    the entry point holds."""
    import torch
    O0, L0 = T["O"].clone(), T["LSE"].clone()
    args = (plan, indptr, indices, T["Q"], T["K"], T["V"], T["O"], T["LSE"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    try:
        with torch.cuda.stream(side):
            for _ in range(3):
                g.gnn_attn_fwd_noalloc(*args)
    except g.GnnError as ex:
        return {"skipped": str(ex)}
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.gnn_attn_fwd_noalloc(*args)
    for _ in range(3):
        graph.replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    same = torch.equal(T["O"].view(torch.int16) if T["O"].dtype == torch.bfloat16 else T["O"].view(torch.int32),
                       O0.view(torch.int16) if O0.dtype == torch.bfloat16 else O0.view(torch.int32)) and \
        torch.equal(T["LSE"].view(torch.int32), L0.view(torch.int32))
    if not same:
        raise RuntimeError("graph replays differ from the eager forward")
    ms = ev0.elapsed_time(ev1) / steps
    return {"ms_per_step": round(ms, 5), "value": round(E / (ms * 1e-3) / 1e9, 4),
            "note": "the same forward through gnn_attn_fwd_noalloc, captured once in a HIP graph and replayed "
                    "back to back (warm caches); outputs equal the eager call's bit for bit"}


def host_cpu() -> str:
    """CPU model and the logical CPUs this process may run on."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {len(os.sched_getaffinity(0))} of {os.cpu_count()} logical CPUs in this process's affinity"


def memory_record(g, plan, T, indptr, indices, wl, E):
    """Device memory of the measured run: what the library holds (the plan's
    structures and its workspace, grown to the largest request) and what the
    caller holds (graph, features and outputs). No per-edge buffer exists; for
    scale, the bytes of one fp32 score per edge and head, the smallest
    intermediate a materialising implementation keeps."""
    info = g.gnn_plan_export(plan)
    tensors = sum(t.numel() * t.element_size() for t in T.values())
    graph = indptr.numel() * indptr.element_size() + indices.numel() * indices.element_size()
    lib = int(info["structure_bytes"]) + int(info["workspace_bytes"])
    rec = {"library_bytes": lib, "plan_structure_bytes": int(info["structure_bytes"]),
           "plan_workspace_bytes": int(info["workspace_bytes"]), "caller_graph_bytes": int(graph),
           "caller_feature_and_output_bytes": int(tensors)}
    if wl.kind in ("gt", "gatv2"):
        rec["per_edge_score_bytes_not_materialised"] = int(E) * wl.heads * 4
    return rec


# parity bar of the outputs (condition-scaled error), by storage type
PARITY_TOL = {"f32": 1e-4, "bf16": 2e-2}


def cpu_baseline(wl, rp, rx, target_s, threads=None, op="max", msg="src", norm="gcn", gpu=None):
    """fp64 oracle on a seeded sample of destination rows (and the same nodes
    as sources for the gradient), sized to about target_s seconds. With the
    GPU's outputs of the measured steps (`gpu`, host arrays), the sampled
    rows of the last timed pass are also compared with them."""
    import numpy as np

    import oracle

    all_threads = oracle.num_threads()
    if threads:
        oracle.set_threads(threads)
    try:
        return _cpu_baseline(oracle, wl, rp, rx, target_s, op, msg, norm, gpu)
    finally:
        oracle.set_threads(all_threads)


def _parity(oracle, wl, rows, res, gpu, op, msg):
    """Condition-scaled and normwise errors of the GPU outputs on the sampled
    rows (sources for the gradients) against the oracle's results."""
    import numpy as np
    tol = PARITY_TOL[wl.dtype]
    out = {"rows": int(rows.size), "tolerance": tol, "max_scaled_error": {}, "normwise_error": {}}

    def add(name, x, ref, scale, t=tol):
        e = float(oracle.scaled_error(x, ref, scale))
        out["max_scaled_error"][name] = float(f"{e:.3e}")
        out["normwise_error"][name] = float(f"{float(oracle.normwise_error(x, ref)):.3e}")
        return e <= t

    ok = True
    if wl.kind == "spmm":
        ok &= add("Y", gpu["Y"][rows], res["f"]["Y"], res["f"]["S"])
        if "b" in res:
            ok &= add("dX", gpu["dX"][rows], res["b"]["Y"], res["b"]["S"])
    elif wl.kind == "reduce":
        ref = res["f"]
        ro = oracle.round_bf16(ref["out"]) if (wl.dtype == "bf16" and msg == "diff") else ref["out"]
        arg_eq = bool(np.array_equal(gpu["arg"][rows], ref["arg"]))
        val_eq = bool(np.array_equal(gpu["out"][rows].astype(np.float32).view(np.uint32),
                                     np.asarray(ro, np.float32).view(np.uint32)))
        out.update(winners_bit_exact=arg_eq, values_bit_exact=val_eq,
                   note="forward only: a sample of rows does not give its sources' whole gradient")
        ok &= arg_eq and val_eq
    else:
        ok &= add("O", gpu["O"][rows], res["f"]["O"], res["f"]["SO"])
        ok &= add("LSE", gpu["LSE"][rows], res["f"]["LSE"], res["f"]["SL"], PARITY_TOL["f32"])
        if "b" in res:
            b = res["b"]
            if wl.kind == "gatv2":
                ok &= add("dXD", gpu["dQ"][rows], b["dXD"], b["SdXD"])
                ok &= add("dXS", gpu["dK"][rows], b["dXS"], b["SdXS"])
            else:
                ok &= add("dQ", gpu["dQ"][rows], b["dQ"], b["SdQ"])
                ok &= add("dK", gpu["dK"][rows], b["dK"], b["SdK"])
                ok &= add("dV", gpu["dV"][rows], b["dV"], b["SdV"])
    out["within_tolerance"] = bool(ok)
    return out


def _cpu_baseline(oracle, wl, rp, rx, target_s, op, msg, norm, gpu=None):
    import numpy as np

    n = wl.n_nodes
    deg = np.diff(rp.astype(np.int64))
    rng = np.random.default_rng(12345)
    order = rng.permutation(n)
    csum = np.cumsum(deg[order])

    if wl.kind in ("reduce", "spmm"):
        X = wl.feats["X"].reshape(n, -1)
        dO = wl.feats["dO"].reshape(n, -1) if wl.backward else None
    elif wl.kind == "gt":
        Q, K, V = (np.asarray(wl.feats[k], np.float64) for k in ("Q", "K", "V"))
        dO = np.asarray(wl.feats["dO"], np.float64) if wl.backward else None
    else:
        XD, XS = (np.asarray(wl.feats[k], np.float64) for k in ("XD", "XS"))
        dO = np.asarray(wl.feats["dO"], np.float64) if wl.backward else None
    csc = oracle.csc(rp, rx, n) if wl.backward and wl.kind != "reduce" else None

    last = {}

    def run(edges):
        k = int(np.searchsorted(csum, edges)) + 1
        rows = np.sort(order[:min(k, n)])
        res = {}
        t0 = time.perf_counter()
        if wl.kind == "spmm":
            res["f"] = oracle.spmm(rp, rx, X, norm, rows=rows)
            if wl.backward:
                res["b"] = oracle.spmm(rp, rx, dO, norm, transpose=True, rows=rows)
        elif wl.kind == "reduce":
            res["f"] = oracle.segment_reduce(rp, rx, X, op, msg, rows=rows)
            if wl.backward:
                oracle.segment_reduce_bwd(rp, rx, dO[rows], res["f"]["arg"], msg, n_nodes=n, rows=rows)
        elif wl.kind == "gatv2":
            res["f"] = oracle.gatv2_fwd(rp, rx, XD, XS, wl.att, slope=0.2, rows=rows)
            if wl.backward:
                res["b"] = oracle.gatv2_bwd(rp, rx, XD, XS, wl.att, dO, slope=0.2, rows=rows, srcs=rows,
                                            csc_arrays=csc, want_da=False)
        else:
            res["f"] = oracle.gt_fwd(rp, rx, Q, K, V, rows=rows)
            if wl.backward:
                res["b"] = oracle.gt_bwd(rp, rx, Q, K, V, dO, rows=rows, srcs=rows, csc_arrays=csc)
        t = time.perf_counter() - t0
        last.update(rows=rows, res=res)
        return t, int(deg[rows].sum()), rows.size

    e_try = min(int(csum[-1]), 200_000)
    t, e, r = run(e_try)
    if t < target_s and e < csum[-1]:
        e_try = min(int(csum[-1]), int(e * target_s / max(t, 1e-3)))
        t, e, r = run(e_try)
    reps, tt = 1, t
    while tt < min(3.0, target_s) and reps < 50:     # whole graph finished fast: repeat it
        t2, _, _ = run(e_try)
        tt += t2
        reps += 1
    t = tt / reps
    cores = 1 if wl.kind == "spmm" else oracle.num_threads()      # scipy's sparse product runs on one thread
    rec = dict(value=round(e / t / 1e9, 6), unit="GEdges/s", cores=cores, kind="oracle", host=host_cpu(),
               sample=f"{r} destination rows drawn uniformly (seed 12345) covering {e} of {int(csum[-1])} edges"
                      + (" (forward + backward, the same nodes as sources)" if wl.backward else " (forward)")
                      + f", {t:.2f} s per pass, mean of {reps}")
    if gpu is not None:
        rec["parity"] = _parity(oracle, wl, last["rows"], last["res"], gpu, op, msg)
    return rec


def bench(args) -> int:
    import numpy as np
    import torch

    import io_aware_sparse_amd as g

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        return 2
    g.lib()
    torch.cuda.set_device(0)
    opts = dict(light_threshold=args.light_threshold, chunk=args.chunk, waves_per_group=args.waves,
                tile_density=args.tile_density, sched_order=args.sched_order)
    log(f"[bench] workload {args.workload}: generating and building the graph")
    wl, indptr, indices, plan, T, E, prep = setup(args.workload, opts, True if args.backward else None, args.reorder,
                                                  args.norm)
    info = g.gnn_plan_export(plan)
    N, H, D = wl.n_nodes, wl.heads, wl.dim
    s = 4 if wl.dtype == "f32" else 2
    log(f"[bench] N={N} E={E} H={H} D={D} dtype={wl.dtype} light={info['n_light']} heavy={info['n_heavy']} "
        f"groups={info['n_groups']} prep={prep}")
    step = make_step(g, wl, indptr, indices, plan, T, args.reduce_op, args.msg)
    stream = torch.cuda.current_stream()
    headline_flushed = args.cache == "flushed"
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for k in range(args.warmup):             # warm up in the headline's cache state
        if headline_flushed:
            flush_buf.fill_(k & 0xFF)
        step()
    torch.cuda.synchronize()

    def timed(flushed):
        """(milliseconds of args.steps steps, per-step milliseconds). Flushed:
        a 512 MiB fill before every step, outside the events; warm: the steps
        back to back (an event between consecutive steps)."""
        if not flushed:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            ev[0].record(stream)
            for k in range(args.steps):
                step()
                ev[k + 1].record(stream)
            torch.cuda.synchronize()
            per = [ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]
            return ev[0].elapsed_time(ev[-1]), per
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
        for k in range(args.steps):
            flush_buf.fill_(k & 0xFF)
            ev[2 * k].record(stream)
            step()
            ev[2 * k + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(args.steps)]
        return sum(per), per

    # The step time comes from a pass without per-kernel events (an event pair
    # around every kernel adds about 15-20 us per step); the per-kernel
    # durations come from the same steps repeated with the library's events on
    # the launch stream.
    wall0 = time.perf_counter()
    ms_total, per_step = timed(headline_flushed)
    wall = time.perf_counter() - wall0
    g.gnn_plan_timing_read(plan)
    g.gnn_plan_set_timing(plan, True)
    ms_inst = timed(headline_flushed)[0] / args.steps
    g.gnn_plan_set_timing(plan, False)
    kt = g.gnn_plan_timing_read(plan)
    ms_other = None if args.no_other_cache else timed(not headline_flushed)[0] / args.steps
    del flush_buf
    replay = graph_replay(g, plan, indptr, indices, T, args.steps, E) \
        if wl.kind == "gt" and not wl.backward and args.reorder == "none" else None
    ms_step = ms_total / args.steps
    value = E / (ms_step * 1e-3) / 1e9

    v_alias = True
    if wl.kind == "spmm":             # the block kernel serves rows of whole 16-feature chunks, <= 256 bytes
        tiled = bool(info["has_tiles"]) and (H * D) % 16 == 0 and H * D * s <= 256
    else:
        tiled = bool(info["has_tiles"]) and wl.dtype == "bf16" and D in (32, 64, 128) and wl.kind == "gt"
    counts = step_counts(g.gnn_plan_export(plan, arrays=True), indptr.cpu().numpy(), indices.cpu().numpy(), tiled)
    counts["msg"] = args.msg
    kernels = {}
    for name, (launches, tot_ms) in kt.items():
        avg_ms = tot_ms / max(1, launches)
        b = kernel_bytes(name, counts, H, D, s, v_alias=v_alias)
        kernels[name] = dict(launches=launches, avg_us=round(1e3 * avg_ms, 3), alg_bytes=b,
                             GBps=round(b / (avg_ms * 1e-3) / 1e9, 1) if avg_ms > 0 else None)
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
    dk = kernels[dom]
    achieved = dk["GBps"]
    import workloads
    tag = profile_tag(args.workload, int(info["n_tiles"]) > 0,
                      wl.backward and not workloads.SPECS[args.workload]["backward"], args.reorder)
    traffic = read_traffic(dom, tag)
    ctx = roofline_context(dom, H, D, s, N, achieved, traffic, dk["avg_us"], v_alias=v_alias)
    for name, k in kernels.items():
        if k["GBps"] and k["GBps"] > HBM_PEAK_GBPS:
            k["note"] = "above 8 TB/s: the per-edge model is not a bound (caches served repeated rows)"
    step_bytes = sum(kernel_bytes(k, counts, H, D, s, v_alias=v_alias) for k in kernels)
    rec = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "GEdges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_ms": {"median": round(float(np.median(per_step)), 5), "min": round(min(per_step), 5),
                    "max": round(max(per_step), 5)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "pass": (f"SpMM aggregation Y = A_w X, {args.norm} weights"
                     + (" + transposed product (gradient)" if wl.backward else "")) if wl.kind == "spmm" else
                    (f"neighbourhood {args.reduce_op} of {args.msg} messages with winners"
                     + (" + gradient" if wl.backward else "")) if wl.kind == "reduce" else
                    ("GATv2" if wl.kind == "gatv2" else "GT") + (" forward + LSE-recompute backward"
                                                                 if wl.backward else " forward"),
            "n_nodes": N, "n_edges": E, "heads": H, "dim": D,
            "storage": wl.dtype, "math": "f32",
            "light_threshold": args.light_threshold, "chunk": args.chunk, "waves_per_group": args.waves,
            "tile_density": args.tile_density, "tiles": int(info["n_tiles"]), "sched_order": args.sched_order,
            "cache": CACHE_TEXT[args.cache], "reorder": args.reorder,
            "parallelism": "single GPU",
        },
        "instrumented": {"ms_per_step": round(ms_inst, 5),
                         "note": "the same steps with a HIP event pair around every kernel, "
                                 "the source of the per-kernel durations"},
        "other_cache": None if ms_other is None else {
            "cache": CACHE_TEXT["warm" if headline_flushed else "flushed"],
            "ms_per_step": round(ms_other, 5), "value": round(E / (ms_other * 1e-3) / 1e9, 4)},
        "graph_replay": replay,
        "step_model_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_model_frac_of_8TBps": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {
            "kernel": dom,
            "bound": ctx.pop("bound"),
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4) if achieved else None,
            "traffic": traffic,
            "traffic_GBps": round(traffic / (dk["avg_us"] * 1e-6) / 1e9, 1) if traffic and dk["avg_us"] else None,
            "traffic_source": f"profiles/{dom}__{tag}__counters.txt" if traffic is not None else None,
            "alg_bytes_per_launch": dk["alg_bytes"],
            "avg_launch_us": dk["avg_us"],
            **ctx,
        },
        "kernels": kernels,
        "kernel_source_sha256": kernel_source_hash(dom),
        "memory": memory_record(g, plan, T, indptr, indices, wl, E),
        "preprocess": prep,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline and args.reorder == "none":
        import oracle
        rp = indptr.cpu().numpy()
        rx = indices.cpu().numpy()
        log(f"[bench] oracle CPU baseline (~{args.cpu_seconds:.0f} s), checked against the measured outputs")
        names = {"spmm": ("Y", "dX"), "reduce": ("out", "arg")}.get(wl.kind, ("O", "LSE", "dQ", "dK", "dV"))
        gpu = {k: (T[k].float() if T[k].dtype == torch.bfloat16 else T[k]).cpu().numpy() for k in names if k in T}
        rec["cpu_baseline"] = cpu_baseline(wl, rp, rx, args.cpu_seconds, op=args.reduce_op, msg=args.msg,
                                           norm=args.norm, gpu=gpu)
        if E <= 10_000_000 and wl.kind != "spmm":
            rec["cpu_baseline_1core"] = cpu_baseline(wl, rp, rx, args.cpu_seconds / 2, threads=1,
                                                     op=args.reduce_op, msg=args.msg)
    print(json.dumps(rec), flush=True)
    return 0


def copy_probe(args) -> int:
    import torch
    nbytes = args.copy_mib << 20
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 3}), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--light-threshold", type=int, default=512)
    ap.add_argument("--chunk", type=int, default=512)
    ap.add_argument("--waves", type=int, default=4)
    ap.add_argument("--sched-order", type=int, default=2, choices=(0, 1, 2),
                    help="light launch order: 0 by id, 1 by descending degree, 2 long rows first")
    ap.add_argument("--reduce-op", choices=("max", "min"), default="max",
                    help="reduction workloads (maxpool_*): max or min")
    ap.add_argument("--msg", choices=("src", "diff"), default="src",
                    help="reduction workloads: message x_j (src) or x_j - x_i (diff)")
    ap.add_argument("--norm", choices=("sum", "mean", "gcn"), default="gcn",
                    help="SpMM workloads (spmm_*): cached weights")
    ap.add_argument("--reorder", choices=("none", "degree", "rcm"), default="none",
                    help="relabel the graph and its feature rows before planning (gnn_reorder)")
    ap.add_argument("--tile-density", type=float, default=0.0,
                    help="16x16 tile threshold tau (0 disables the tile path)")
    ap.add_argument("--cache", choices=("flushed", "warm"), default="flushed",
                    help="cache state of the headline timing: a 512 MiB fill before every step (flushed) or "
                         "steps back to back (warm); the other state is timed after it and reported beside it")
    ap.add_argument("--no-other-cache", action="store_true",
                    help="skip the second timing in the other cache state (profiling runs)")
    ap.add_argument("--backward", action="store_true",
                    help="add the LSE-recompute backward to the step (seeded upstream gradient)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    ap.add_argument("--out", help="summary output file")
    ap.add_argument("--units", metavar="DIR", help="summarise an execution-unit counter pass (UNIT_COUNTERS)")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--kernel", help="kernel kind for --traffic (e.g. gatv2_fwd_main)")
    ap.add_argument("--kernel-regex", default="k_fwd_main", help="symbol pattern for --traffic")
    ap.add_argument("--bench-args", default="--no-cpu-baseline --steps 3 --warmup 1")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args)
    if args.traffic:
        return traffic_summary(args)
    if args.units:
        return units_summary(args)
    if args.copy_probe:
        return copy_probe(args)
    return bench(args)


if __name__ == "__main__":
    sys.exit(main())
