"""Benchmark of one absorbed split-KV MLA decode step on one MI355X.

Default workload: B=32, H=128, q_len=1, L=32768 per sequence, paged latent
cache (block 32, blocks in a seeded random permutation), keys split into 8
contiguous parts of 4096 (decode context parallelism emulated on one GPU),
bf16 partial outputs and LSEs, LSE combine, V-up. One step = q-absorb +
partial attention over all parts + LSE combine + V-up (the last two as one
fused launch for bf16 / fp16), inputs resident in HBM. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode µs/step, TFLOP/s & KV GB/s (% roofline) at B=32 H=128 L=32K"
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20   # MI355X Infinity Cache
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
KERNEL_SRCS = [os.path.join(ROOT, "mla_split_kv_absorbed_amd", "csrc", f)
               for f in ("partial_mfma.hip", "common.h", "kernels.h", "plan.h", "short.h")]
PMC_FILE = os.path.join(ROOT, "profiles", "partial_mfma_kernel_pmc.json")
# how the timed decode step is built (the full-size parity tests build theirs
# the same way): a single part's sub-ranges are cut on the host and merged by
# the fused combine + V-up; a ragged batch's split plan is built on the host
# with the other metadata (before the timed region, as the ranges are); the
# MTP workload's current chunk runs in the history call's launch
# (mla_decode_partial_pair: its workgroups fill the end of the history's
# schedule)
BENCH_STEP_OPTS = {"host_subranges": True, "host_plan": True, "pair_current": True}


def kernel_hash(srcs=None) -> str:
    """Hash of the partial kernel's code: its source and the headers it
    includes, with // comments, blank lines and indentation dropped (a
    comment edit does not invalidate counters taken on the same code)."""
    h = hashlib.sha256()
    for path in srcs or KERNEL_SRCS:
        with open(path) as f:
            for line in f:
                code = re.sub(r"//.*", "", line).strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch of the partial kernel from committed rocprofv3
    counter runs, if they were taken on the current kernel source."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_sha") != kernel_hash() or d.get("workload") != workload:
        return None
    return d.get("hbm_bytes_per_launch")


PMC_GRID = 65536  # grid of the 8-part decode-step launch of the 32K workload


def _pmc_rows(run_dir: str, counter: str):
    import csv
    path = os.path.join(run_dir, "run_counter_collection.csv")
    with open(path) as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]


def _step_launches(rows):
    """The partial kernel's decode-step (all parts) launches among profiled
    rows: partial_mfma_kernel dispatches that take at least half as long as
    the longest one. The one-part calls that bench.py times afterwards can
    have the same grid but take a fraction of the time."""
    rows = [r for r in rows if "partial_mfma_kernel" in r["Kernel_Name"]]
    dur = lambda r: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])  # noqa: E731
    if not rows:
        return rows
    longest = max(dur(r) for r in rows)
    return [r for r in rows if 2 * dur(r) >= longest]


def pmc_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, commands):
    """HBM traffic per launch of the partial kernel from two rocprofv3 --pmc
    runs of the decode step (FETCH_SIZE, then WRITE_SIZE, in KiB per
    dispatch), each scaled by what the same counter reads for a plain device
    copy of known size (the copy probe)."""
    def kern_mean(d, c):
        v = [float(r["Counter_Value"]) for r in _step_launches(_pmc_rows(d, c))
             if int(r["Grid_Size"]) == PMC_GRID]
        if not v:
            raise SystemExit(f"no partial_mfma_kernel decode-step dispatch of grid {PMC_GRID} in {d}")
        return sum(v) / len(v), len(v)

    def copy_mean(d, c):
        rows = [r for r in _pmc_rows(d, c) if "copy" in r["Kernel_Name"].lower()]
        big = max(int(r["Grid_Size"]) for r in rows)
        v = [float(r["Counter_Value"]) for r in rows if int(r["Grid_Size"]) == big]
        return sum(v) / len(v)

    fetch, nf = kern_mean(fetch_dir, "FETCH_SIZE")
    write, nw = kern_mean(write_dir, "WRITE_SIZE")
    n_copy = 2 * 256 * 1024 * 1024  # bytes read and written by the copy probe
    cf, cw = copy_mean(copy_fetch_dir, "FETCH_SIZE"), copy_mean(copy_write_dir, "WRITE_SIZE")
    ff, wf = n_copy / (cf * 1024), n_copy / (cw * 1024)
    rd, wr = fetch * 1024 * ff, write * 1024 * wf
    return {
        "kernel": "partial_mfma_kernel<bf16>",
        "workload": "config2:bf16_B32_H128_L32768_paged32_8parts",
        "kernel_sha": kernel_hash(),
        "kernel_sha_of": "bench.kernel_hash(): partial_mfma.hip, common.h, kernels.h, plan.h "
                         "and short.h with comments and blank lines dropped",
        "fetch_kib_per_dispatch": round(fetch, 3),
        "write_kib_per_dispatch": round(write, 3),
        "dispatches": {"fetch": nf, "write": nw},
        "copy_probe": {"bytes_read": n_copy, "bytes_written": n_copy,
                       "fetch_kib": round(cf, 3), "write_kib": round(cw, 3)},
        "fetch_factor": round(ff, 4),
        "write_factor": round(wf, 4),
        "hbm_read_bytes_per_launch": int(rd),
        "hbm_write_bytes_per_launch": int(wr),
        "hbm_bytes_per_launch": int(rd + wr),
        "commands": commands,
        "note": f"partial_mfma_kernel decode-step dispatches (grid {PMC_GRID}, the 8-part launch; "
                "the shorter one-part calls are excluded) only; the copy probe is the device copy "
                "of 512 MiB",
    }


SQ_PASSES = (
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_LDS "
    "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE",
    "SQ_INSTS_VALU_MFMA_BF16 SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY "
    "SQ_WAIT_INST_ANY SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_LDS SQ_INSTS_SALU GRBM_GUI_ACTIVE",
)


def sq_summary(dirs, last: int = 0):
    """Matrix-core and LDS counters of the partial kernel's decode-step launch
    (the all-parts history call: the longest partial_mfma_kernel dispatches),
    from rocprofv3 --pmc runs of the SQ_PASSES counter sets, as markdown.
    last > 0: only the last `last` such launches of each run (the steady
    state after a settle phase)."""
    import csv
    vals, durs = {}, []
    for d in dirs:
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            rows = _step_launches(list(csv.DictReader(f)))
        if last > 0:
            ids = sorted({int(r["Dispatch_Id"]) for r in rows})[-last:]
            keep = set(ids)
            rows = [r for r in rows if int(r["Dispatch_Id"]) in keep]
        if not rows:
            raise SystemExit(f"no partial_mfma_kernel dispatch in {d}")
        grid = int(rows[0]["Grid_Size"])
        per = {}
        for r in rows:
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
        for c, v in per.items():
            vals.setdefault(c, sum(v) / len(v))
    us = sum(durs) / len(durs)
    simds, xcds = 256 * 4, 8
    waves = grid // 64
    clk = vals["GRBM_GUI_ACTIVE"] / xcds / us * 1e-3  # GHz; the counter sums the 8 XCDs
    kcyc = vals["GRBM_GUI_ACTIVE"] / xcds
    mfma_busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
    flops = vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    lines = [
        "| counter | per launch |", "|---|---:|"] + [
        f"| `{c}` | {v:,.0f} |" for c, v in sorted(vals.items())] + [
        "", "| derived | value |", "|---|---:|",
        f"| launch profiled | grid {grid} threads ({waves} waves) |",
        f"| kernel duration (mean over the profiled launches) | {us:.1f} us |",
        f"| core clock (GRBM_GUI_ACTIVE / 8 XCDs / duration) | {clk:.2f} GHz |",
        f"| matrix-core busy cycles per SIMD (SQ_VALU_MFMA_BUSY_CYCLES / 1024) | {mfma_busy:,.0f} |",
        f"| matrix-core busy fraction (/ kernel cycles {kcyc:,.0f}) | {mfma_busy / kcyc:.3f} |",
        f"| bf16 matrix FLOPs (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) | {flops / 1e9:.1f} GFLOP |",
        f"| matrix rate | {flops / (us * 1e-6) / 1e12:.0f} TFLOP/s = "
        f"{flops / (us * 1e-6) / 2.5e15:.3f} of 2.5 PFLOP/s, "
        f"{flops / (us * 1e-6) / (2.5e15 * clk / 2.4):.3f} of the peak at {clk:.2f} GHz |",
        f"| cycles per matrix instruction issued (busy / count per SIMD) | "
        f"{mfma_busy / (vals['SQ_INSTS_VALU_MFMA_BF16'] / simds):.1f} |",
        f"| LDS instructions per wave | {vals['SQ_INSTS_LDS'] / waves:,.0f} |",
        f"| LDS bank-conflict cycles per wave (SQ_LDS_BANK_CONFLICT / {waves} waves) | "
        f"{vals['SQ_LDS_BANK_CONFLICT'] / waves:,.0f} |",
        f"| wave cycles waiting on a counter (SQ_WAIT_ANY / SQ_WAVE_CYCLES) | "
        f"{vals['SQ_WAIT_ANY'] / vals['SQ_WAVE_CYCLES']:.3f} |",
    ]
    return "\n".join(lines) + "\n"


def cpu_baseline(w, budget_s: float = 15.0):
    """The float64 oracle on a bounded sample of (sequence, head) pairs of the
    same workload, scaled to microseconds per full step."""
    import oracle.mla_oracle as mo
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    sp = w.spec
    qn, qr = w.f64("q_nope"), w.f64("q_rope")
    wuk, wuv = w.f64("w_uk"), w.f64("w_uv")
    cur = (lambda b: w.cur_rows64(b)) if sp.current else None
    r = np.random.Generator(np.random.PCG64(11))
    pairs = [(int(b), int(h)) for b, h in zip(r.integers(0, sp.B, 10_000),
                                               r.integers(0, sp.H, 10_000))]
    done, keys = 0, 0
    rows_cache = {}
    t0 = time.perf_counter()
    for b, h in pairs:
        if b not in rows_cache:
            rows_cache.clear()
            rows_cache[b] = w.seq_rows64(b)
        mo.mla_decode_step(qn, qr, lambda bb: rows_cache[bb], wuk, wuv, sp.scale, sp.S,
                           cur_rows=cur, seqs=[b], heads=[h])
        done += 1
        keys += int(w.lengths[b])
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    total_pairs = sp.B * sp.H
    us_step = el / done * total_pairs * 1e6
    return {"value": round(us_step, 1), "unit": "us/step", "cores": int(threads),
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{done} of {total_pairs} (sequence, head) pairs of the same workload "
                      f"(float64, per-head K/V materialised), {el:.1f} s, scaled by "
                      f"{total_pairs}/{done}"}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def spread(xs):
    """Median, 10th and 90th percentile of a list of durations (us)."""
    q = np.percentile(np.asarray(xs, np.float64), [50, 10, 90])
    return {"median": round(float(q[0]), 2), "p10": round(float(q[1]), 2),
            "p90": round(float(q[2]), 2), "n": len(xs)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    # The card's power management needs tens of milliseconds of sustained
    # load to settle: on a cold start the first few launches run boosted,
    # the next ~150 (about 50 ms) run 20-40% slower while the clock is
    # pulled back, then the steady state holds. After the warm-up, steps
    # run for this much device time before the timed region; the JSON line
    # reports the phase (its length and the first and last steps' times).
    ap.add_argument("--settle-ms", type=float, default=150.0)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--copies", type=int, default=0,
                    help="independent KV caches rotated over the steps (0 = enough to exceed "
                         "twice the 256 MB Infinity Cache when one cache is smaller)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of 512 MiB three times (the "
                         "calibration kernel for the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--peaks", action="store_true",
                    help="only run the device peak microbenchmarks (HBM read and copy, bf16 "
                         "matrix cores, LDS reads) and print them beside the published peaks")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                                                       "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the partial kernel's HBM traffic file from four rocprofv3 "
                         "--pmc output directories (no GPU needed)")
    ap.add_argument("--sq-last", type=int, default=0,
                    help="with --sq-summary: only the last N decode-step launches of each run")
    ap.add_argument("--sq-summary", nargs=2, metavar=("PASS1_DIR", "PASS2_DIR"),
                    help="print the partial kernel's matrix-core and LDS counters (two rocprofv3 "
                         "--pmc runs of the SQ_PASSES sets) as markdown (no GPU needed)")
    args = ap.parse_args()
    if args.sq_summary:
        print(sq_summary(args.sq_summary, args.sq_last), end="", flush=True)
        return
    if args.pmc_summary:
        dirs = args.pmc_summary
        # the commands name the output folders relative to the repository
        rel = [os.path.relpath(os.path.abspath(d), ROOT)
               if os.path.abspath(d).startswith(ROOT + os.sep) else d for d in dirs]
        cmds = [f"rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- python3 bench.py "
                + ("--copy-probe" if i >= 2 else "--steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline")
                for i, (c, d) in enumerate(zip(("FETCH_SIZE", "WRITE_SIZE") * 2, rel))]
        res = pmc_summary(*dirs, cmds)
        with open(PMC_FILE, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")
        print(json.dumps(res), flush=True)
        return
    if args.peaks:
        from mla_split_kv_absorbed_amd import build as B
        if not os.path.exists(B.PEAKS_BIN):
            print(f"bench.py: {B.PEAKS_BIN} is not built", file=sys.stderr)
            sys.exit(1)
        import subprocess
        r = subprocess.run([B.PEAKS_BIN], stdout=subprocess.PIPE, text=True)
        if r.returncode != 0:
            sys.exit(r.returncode)
        meas = json.loads(r.stdout.strip().splitlines()[-1])
        print(json.dumps({"measured": meas,
                          "published": {"hbm_gbs": HBM_PEAK_GBS,
                                        "mfma_bf16_tflops": MFMA_PEAK_TFLOPS["bf16"],
                                        "clock_ghz": 2.4, "compute_units": 256}}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the DCP parts are processed on the one device", file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_split_kv_absorbed_amd import _lib as L
    from mla_split_kv_absorbed_amd import workloads as W
    from mla_split_kv_absorbed_amd.step import DecodeStep

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        n = 256 * 1024 * 1024
        x = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 2 * n, "copy_probe_bytes_written": 2 * n,
                          "launches": 3}), flush=True)
        return
    L.lib()  # fail loudly if the HIP library is missing
    sp = W.SPECS[args.workload]
    print(f"[bench] generating workload {sp.name}", file=sys.stderr, flush=True)
    w = W.make_workload(sp)
    work = W.step_work(w)
    # Cold-cache discipline: a cache smaller than twice the 256 MB Infinity
    # Cache (MALL) would stay resident across steps, so enough independent
    # copies are rotated that the steps touch more than 512 MB in turn.
    kv_bytes = w.kv.nbytes
    copies = args.copies or (1 if kv_bytes >= MALL_BYTES * 2 or kv_bytes < 16 << 20
                             else -(-(2 * MALL_BYTES) // kv_bytes) + 1)
    sts = [DecodeStep(w, device="cuda:0", **BENCH_STEP_OPTS) for _ in range(copies)]
    st = sts[0]
    stream = torch.cuda.current_stream()

    # one DCP rank's share: each part alone, a single-part call per part
    def share_args(p):
        # the workload's own range of part p (the step's device ranges may be
        # its host-cut sub-ranges)
        rs = torch.from_numpy(np.ascontiguousarray(w.range_start[p:p + 1])).to("cuda:0")
        re_ = torch.from_numpy(np.ascontiguousarray(w.range_end[p:p + 1])).to("cuda:0")
        a = L.partial_args(st.q_lat, st.q_rope, st.kv, rs, re_, st.parts_out[p:p + 1],
                           st.parts_lse[p:p + 1], B=sp.B, S=sp.S, H=sp.H, scale=sp.scale,
                           **({"block_table": st.block_table, "block_size": sp.block_size,
                               "num_blocks": w.kv.shape[0]} if sp.block_size else
                              {"kv_seq_stride": w.kv.shape[1]}))
        # equal ranges: the automatic plan's chunk count, passed explicitly
        a.num_splits = L.mla_decode_partial_plan(a, w.range_start[p:p + 1],
                                                 w.range_end[p:p + 1]).equal_splits
        ws_ = torch.empty(max(1, L.mla_decode_partial_workspace_size(a)), dtype=torch.uint8,
                          device="cuda:0")
        a.workspace, a.workspace_bytes = ws_.data_ptr(), ws_.numel()
        return a, (ws_, rs, re_)  # kept alive with the arguments
    shares = [share_args(p) for p in range(sp.parts)]

    print(f"[bench] warmup ({copies} cache cop{'y' if copies == 1 else 'ies'})",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        sts[i % copies].run(stream)
    torch.cuda.synchronize()

    # settle phase: whole steps, in batches of 10 with an event between
    # consecutive steps, until the device has run settle_ms of them
    print(f"[bench] settle ({args.settle_ms:.0f} ms of steps)", file=sys.stderr, flush=True)
    settle_us, n_settle = [], 0
    while sum(settle_us) < args.settle_ms * 1e3:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(11)]
        evs[0].record(stream)
        for k in range(10):
            sts[(n_settle + k) % copies].run(stream)
            evs[k + 1].record(stream)
        torch.cuda.synchronize()
        settle_us += [evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(10)]
        n_settle += 10

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    # one decode step on cache copy i % copies, the partial call bracketed by
    # the events ev[i]
    def one_step(i):
        st = sts[i % copies]
        if st.absorb:
            L.mla_q_absorb(st.q_nope, st.w_uk, st.q_lat, stream)
        ev[i][0].record(stream)
        if st.pair:
            L.mla_decode_partial_pair(st.hist_args, st.cur_args, stream)
        else:
            L.mla_decode_partial(st.hist_args, stream)
        ev[i][1].record(stream)
        if sp.current and not st.pair:
            L.mla_decode_partial(st.cur_args, stream)
        if st.fused_tail:
            L.mla_combine_vup(st.parts_out, st.parts_lse, st.w_uv, st.out, st.lse,
                              local_out=st.cur_out if sp.current else None,
                              local_lse=st.cur_lse if sp.current else None, stream=stream)
        else:
            if st.skip_combine:
                x = st.parts_out[0]
            else:
                L.mla_lse_combine(st.parts_out, st.parts_lse, st.lat, st.lse,
                                  local_out=st.cur_out if sp.current else None,
                                  local_lse=st.cur_lse if sp.current else None, stream=stream)
                x = st.lat
            L.mla_vup(x, st.w_uv, st.out, stream)

    print("[bench] timing", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_start.record(stream)
    for i in range(args.steps):
        one_step(i)
    e_end.record(stream)
    enqueue_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e_start.elapsed_time(e_end) / args.steps
    part_launch = [a.elapsed_time(b) * 1e3 for a, b in ev]
    part_ms = float(np.mean(part_launch)) * 1e-3

    # the spread of single steps, from a second pass with an event between
    # consecutive steps (outside the timed region: the events are the only
    # difference)
    sev_step = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    sev_step[0].record(stream)
    for i in range(args.steps):
        one_step(i)
        sev_step[i + 1].record(stream)
    torch.cuda.synchronize()
    step_us = [sev_step[i].elapsed_time(sev_step[i + 1]) * 1e3 for i in range(args.steps)]

    # each rank's share timed alone, the parts called in turn (each call
    # meets its part's keys cold: the other parts' keys came in between)
    rounds = max(10, args.steps // sp.parts)
    for _ in range(3):
        for a, _ws in shares:
            L.mla_decode_partial(a, stream)
    sev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(rounds)] for _ in shares]
    for r in range(rounds):
        for p, (a, _ws) in enumerate(shares):
            sev[p][r][0].record(stream)
            L.mla_decode_partial(a, stream)
            sev[p][r][1].record(stream)
    torch.cuda.synchronize()
    share_per_part = [float(np.mean([e0.elapsed_time(e1) for e0, e1 in sev[p]])) * 1e3
                      for p in range(len(shares))]
    share_us = float(np.mean(share_per_part))
    st = sts[0]

    us = ms_step * 1e3
    tflops = work["total_flops"] / (us * 1e-6) / 1e12
    kv_gbs = work["kv_bytes"] / (us * 1e-6) / 1e9
    t_roof = max(work["total_bytes"] / (HBM_PEAK_GBS * 1e9),
                 work["total_flops"] / (MFMA_PEAK_TFLOPS[sp.dtype] * 1e12))
    bound_step = ("hbm" if work["total_bytes"] / (HBM_PEAK_GBS * 1e9) >=
                  work["total_flops"] / (MFMA_PEAK_TFLOPS[sp.dtype] * 1e12) else "mfma")
    part_bytes = work["partial_bytes"]
    # the partial kernel's own bound: bytes at the HBM peak or matrix work at
    # the MFMA peak, whichever takes longer
    part_mfma = work["attn_flops"] / (MFMA_PEAK_TFLOPS[sp.dtype] * 1e12) > part_bytes / (
        HBM_PEAK_GBS * 1e9)
    if part_mfma:
        achieved, peak, unit = work["attn_flops"] / (part_ms * 1e-3) / 1e12, \
            MFMA_PEAK_TFLOPS[sp.dtype], "TFLOP/s"
    else:
        achieved, peak, unit = part_bytes / (part_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    wl = f"config{sp.wid}:{sp.name}"
    traffic = traffic_from_profile(wl)
    res = {
        "metric": METRIC,
        "value": round(us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sp.dtype,
        "data": "synthetic (seeded; DeepSeek-shaped MLA: d_c=512, d_R=64, random weights)",
        "config": {"workload": wl, "B": sp.B, "H": sp.H, "q_len": sp.S,
                   "L": list(sp.lengths), "block_size": sp.block_size, "parts": sp.parts,
                   "part_out_dtype": sp.part_out_dtype, "part_lse_dtype": sp.part_lse_dtype},
        "tflops": round(tflops, 2),
        "kv_gbs": round(kv_gbs, 1),
        "step_roofline": {"bound": bound_step, "t_roof_us": round(t_roof * 1e6, 2),
                          "frac": round(t_roof * 1e6 / us, 4),
                          "algorithmic_bytes": work["total_bytes"],
                          "algorithmic_flops": work["total_flops"]},
        "roofline": {"kernel": ("partial_mfma_kernel (mla_decode_partial_pair: all history "
                                "parts + the current chunk)" if st.pair else
                                "partial_mfma_kernel (mla_decode_partial, all parts)"),
                     "bound": "mfma" if part_mfma else "hbm", "achieved": round(achieved, 1),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic, "bytes_per_launch": part_bytes,
                     "avg_launch_us": round(part_ms * 1e3, 2),
                     "mfma_tflops": round(work["attn_flops"] / (part_ms * 1e-3) / 1e12, 1)},
        "step_us_spread": spread(step_us),
        "partial_launch_us_spread": spread(part_launch),
        "one_rank_share_us": round(share_us, 2),
        "one_rank_share_per_part_us": [round(x, 2) for x in share_per_part],
        "kv_cache_copies": copies,
        "settle": {"steps": n_settle, "ms": round(sum(settle_us) * 1e-3, 2),
                   "first_10_steps_us": round(float(np.mean(settle_us[:10])), 2),
                   "last_10_steps_us": round(float(np.mean(settle_us[-10:])), 2),
                   "note": "untimed steps between the warm-up and the timed region, run until "
                           "the card's clock has settled under sustained load"},
        "wall_s": round(wall, 3),
        "host_enqueue_s": round(enqueue_s, 4),
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
