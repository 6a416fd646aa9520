"""Host logic of the measurement tools in bench.py (no GPU): the HBM-traffic
summary and the matrix-core / LDS counter summary computed from rocprofv3
counter-collection CSV files, on small synthetic files of the same format."""
import csv
import os

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]
PARTIAL = "_ZN3mla19partial_mfma_kernelIDF16bEEvNS_10MfmaParamsE"
COPY = "__amd_rocclr_copyBuffer"


def write_run(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, grid, counter, value, dur_ns) in enumerate(rows):
            r = {k: 0 for k in FIELDS}
            r.update(Dispatch_Id=i + 1, Grid_Size=grid, Kernel_Name=kernel, Counter_Name=counter,
                     Counter_Value=value, Start_Timestamp=1000, End_Timestamp=1000 + dur_ns)
            w.writerow(r)


def test_pmc_summary_scales_by_the_copy_probe(tmp_path):
    n_copy = 2 * 256 * 1024 * 1024
    # the copy probe reads half its bytes in FETCH_SIZE units (factor 2), writes all (factor 1)
    write_run(tmp_path / "cf", [(COPY, 1 << 20, "FETCH_SIZE", n_copy / 2048, 10)] * 3)
    write_run(tmp_path / "cw", [(COPY, 1 << 20, "WRITE_SIZE", n_copy / 1024, 10)] * 3)
    # two decode-step launches (the counted grid), one one-part launch of another
    # grid and one of the same grid but a quarter of the duration (both ignored)
    write_run(tmp_path / "kf", [(PARTIAL, bench.PMC_GRID, "FETCH_SIZE", 500.0, 100),
                                (PARTIAL, bench.PMC_GRID, "FETCH_SIZE", 700.0, 100),
                                (PARTIAL, 73984, "FETCH_SIZE", 1e9, 10),
                                (PARTIAL, bench.PMC_GRID, "FETCH_SIZE", 1e9, 25)])
    write_run(tmp_path / "kw", [(PARTIAL, bench.PMC_GRID, "WRITE_SIZE", 40.0, 10)])
    res = bench.pmc_summary(str(tmp_path / "kf"), str(tmp_path / "kw"), str(tmp_path / "cf"),
                            str(tmp_path / "cw"), ["cmd"])
    assert res["fetch_factor"] == pytest.approx(2.0)
    assert res["write_factor"] == pytest.approx(1.0)
    assert res["fetch_kib_per_dispatch"] == pytest.approx(600.0)
    assert res["dispatches"] == {"fetch": 2, "write": 1}
    assert res["hbm_read_bytes_per_launch"] == int(600.0 * 1024 * 2.0)
    assert res["hbm_write_bytes_per_launch"] == int(40.0 * 1024)
    assert res["hbm_bytes_per_launch"] == int(600.0 * 1024 * 2.0) + int(40.0 * 1024)
    assert res["kernel_sha"] == bench.kernel_hash()


def test_pmc_summary_needs_the_decode_step_launch(tmp_path):
    write_run(tmp_path / "k", [(PARTIAL, 73984, "FETCH_SIZE", 1.0, 10)])
    write_run(tmp_path / "c", [(COPY, 512, "FETCH_SIZE", 1.0, 10)])
    with pytest.raises(SystemExit):
        bench.pmc_summary(str(tmp_path / "k"), str(tmp_path / "k"), str(tmp_path / "c"),
                          str(tmp_path / "c"), [])


def test_sq_summary_derived_figures(tmp_path):
    dur_ns = 250_000  # 250 us
    clk_ghz = 2.0
    kcyc = dur_ns * 1e-3 * clk_ghz * 1e3  # kernel cycles
    v1 = {"GRBM_GUI_ACTIVE": kcyc * 8, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * kcyc * 1024,
          "SQ_INSTS_VALU_MFMA_MOPS_BF16": 292e9 / 512, "SQ_INSTS_LDS": 1024 * 100.0,
          "SQ_LDS_BANK_CONFLICT": 1024 * 128 * 3.0, "SQ_WAIT_ANY": 25.0, "SQ_WAVE_CYCLES": 100.0,
          "SQ_BUSY_CYCLES": 1.0, "SQ_WAIT_INST_LDS": 1.0}
    v2 = {"GRBM_GUI_ACTIVE": kcyc * 8, "SQ_INSTS_VALU_MFMA_BF16": 0.5 * kcyc * 1024 / 32.0,
          "SQ_ACTIVE_INST_LDS": 1.0, "SQ_INSTS_VALU": 1.0, "SQ_ACTIVE_INST_VALU": 1.0,
          "SQ_ACTIVE_INST_ANY": 1.0, "SQ_WAIT_INST_ANY": 1.0, "SQ_LDS_IDX_ACTIVE": 1.0,
          "SQ_INSTS_SALU": 1.0}
    # shorter launches (one-part calls, of another grid or the same one) are not summarised
    write_run(tmp_path / "p1", [(PARTIAL, bench.PMC_GRID, c, v, dur_ns) for c, v in v1.items()]
              + [(PARTIAL, 73984, c, 1.0, dur_ns // 4) for c in v1]
              + [(PARTIAL, bench.PMC_GRID, c, 1.0, dur_ns // 4) for c in v1])
    write_run(tmp_path / "p2", [(PARTIAL, bench.PMC_GRID, c, v, dur_ns) for c, v in v2.items()])
    md = bench.sq_summary([str(tmp_path / "p1"), str(tmp_path / "p2")])
    rows = dict(line.strip("|").split("|", 1) for line in md.splitlines()
                if line.startswith("| ") and "---" not in line)
    rows = {k.strip(): v.strip() for k, v in rows.items()}

    def find(prefix):
        return next(v for k, v in rows.items() if k.startswith(prefix))

    assert find("kernel duration") == "250.0 us"
    assert find("core clock") == "2.00 GHz"
    assert find("matrix-core busy fraction") == "0.500"
    assert find("bf16 matrix FLOPs") == "292.0 GFLOP"
    assert find("cycles per matrix instruction") == "32.0"
    assert find("LDS instructions per wave") == "100"
    assert find("LDS bank-conflict cycles per wave") == "384"
    assert find("launch profiled") == f"grid {bench.PMC_GRID} threads (1024 waves)"
    assert find("wave cycles waiting") == "0.250"
    # every counter of both passes is listed
    for c in list(v1) + list(v2):
        assert f"`{c}`" in md


def test_sq_passes_fit_one_run_each():
    """Each counter pass stays within one rocprofv3 run's limits (8 SQ_, 2 GRBM_)."""
    for p in bench.SQ_PASSES:
        names = p.split()
        assert sum(n.startswith("SQ_") for n in names) <= 8
        assert sum(n.startswith("GRBM_") for n in names) <= 2
        assert len(set(names)) == len(names)


def test_spread_percentiles():
    """Median and 10th / 90th percentiles of step durations (linear interpolation)."""
    xs = [float(v) for v in range(1, 102)]  # 1 .. 101
    r = bench.spread(xs[::-1])
    assert r == {"median": 51.0, "p10": 11.0, "p90": 91.0, "n": 101}

