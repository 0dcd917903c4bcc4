"""Host-side logic of bench.py (no GPU): byte counts, copy counts, launch-shape labels, the
rocprofv3 summarisers and the counter lookup, and the one-GPU guard."""
import csv
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_byte_counts_and_copies():
    assert bench.weight_bytes("e4m3", 17408, 5120) == 89_128_960
    assert bench.weight_bytes("q8_0", 17408, 5120) == 94_699_520
    assert bench.grid_bytes("blk128", 17408, 5120) == 21_760
    assert bench.grid_bytes("e4m3", 17408, 5120) == 0
    # weights + grid + q8_1 activation (in_f + in_f/8) + f32 output
    assert bench.algorithmic_bytes("blk128", 17408, 5120, 2) == \
        89_128_960 + 21_760 + 2 * (5120 + 640) + 4 * 2 * 17408
    # rotation sets exceed twice the 256 MiB last-level cache
    for nbytes in (26_214_400, 89_128_960, 94_699_520, 4_194_304):
        c = bench.n_copies(nbytes)
        assert c >= 2 and c * nbytes >= 2 * bench.LLC_BYTES and (c - 1) * nbytes < 2 * bench.LLC_BYTES


def test_launch_labels_are_unique_over_the_step():
    sigs = {}
    for out_f, in_f in bench.SHAPES:
        for arm in bench.ARMS:
            fam, cfg, grid, wg, _ = bench.launch_signature(arm, out_f, in_f)
            key = (fam, cfg, grid, wg)
            assert key not in sigs, (key, sigs.get(key))
            sigs[key] = f"{arm}@{out_f}x{in_f}"
            name = f"void fp8gemv::(anonymous namespace)::{fam}, fp8gemv::{cfg} >(int)"
            assert bench._label_of(name, grid, wg, 0) == f"{arm}@{out_f}x{in_f}"


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_summarize_trace(tmp_path):
    rows = []
    for i, dur in enumerate([1000, 3000, 2000]):
        rows.append({"Kernel_Name": "void fp8gemv::(anonymous namespace)::k_read_bytes(int)",
                     "Grid_Size": "1024", "Workgroup_Size": "256",
                     "Start_Timestamp": str(10_000 * i), "End_Timestamp": str(10_000 * i + dur)})
    p = tmp_path / "trace.csv"
    _write_csv(p, rows)
    out = bench.summarize_trace(str(p))
    line = [l for l in out.splitlines() if "k_read_bytes" in l][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "3"                         # calls
    assert cells[2:6] == ["2.000", "2.000", "1.000", "3.000"]  # avg, median, min, max (us)


def test_summarize_pmc_scales_by_the_calibration_copy(tmp_path):
    known = bench.CALIB_MIB * 1024
    fetch, write = [], []

    def add(i, name, grid, wg, f, w):
        base = {"Dispatch_Id": str(i), "Kernel_Name": name, "Grid_Size": str(grid),
                "Workgroup_Size": str(wg), "LDS_Block_Size": "0"}
        fetch.append({**base, "Counter_Name": "FETCH_SIZE", "Counter_Value": str(f)})
        write.append({**base, "Counter_Name": "WRITE_SIZE", "Counter_Value": str(w)})
    add(1, "__amd_rocclr_copyBuffer", 131072, 512, known / 2, known)  # FETCH reads half
    fam, cfg, grid, wg, _ = bench.launch_signature("q8_0", 5120, 17408)
    add(2, f"void fp8gemv::(anonymous namespace)::{fam}<{cfg} >(int)", grid, wg, 46000.0, 40.0)
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_csv(fp, fetch)
    _write_csv(wp, write)
    out = bench.summarize_pmc(str(fp), str(wp))
    assert "fetch_scale 2.0000" in out and "write_scale 1.0000" in out
    line = [l for l in out.splitlines() if "label=q8_0@5120x17408" in l][0]
    assert int(line.rstrip(" |").split("|")[-1]) == round((46000.0 * 2 + 40.0) * 1024)


def test_traffic_lookup_requires_the_current_source_hash(tmp_path, monkeypatch):
    p = tmp_path / "pmc.md"
    row = "| label=q8_0@5120x17408 | k grid=1 wg=1 | 1 | 1.0 | 1.0 | 123456 |"
    p.write_text(f"source {bench.gemv_source_hash()}\n{row}\n")
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(p))
    assert bench.traffic_for("q8_0@5120x17408") == 123456
    assert bench.traffic_for("e4m3@5120x17408") is None
    p.write_text(f"source 0000000000000000\n{row}\n")
    assert bench.traffic_for("q8_0@5120x17408") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_read_ceiling_fit_recovers_a_line():
    # t = 1.5 us + bytes / 7000 GB/s, sampled at four sizes: the fit must return both exactly.
    pts = [(b, 1.5 + b / 7000e3) for b in (26214400, 89128960, 178257920, 356515840)]
    fit = bench.fit_read_ceiling(pts)
    assert fit["steady_GBs"] == pytest.approx(7000.0, abs=0.05)
    assert fit["fixed_us"] == pytest.approx(1.5, abs=5e-4)
    assert fit["steady_pct_peak"] == pytest.approx(87.5, abs=0.05)
    # fixed cost allowed at 89 MB for 85% of 8 TB/s at a 7 TB/s stream
    b = 89128960
    assert fit["fixed_budget_for_85pct_us"]["89.1MB"] == pytest.approx(
        b / 6800e3 - b / 7000e3, abs=1e-3)
    with pytest.raises(ValueError):
        bench.fit_read_ceiling(pts[:1])
    with pytest.raises(ValueError):
        bench.fit_read_ceiling([pts[0], pts[0]])


def test_summarize_sq_derives_shares_from_counters_and_duration(tmp_path):
    # one dispatch of 10 us at 2.4 GHz = 24000 cycles; 1024 SIMDs
    dur_ns = 10_000
    name = "void fp8gemv::(anonymous namespace)::k_gemv_e4m3<false, Cfg<4> >(int)"
    counters = {
        "SQ_INSTS_VALU": 0.5 * 24000 / 4 * 1024,      # half the SIMD time in VALU
        "SQ_ACTIVE_INST_LDS": 0.1 * 24000 / 4 * 1024,  # a tenth in LDS instructions
        "SQ_WAVE_CYCLES": 0.25 * 24000 / 4 * 256 * 32,  # a quarter of the wave slots
        "SQ_WAIT_INST_LDS": 0.02 * 0.25 * 24000 / 4 * 256 * 32,
        "SQ_WAIT_INST_ANY": 0.3 * 0.25 * 24000 / 4 * 256 * 32,
        "SQ_WAVES": 1000.0, "SQ_INSTS_LDS": 20000.0,
        "SQ_LDS_BANK_CONFLICT": 10.0, "SQ_LDS_IDX_ACTIVE": 110.0,
    }
    rows = [{"Dispatch_Id": "7", "Kernel_Name": name, "Grid_Size": "1024", "Workgroup_Size": "256",
             "Counter_Name": c, "Counter_Value": str(v), "Start_Timestamp": "1000",
             "End_Timestamp": str(1000 + dur_ns)} for c, v in counters.items()]
    p = tmp_path / "sq.csv"
    _write_csv(p, rows)
    out = bench.summarize_sq([str(p)])
    line = [l for l in out.splitlines() if "k_gemv_e4m3" in l and "grid=1024" in l][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1:] == ["10.00", "50.00", "10.00", "25.00", "2.00", "30.00", "3072.00",
                         "20.00", "0.10"]


def test_summarize_mem_request_ratios(tmp_path):
    # One e4m3 17408x5120 launch (87,040 KiB of weights) over two counter passes, and one
    # Q8_0-row read kernel: per-KiB counts, L1->L2 requests per memory request, hit rate and
    # mean latency.
    fam, cfg, grid, wg, _ = bench.launch_signature("e4m3", 17408, 5120)
    gemv = f"void fp8gemv::(anonymous namespace)::{fam}, fp8gemv::{cfg} >(int)"
    read = "void fp8gemv::(anonymous namespace)::k_read_rows<51>(int)"
    kib = 17408 * 5120 / 1024
    passes = [
        {"TCC_REQ_sum": 9 * kib, "TCC_EA0_RDREQ_sum": 8 * kib, "TCC_EA0_RDREQ_32B_sum": 0,
         "TCC_HIT_sum": kib},
        {"TCC_MISS_sum": 9 * kib, "TCP_TCC_READ_REQ_sum": 10 * kib,
         "TCP_TCC_READ_REQ_LATENCY_sum": 10 * kib * 800},
    ]
    paths = []
    for i, counters in enumerate(passes):
        rows = []
        for name, g, dram in ((gemv, grid, None), (read, 1114112, 1000.0)):
            for c, v in counters.items():
                if dram is not None:  # the read kernel: 1000 memory requests, 1130 L1->L2
                    v = {"TCC_EA0_RDREQ_sum": dram, "TCP_TCC_READ_REQ_sum": 1130.0}.get(c, 1.0)
                rows.append({"Dispatch_Id": str(i), "Kernel_Name": name, "Grid_Size": str(g),
                             "Workgroup_Size": str(wg), "LDS_Block_Size": "0",
                             "Counter_Name": c, "Counter_Value": str(v)})
        p = tmp_path / f"pass{i}.csv"
        _write_csv(p, rows)
        paths.append(str(p))
    out = bench.summarize_mem(paths)
    line = [l for l in out.splitlines() if l.startswith("| e4m3@17408x5120 |")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    dram_mb = 8 * kib * 128 / 1e6
    assert cells[2:] == [f"{dram_mb:.2f}", "1.25", "9.00", "8.00", "0.00", "10.00", "10.00",
                         "800.00"]
    read_line = [l for l in out.splitlines() if l.startswith("| read |") and "k_read_rows<51>" in l][0]
    cells = [c.strip() for c in read_line.strip("|").split("|")]
    assert cells[2:4] == ["0.13", "1.13"] and cells[4] == "-"  # no per-KiB figures for reads
