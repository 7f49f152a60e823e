"""bench.py's command line without a GPU: a run for more than one GPU is
refused with a message and a nonzero status, before anything touches a
device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_profile_parsing_scales_counters_by_the_copy_calibration(tmp_path):
    """The counters of the child runs are turned into bytes with the factor
    the calibration copies give (known bytes / counted bytes), per dispatch
    of the scan kernel; trace durations average the last dispatches."""
    sys.path.insert(0, ROOT)
    import bench
    scan, pack = bench.KERNEL_NAME, bench.PACK_KERNEL_NAME
    gib_kib = bench.CALIB_BYTES / 1024
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # FETCH_SIZE counts half of the bytes a copy reads, WRITE_SIZE all of them
    fetch = [[1, pack, "FETCH_SIZE", 1000.0], [2, scan, "FETCH_SIZE", 500000.0],
             [3, "void " + scan, "FETCH_SIZE", 502000.0],
             [4, "__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2] ,
             [5, "__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2],
             [6, "__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2]]
    write = [[1, pack, "WRITE_SIZE", 2048.0], [2, scan, "WRITE_SIZE", 330000.0],
             [3, scan, "WRITE_SIZE", 330000.0]] + \
            [[4 + i, "__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib] for i in range(3)]
    _write_csv(str(tmp_path / "fetch" / "host" / "fetch_counter_collection.csv"), hdr, fetch)
    _write_csv(str(tmp_path / "write" / "write_counter_collection.csv"), hdr, write)
    trace = [[scan, 1000 * i, 1000 * i + (900 if i < 2 else 600)] for i in range(6)]
    _write_csv(str(tmp_path / "trace" / "trace_kernel_trace.csv"),
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    dirs = {k: str(tmp_path / k) for k in ("fetch", "write", "trace")}
    calib, kernels, err = bench.parse_profile_dirs(dirs, steps=4)
    assert err is None
    assert abs(calib["FETCH_SIZE"]["scale"] - 2.0) < 1e-9 and abs(calib["WRITE_SIZE"]["scale"] - 1.0) < 1e-9
    k = kernels[scan]
    assert k["read_bytes"] == round(501000.0 * 1024 * 2)
    assert k["write_bytes"] == round(330000.0 * 1024)
    assert k["hbm_bytes_per_launch"] == k["read_bytes"] + k["write_bytes"]
    assert k["trace_avg_ns"] == 600.0 and k["trace_dispatches_averaged"] == 4
    assert kernels[pack]["read_bytes"] == round(1000.0 * 1024 * 2)


def test_profile_parsing_reports_a_missing_calibration(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    _write_csv(str(tmp_path / "fetch" / "f_counter_collection.csv"),
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
               [[1, bench.KERNEL_NAME, "FETCH_SIZE", 5.0]])
    calib, kernels, err = bench.parse_profile_dirs({"fetch": str(tmp_path / "fetch")}, steps=2)
    assert "calibration" in err and calib == {} and kernels == {}


def test_profile_parsing_reads_the_valu_counters(tmp_path):
    """The VALU pass gives each counter's mean per dispatch of the scan
    kernel; a pass without the scan kernel's rows is reported."""
    sys.path.insert(0, ROOT)
    import bench
    scan = bench.KERNEL_NAME
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    for d, (waves, insts, active) in enumerate([(5120, 2.9e8, 3.4e8), (5120, 3.1e8, 3.6e8)]):
        rows += [[d, scan, "SQ_WAVES", waves], [d, scan, "SQ_INSTS_VALU", insts],
                 [d, scan, "SQ_ACTIVE_INST_VALU", active]]
    rows += [[9, bench.PACK_KERNEL_NAME, "SQ_INSTS_VALU", 5.0]]
    _write_csv(str(tmp_path / "valu" / "v_counter_collection.csv"), hdr, rows)
    calib, kernels, err = bench.parse_profile_dirs({"valu": str(tmp_path / "valu")}, steps=2)
    assert err is None
    assert kernels[scan]["valu_counters"] == {"SQ_WAVES": 5120, "SQ_INSTS_VALU": 300000000,
                                              "SQ_ACTIVE_INST_VALU": 350000000}
    _write_csv(str(tmp_path / "valu2" / "v_counter_collection.csv"), hdr, rows[-1:])
    _, _, err = bench.parse_profile_dirs({"valu": str(tmp_path / "valu2")}, steps=2)
    assert err is not None and "VALU" in err
