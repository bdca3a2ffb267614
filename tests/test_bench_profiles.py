"""Host logic of bench.py's rocprofv3 summaries (no GPU): dispatches are cut at
the markers that bracket the timed steps, trace and counter dispatches are paired
by their ordinal within (kernel, grid, workgroup), 2-D grids compare by their
total size, implausible pairs (over 8 TB/s) are dropped, the counters are scaled
by the plain copy's, and per-step / per-call traffic follows the launch counts."""
import csv
import json
import os

import bench

SPIN = "at::cuda::(anonymous namespace)::spin_kernel(long)"
IDX = "void csa::(anonymous namespace)::idx_topk_kernel<2, 8>(csa::IndexArgs, csa::IndexPlan, long)"
APP = "void csa::(anonymous namespace)::compress_kernel<unsigned short, 1, true, false>(unsigned short const*)"
CMP = "void csa::(anonymous namespace)::compress_kernel<unsigned short, 1, false, true>(unsigned short const*)"
COPY = "__amd_rocclr_copyBuffer"


def write_trace(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X",
                    "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"])
        for i, (name, us, gx, gy) in enumerate(rows, start=1):
            w.writerow([i, name, 1000 * i * 100, 1000 * i * 100 + int(us * 1000), 256, 1, 1, gx, gy, 1])


def write_counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"])
        for i, (name, grid, kib) in enumerate(rows, start=1):
            if kib is None:
                continue
            # two rows per dispatch (per-XCD partial sums), which the summary adds up
            w.writerow([i, name, grid, 256, counter, kib / 2])
            w.writerow([i, name, grid, 256, counter, kib / 2])


def make_run(root, idx_kib=(70000.0, 70000.0), idx_us=(28.0, 30.0)):
    # setup launch, marker, two timed steps (index + 2-D append), end marker, a late launch
    trace = [(IDX, 50.0, 131072, 1), (SPIN, 1.0, 1, 1),
             (IDX, idx_us[0], 131072, 1), (APP, 6.0, 512, 4),
             (IDX, idx_us[1], 131072, 1), (APP, 6.0, 512, 4),
             (SPIN, 1.0, 1, 1), (IDX, 99.0, 131072, 1)]
    write_trace(os.path.join(root, "trace"), trace)
    fetch = [(IDX, 131072, 1.0), (SPIN, 1, 0.0), (IDX, 131072, idx_kib[0]), (APP, 2048, 50.0),
             (IDX, 131072, idx_kib[1]), (APP, 2048, 50.0), (SPIN, 1, 0.0), (IDX, 131072, 1.0)]
    write_counters(os.path.join(root, "fetch"), "FETCH_SIZE", fetch)
    write = [(n, g, 100.0) for n, g, _ in fetch]
    write_counters(os.path.join(root, "write"), "WRITE_SIZE", write)


def make_calibration(root):
    n = bench.COPY_CALIBRATION_BYTES
    write_counters(os.path.join(root, "fetch"), "FETCH_SIZE", [(COPY, 1, n / 2048)] * 3)   # reads half
    write_counters(os.path.join(root, "write"), "WRITE_SIZE", [(COPY, 1, n / 1024)] * 3)


def test_summary_pairs_timed_dispatches_and_scales_counters(tmp_path):
    run, cal = str(tmp_path / "run"), str(tmp_path / "cal")
    make_run(run)
    make_calibration(cal)
    out = str(tmp_path / "traffic.json")
    md = bench.profile_summary(run, cal, "csa_decode_pro_1m", out, "cmd one ;; cmd two", timed_steps=2)
    assert "    cmd one" in md and "    cmd two" in md
    assert "idx_topk_kernel<2, 8> | index_topk | 131072 | 256 | 2 | 29.00 |" in md   # setup and late ones cut
    assert "compress_kernel<unsigned short, 1, true, false> | append | 2048 | 256 | 2 |" in md  # 512 x 4 = 2048
    t = json.load(open(out))
    idx = t["index_topk@csa_decode_pro_1m"]
    assert idx["scale"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    assert idx["read_bytes_per_step"] == int(70000.0 * 1024 * 2.0)
    assert idx["hbm_bytes_per_launch"] == idx["hbm_bytes_per_step"]
    assert t["append@csa_decode_pro_1m"]["hbm_bytes_per_step"] == int((50.0 * 2 + 100.0) * 1024)
    assert idx["source_digest"] == bench.kernel_source_digest()


def test_summary_drops_pairs_above_peak_bandwidth(tmp_path):
    run, cal = str(tmp_path / "run"), str(tmp_path / "cal")
    # the second timed index launch would move 2 GB in 30 us: not the same launch
    make_run(run, idx_kib=(70000.0, 2.0e6))
    make_calibration(cal)
    md = bench.profile_summary(run, cal, "csa_decode_pro_1m", None, "", timed_steps=2)
    assert "1 dropped" in md


def test_kernel_roles():
    """Roles follow the template arguments: the third compressor argument is APPEND
    (the fourth, SPLIT, splits long blocks over slot groups)."""
    assert bench._role(APP, "csa_decode_pro_1m+state") == "append"
    assert bench._role(CMP, "hca_prefill_chunk_1m") == "compress"
    assert bench._role(IDX, "csa_decode_pro_1m") == "index_topk"
    att = "void csa::(anonymous namespace)::attend_bf16_kernel<128, 8, true, 2, false, 1>(csa::AttendArgs)"
    assert bench._role(att, "hca_decode_1m") == "hca_attend"
