"""Host-side checks of the profile summarisers (synthetic rocprofv3 CSVs)."""
import csv
import json
import types

import pytest

from compressed_cache_decode_jolt_amd import profiling as P


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


def test_window_mean_orders_by_start_and_filters_by_name(tmp_path):
    # dispatches out of file order; a second kernel interleaved
    rows = [("decode_mfma<1>", 300, 340), ("merge", 150, 160), ("decode_mfma<2>", 100, 110),
            ("decode_mfma<1>", 200, 230), ("decode_mfma<2>", 400, 450)]
    p = _write(tmp_path / "trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    # decode_mfma in start order: 10, 30, 40, 50 ns
    assert P.window_mean(p, "decode_mfma", 0, 4) == pytest.approx(32.5e-3)
    assert P.window_mean(p, "decode_mfma", 1, 2) == pytest.approx(35e-3)
    assert P.window_mean(p, "merge", 0, 1) == pytest.approx(10e-3)
    with pytest.raises(AssertionError):
        P.window_mean(p, "decode_mfma", 3, 2)


def test_traffic_scales_counters_by_the_copy_calibration(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    copy = 1 << 20
    # the copy kernel reads 512 units and writes 1024 units for 1 MiB each way;
    # counters of one dispatch may come split over several rows (summed)
    cf = _write(tmp_path / "cf.csv", hdr, [(1, "copy", "FETCH_SIZE", 300), (1, "copy", "FETCH_SIZE", 212),
                                           (2, "fill", "FETCH_SIZE", 7)])
    cw = _write(tmp_path / "cw.csv", hdr, [(1, "copy", "WRITE_SIZE", 1024)])
    kf = _write(tmp_path / "kf.csv", hdr, [(5, "decode_mfma<x>", "FETCH_SIZE", 10),
                                           (9, "decode_mfma<x>", "FETCH_SIZE", 30),
                                           (7, "other", "FETCH_SIZE", 999)])
    kw = _write(tmp_path / "kw.csv", hdr, [(5, "decode_mfma<x>", "WRITE_SIZE", 4),
                                           (9, "decode_mfma<x>", "WRITE_SIZE", 4)])
    out = tmp_path / "traffic.json"
    a = types.SimpleNamespace(calib_fetch=cf, calib_write=cw, fetch=kf, write=kw, kernel="decode_mfma",
                              copy_bytes=copy, out=str(out), workload="w", name=None)
    P.traffic(a)
    rec = json.load(open(out))["w/decode_mfma"]
    assert rec["calibration"]["fetch_bytes_per_unit"] == pytest.approx(copy / 512)
    assert rec["calibration"]["write_bytes_per_unit"] == pytest.approx(copy / 1024)
    assert rec["fetch_bytes_per_launch"] == pytest.approx(20 * copy / 512)
    assert rec["write_bytes_per_launch"] == pytest.approx(4 * copy / 1024)
    assert rec["dispatches"] == [2, 2]
    assert rec["kernel_hash"] == P.kernel_hash()


def test_kernel_hash_is_stable():
    h = P.kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert P.kernel_hash() == h


def test_counters_table_means_per_dispatch_and_ratios(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = [(1, "decode_mfma<a>", "SQ_BUSY_CU_CYCLES", 100), (1, "decode_mfma<a>", "SQ_BUSY_CU_CYCLES", 100),
            (1, "decode_mfma<a>", "SQ_VALU_MFMA_BUSY_CYCLES", 50),
            (2, "decode_mfma<a>", "SQ_BUSY_CU_CYCLES", 400), (2, "decode_mfma<a>", "SQ_VALU_MFMA_BUSY_CYCLES", 250),
            (3, "merge", "SQ_BUSY_CU_CYCLES", 7), (3, "merge", "SQ_VALU_MFMA_BUSY_CYCLES", 7)]
    p = _write(tmp_path / "pmc.csv", hdr, rows)
    t = P.counters_table(p, "decode_mfma").splitlines()
    assert len(t) == 3 and "merge" not in "\n".join(t)
    cells = [c.strip() for c in t[2].strip("|").split("|")]
    # busy: (200 + 400) / 2 = 300; mfma: (50 + 250) / 2 = 150; ratio 0.5
    assert cells[1] == "2" and cells[2] == "300" and cells[3] == "150" and cells[4] == "0.500"


def test_call_window_spans_split_kernels_and_the_value_pass(tmp_path):
    # call 1: two split launches, merge, value pass; call 2: one split launch
    # and merge only (no value pass); call 3: split, merge, value pass
    rows = [("decode_mfma<a>", 100, 150), ("decode_mfma<b>", 150, 190), ("merge_outputs", 190, 195),
            ("value_gemm", 195, 230), ("value_finish", 230, 250),
            ("decode_mfma<a>", 300, 340), ("merge_outputs", 340, 345), ("other", 350, 900),
            ("decode_mfma<a>", 1000, 1040), ("merge_outputs", 1040, 1045), ("value_gemm", 1045, 1060),
            ("value_finish", 1060, 1070)]
    p = _write(tmp_path / "trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    # spans: 250 - 100, 340 - 300, 1070 - 1000 ns
    assert P.call_window_mean(p, 0, 3) == pytest.approx((150 + 40 + 70) / 3 / 1e3)
    assert P.call_window_mean(p, 1, 1) == pytest.approx(40e-3)


def test_call_window_splits_back_to_back_calls_of_one_class(tmp_path):
    # single-split calls write their output in the split kernel: three calls
    # of one class with nothing in between, then a call with two classes
    rows = [("decode_mfma<a>", 100, 140), ("decode_mfma<a>", 150, 180), ("decode_mfma<a>", 190, 200),
            ("decode_mfma<a>", 300, 320), ("decode_mfma<b>", 320, 360), ("merge_outputs", 360, 370)]
    p = _write(tmp_path / "trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    # spans: 40, 30, 10, 360 - 300 ns
    assert P.call_window_mean(p, 0, 4) == pytest.approx((40 + 30 + 10 + 60) / 4 / 1e3)
    assert P.call_window_mean(p, 3, 1) == pytest.approx(60e-3)


def test_call_window_with_one_dispatch_per_call(tmp_path):
    # one-class calls of different classes back to back, nothing in between
    rows = [("decode_mfma<a>", 100, 140), ("decode_mfma<b>", 150, 180), ("value_gemm", 180, 190),
            ("value_finish", 190, 195), ("decode_mfma<c>", 200, 260)]
    p = _write(tmp_path / "trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    assert P.call_window_mean(p, 0, 3, per_call=1) == pytest.approx((40 + 45 + 60) / 3 / 1e3)


def test_traffic_per_launch_counts_every_kernel_of_a_call(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    cf = _write(tmp_path / "cf.csv", hdr, [(1, "copy", "FETCH_SIZE", 1024)])
    cw = _write(tmp_path / "cw.csv", hdr, [(1, "copy", "WRITE_SIZE", 1024)])
    # two layer calls: decode + value pass, decode alone
    kf = _write(tmp_path / "kf.csv", hdr, [(1, "decode_mfma<x>", "FETCH_SIZE", 10),
                                           (2, "value_gemm", "FETCH_SIZE", 6),
                                           (3, "value_finish", "FETCH_SIZE", 2),
                                           (4, "decode_mfma<y>", "FETCH_SIZE", 30)])
    kw = _write(tmp_path / "kw.csv", hdr, [(1, "decode_mfma<x>", "WRITE_SIZE", 4),
                                           (4, "decode_mfma<y>", "WRITE_SIZE", 4)])
    out = tmp_path / "traffic.json"
    a = types.SimpleNamespace(calib_fetch=cf, calib_write=cw, fetch=kf, write=kw,
                              kernel="decode_mfma|value_gemm|value_finish", copy_bytes=1024,
                              out=str(out), workload="w", name="decode_mfma", dispatches_per_launch=1.0)
    P.traffic(a)
    rec = json.load(open(out))["w/decode_mfma"]
    assert rec["fetch_bytes_per_launch"] == pytest.approx((10 + 6 + 2 + 30) / 2)
    assert rec["write_bytes_per_launch"] == pytest.approx(4.0)
