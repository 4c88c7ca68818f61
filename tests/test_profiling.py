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
