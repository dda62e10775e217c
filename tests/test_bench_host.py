"""Host-side checks of bench.py's counter arithmetic (no GPU needed): the HBM
traffic summary scales FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the
same counters read for a 1 GiB device copy, keeps only the gate/up launches,
and the bench line reports the summary only while the GEMM sources are the
ones it was taken on."""
import csv
import json
import os

import bench


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


class _Cfg:
    cid, name, T = 9, "test-recipe", 77


def test_traffic_summary_scaling_and_kernel_filter(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    gu = "void moe::k_grouped_gemm_bf16<128, 128, 2, 4, 2, true, false>(moe::GemmArgs)"
    dn = "void moe::k_grouped_gemm_bf16<128, 256, 2, 4, 2, false, false>(moe::GemmArgs)"
    f, w, cf, cw = (str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    # two gate/up dispatches (1000 and 3000 KiB) and a down dispatch that must be ignored
    _write_counters(f, [{"Kernel_Name": gu, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000},
                        {"Kernel_Name": dn, "Counter_Name": "FETCH_SIZE", "Counter_Value": 9e9},
                        {"Kernel_Name": gu, "Counter_Name": "FETCH_SIZE", "Counter_Value": 3000}])
    _write_counters(w, [{"Kernel_Name": gu, "Counter_Name": "WRITE_SIZE", "Counter_Value": 10},
                        {"Kernel_Name": gu, "Counter_Name": "WRITE_SIZE", "Counter_Value": 30}])
    # the 1 GiB copy: FETCH_SIZE reads half of it, WRITE_SIZE all of it
    half, full = (1 << 30) / 2 / 1024, (1 << 30) / 1024
    _write_counters(cf, [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
                          "Counter_Value": half}])
    _write_counters(cw, [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
                          "Counter_Value": full}])
    bench.traffic_summary(_Cfg, f, w, cf, cw)
    d = json.load(open(bench.traffic_path(_Cfg)))
    assert d["dispatches"] == [2, 2]
    assert d["copy_factor_fetch"] == 2.0 and d["copy_factor_write"] == 1.0
    assert d["fetch_bytes_per_launch"] == 2 * 2000 * 1024
    assert d["write_bytes_per_launch"] == 20 * 1024
    assert d["bytes_per_launch"] == d["fetch_bytes_per_launch"] + d["write_bytes_per_launch"]
    assert d["kernel_source_hash"] == bench.kernel_source_hash()
    # reported while the sources match, withheld once they differ
    assert bench.measured_traffic(_Cfg) == d["bytes_per_launch"]
    d["kernel_source_hash"] = "0" * 16
    json.dump(d, open(bench.traffic_path(_Cfg), "w"))
    assert bench.measured_traffic(_Cfg) is None
    os.remove(bench.traffic_path(_Cfg))
    assert bench.measured_traffic(_Cfg) is None

