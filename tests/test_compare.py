"""Host logic of the tiled-vs-dense comparison: rocprofv3 counter files -> HBM bytes per call and GPU clock.

Synthetic counter files: a 1 GiB device copy whose FETCH_SIZE reads 0.5 GiB and
whose WRITE_SIZE reads 1 GiB (so the scale factors are 2 and 1, as measured on
gfx950), and one call of each path with known counter values.
"""
import csv

from tiled_online_softmax_causal_amd.compare import clock, page_grid, traffic, traffic_by_call

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counters_scaled_by_copy_calibration(tmp_path):
    kib = 1024 * 1024  # KiB in 1 GiB
    _write(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2)] * 3 +
           [("vectorized_elementwise_kernel<FillFunctor>", "FETCH_SIZE", 123.0)])
    _write(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", kib)] * 3)
    _write(tmp_path / "f.csv", [
        ("distribution_elementwise_grid_stride_kernel", "FETCH_SIZE", 999.0),  # input generation: ignored
        ("void fa::pp::attn_fwd_pingpong<128, 128, true, true>(...)", "FETCH_SIZE", 100.0),
        ("void fa::dense::dense_scores<128, true>(...)", "FETCH_SIZE", 10.0),
        ("void fa::dense::dense_softmax<true>(...)", "FETCH_SIZE", 20.0),
        ("void fa::dense::dense_pv<128, true>(...)", "FETCH_SIZE", 30.0)])
    _write(tmp_path / "w.csv", [
        ("void fa::pp::attn_fwd_pingpong<128, 128, true, true>(...)", "WRITE_SIZE", 7.0),
        ("void fa::dense::dense_scores<128, true>(...)", "WRITE_SIZE", 40.0),
        ("void fa::dense::dense_pv<128, true>(...)", "WRITE_SIZE", 2.0)])
    out = traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                  str(tmp_path / "cw.csv"), calls=1)
    assert out["fetch_factor"] == 2.0 and out["write_factor"] == 1.0
    assert out["flash"] == {"read_bytes": 100 * 1024 * 2, "write_bytes": 7 * 1024, "total_bytes": 207 * 1024,
                            "dispatches_per_call": 1.0}
    assert out["dense"]["read_bytes"] == 60 * 1024 * 2
    assert out["dense"]["write_bytes"] == 42 * 1024
    assert out["dense"]["dispatches_per_call"] == 3.0
    halved = traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                     str(tmp_path / "cw.csv"), calls=2)
    assert halved["dense"]["total_bytes"] == out["dense"]["total_bytes"] // 2


def test_clock_from_busy_cycles(tmp_path):
    """GRBM_GUI_ACTIVE is summed over the 8 XCDs: 8 * 1.6e6 busy cycles in 1 ms is 1.6 GHz."""
    fields = FIELDS + ["Start_Timestamp", "End_Timestamp"]
    with open(tmp_path / "g.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        rows = [("void fa::pp::attn_fwd_pingpong<128, 128, true, true>(...)", 8 * 1.6e6, 1_000_000),
                ("void fa::pp::attn_fwd_pingpong<128, 128, true, true>(...)", 8 * 2.0e6, 1_000_000),
                ("void fa::bwd::attn_bwd_dq<128, true, 2>(...)", 8 * 1.0e6, 500_000),
                ("distribution_elementwise_grid_stride_kernel", 1.0, 10)]
        for i, (name, value, ns) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": "GRBM_GUI_ACTIVE",
                        "Counter_Value": value, "Start_Timestamp": 1000, "End_Timestamp": 1000 + ns})
    out = clock(str(tmp_path / "g.csv"))
    assert out == {"bwd": {"ghz": 2.0, "dispatches": 1}, "flash": {"ghz": 1.8, "dispatches": 2}}


def test_traffic_split_per_call(tmp_path):
    """Two lengths, one call per path each: a tiled dispatch opens each call; the dense
    dispatches (3 kernels; 2 head chunks at the second length) after it belong to it."""
    kib = 1024 * 1024
    _write(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", kib / 2)])
    _write(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", kib)])
    gen = ("distribution_elementwise_grid_stride_kernel", 5.0)
    fl = "void fa::pp::attn_fwd_pingpong<128, 128, true, true>(...)"
    small = "void fa::mfma::attn_fwd_mfma_bf16<128, 64, 64, true>(...)"
    dn = ["void fa::dense::dense_scores<128, true>(...)", "void fa::dense::dense_softmax<true>(...)",
          "void fa::dense::dense_pv<128, true>(...)"]
    seq = [gen, (small, 1.0)] + [(k, 2.0) for k in dn] + [gen, (fl, 10.0)] + [(k, 3.0) for k in dn + dn]
    _write(tmp_path / "f.csv", [(n, "FETCH_SIZE", v) for n, v in seq])
    _write(tmp_path / "w.csv", [(n, "WRITE_SIZE", v / 2) for n, v in seq])
    calls = traffic_by_call(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                            str(tmp_path / "cw.csv"))
    assert len(calls) == 2
    assert calls[0]["flash"] == {"read_bytes": 2048, "write_bytes": 512, "dispatches": 1, "total_bytes": 2560}
    assert calls[0]["dense"] == {"read_bytes": 3 * 4096, "write_bytes": 3 * 1024, "dispatches": 3,
                                 "total_bytes": 15 * 1024}
    assert calls[1]["flash"]["read_bytes"] == 20 * 1024 and calls[1]["flash"]["write_bytes"] == 5 * 1024
    assert calls[1]["dense"]["dispatches"] == 6 and calls[1]["dense"]["read_bytes"] == 6 * 6 * 1024


def test_page_grid():
    """The model's profile grid: 48 lengths from 512 to 131072, each step x 256^(1/47)."""
    g = page_grid()
    assert len(g) == 48 and g[0] == 512 and g[-1] == 131072
    assert g[1] == 576 and g[2] == 648  # 512 * 1.12522 = 576.1, * 1.12522^2 = 648.3
    assert all(b > a for a, b in zip(g, g[1:]))
