"""Host-side contract of bench.py: it measures one GPU and refuses more, before
touching a device (the forward pass shards over (batch, head) with no
communication, so a multi-GPU run is one process per GPU, outside the bench)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_world_size_above_one_is_refused():
    r = _run(["--steps", "1", "--warmup", "0"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU" in r.stderr


def _counter_csv(path, kernel, counter, value, n=3):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i in range(n):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_record_is_keyed_by_kernel_and_sources(tmp_path, monkeypatch):
    """bench.py's roofline.traffic: counter KiB scaled by a plain copy's reading,
    reported only for the kernel and the sources the counters were taken on."""
    import json

    sys.path.insert(0, ROOT)
    import bench

    rec_file = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec_file))
    kernel = "fa::pp::attn_fwd_pingpong<128, 128, true, true>"
    _counter_csv(tmp_path / "f.csv", f"void {kernel}(unsigned short const*, ...)", "FETCH_SIZE", 1000.0)
    _counter_csv(tmp_path / "w.csv", f"void {kernel}(unsigned short const*, ...)", "WRITE_SIZE", 300.0)
    # a 1 MiB copy whose FETCH_SIZE reads half of what moved and WRITE_SIZE all of it
    _counter_csv(tmp_path / "cf.csv", "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)
    _counter_csv(tmp_path / "cw.csv", "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)
    bench.record_traffic("b8_h32_s8192_d128_causal", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                         str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 1)
    want = 1000.0 * 1024 * 2 + 300.0 * 1024 * 1
    assert bench.measured_traffic("b8_h32_s8192_d128_causal", kernel) == round(want)
    # another schedule of the same kernel, or another workload: no figure
    assert bench.measured_traffic("b8_h32_s8192_d128_causal", "fa::pp::attn_fwd_pingpong<128, 128, true, false>") is None
    assert bench.measured_traffic("b1_h32_s1024_d128_causal", kernel) is None
    # sources changed since the counters were taken: no figure
    rec = json.loads(rec_file.read_text())
    rec["source_sha256"] = "0" * 64
    rec_file.write_text(json.dumps(rec))
    assert bench.measured_traffic("b8_h32_s8192_d128_causal", kernel) is None
