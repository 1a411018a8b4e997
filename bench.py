"""Throughput of the causal attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--cold]
                    [--entry fa_fwd_ws|fa_fwd]

One step is one forward call (the whole forward pass: causal tile schedule,
Q/K/V tile loads, both matrix products, online softmax, epilogue with the
log-sum-exp) over one batch of synthetic bf16 input that is already resident in
HBM.  The call is fa_fwd_ws by default: fa_fwd with a scheduling workspace,
which balances the last work items across XCDs at run time (the same results,
bit for bit); --entry fa_fwd times the static schedule.  W untimed steps, then K timed steps between two device synchronisations.
Prints ONE JSON line on stdout; progress goes to stderr.

FLOPs follow the chipfoundryservices.com "FlashAttention" reduced-order model
(outputs.flops_gflop): the two matrix products only, 4*B*H*S^2*D, halved under
the causal rule.  Bytes are the compulsory ones: Q, K, V read once, O written
once, the fp32 log-sum-exp written once.

With --cold, each of K further launches is preceded by a 1 GiB write to a
scratch buffer, which evicts Q, K and V from the L2 caches and the 256 MB
Infinity Cache, and timed alone with HIP events (the median is reported in
"cold"): the working set of the smaller workloads otherwise stays cached
between steps.

The CPU baseline times the fp64 oracle (plain C, all visible cores up to 16) on
a bounded sample of the same workload -- whole heads, every row -- and checks
the GPU output on that sample at the same time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd TFLOP/s and % of bf16 MFMA peak, b8 h32 S8192 d128"
# MI355X: 256 CUs x 4096 dense bf16 MFMA flop/clk x 2.4 GHz (AMD's 2.5 PFLOP/s), 8 TB/s HBM3E
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0

# name -> (B, H, S, D, causal, cpu-sample heads)
WORKLOADS = {
    "b8_h32_s8192_d128_causal": (8, 32, 8192, 128, True, 8),
    "b1_h32_s1024_d128_causal": (1, 32, 1024, 128, True, 32),
    "b1_h32_s4096_d128_causal": (1, 32, 4096, 128, True, 16),
    "b1_h32_s4096_d128_noncausal": (1, 32, 4096, 128, False, 8),
    "b1_h32_s32768_d128_causal": (1, 32, 32768, 128, True, 1),
}
DEFAULT = "b8_h32_s8192_d128_causal"
CSRC = os.path.join(ROOT, "tiled_online_softmax_causal_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_traffic.json")


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3
    counter runs, or None if the kernel sources changed since the counters were
    taken or the counters are for another kernel (another schedule or variant)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload)
    if not entry or rec.get("source_sha256") != kernel_source_hash():
        return None
    if not str(entry.get("kernel", "")).startswith(kernel):
        return None
    return entry.get("hbm_bytes_per_launch")


def _counter_mean(csv_path: str, counter: str, kernel_substr: str):
    """Mean of `counter` over the dispatches of the one kernel matching kernel_substr,
    and that kernel's name (without its argument list)."""
    import csv
    rows = [r for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"no {counter} rows for a kernel matching {kernel_substr!r} in {csv_path}")
    names = {r["Kernel_Name"].split("(")[0].replace("void ", "").strip() for r in rows}
    if len(names) != 1:
        raise SystemExit(f"several kernels match {kernel_substr!r} in {csv_path}: {sorted(names)}")
    return sum(float(r["Counter_Value"]) for r in rows) / len(rows), names.pop()


def record_traffic(workload: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str,
                   copy_write_csv: str, copy_mib: int):
    """Turn four rocprofv3 --pmc counter_collection.csv files into HBM bytes per launch.

    FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by what the same
    counter reports for a plain device copy of copy_mib MiB (read and written once).
    The result is stored with a hash of the kernel sources, so it is reported only
    while the kernel is unchanged.
    """
    fetch_kib, kernel = _counter_mean(fetch_csv, "FETCH_SIZE", "attn_fwd")
    write_kib, kernel_w = _counter_mean(write_csv, "WRITE_SIZE", "attn_fwd")
    if kernel_w != kernel:
        raise SystemExit(f"the counter runs are of different kernels: {kernel} / {kernel_w}")
    copy_fetch_kib, _ = _counter_mean(copy_fetch_csv, "FETCH_SIZE", "copyBuffer")
    copy_write_kib, _ = _counter_mean(copy_write_csv, "WRITE_SIZE", "copyBuffer")
    true_kib = copy_mib * 1024.0
    f_fetch, f_write = true_kib / copy_fetch_kib, true_kib / copy_write_kib
    hbm = fetch_kib * 1024 * f_fetch + write_kib * 1024 * f_write
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    if rec.get("source_sha256") != kernel_source_hash():
        rec = {"source_sha256": kernel_source_hash(), "workloads": {}}
    rec["workloads"][workload] = {
        "kernel": kernel,
        "hbm_bytes_per_launch": round(hbm),
        "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
        "copy_calibration": {"mib": copy_mib, "fetch_kib": copy_fetch_kib, "write_kib": copy_write_kib,
                             "fetch_factor": f_fetch, "write_factor": f_write},
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec["workloads"][workload]))


def cpu_baseline(q, k, v, o, lse, n_heads: int, causal: bool, scale: float):
    """Time the fp64 oracle on n_heads whole heads (every row); check the GPU on them."""
    import numpy as np
    import torch

    from oracle import attention_dense
    from oracle.dense import default_threads

    B, H, S, D = q.shape
    step = max(1, (B * H) // n_heads)
    bh = [min(B * H - 1, i * step + (i * 7) % step) for i in range(n_heads)]
    idx = torch.as_tensor(bh, device=q.device)
    host = [t.reshape(B * H, S, D).index_select(0, idx).view(torch.uint16).cpu().numpy()[None]
            for t in (q, k, v)]
    threads = default_threads()
    t0 = time.perf_counter()
    ref_o, ref_l = attention_dense(*host, dtype="bf16", causal=causal, scale=scale, n_threads=threads)
    secs = time.perf_counter() - t0
    rows = np.arange(S)
    flops = sum(4.0 * D * ((r + 1) if causal else S) for r in rows) * n_heads
    og = o.reshape(B * H, S, D).index_select(0, idx).float().cpu().numpy().astype(np.float64)
    lg = lse.reshape(B * H, S).index_select(0, idx).cpu().numpy().astype(np.float64)
    err = np.abs(og - ref_o)
    parity = {"heads_checked": bh, "rows_per_head": S, "o_max_abs": float(err.max()),
              "o_mean_abs": float(err.mean()), "lse_max_abs": float(np.abs(lg - ref_l).max()),
              "tolerance": {"o_max": 1e-2, "o_mean": 1e-3, "lse_max": 1e-3}}
    parity["ok"] = (parity["o_max_abs"] <= 1e-2 and parity["o_mean_abs"] <= 1e-3
                    and parity["lse_max_abs"] <= 1e-3)
    base = {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(),
            "sample": f"{n_heads} of {B * H} (batch, head) pairs, all {S} rows each "
                      f"({flops / 1e9:.1f} GFLOP fp64), {secs:.2f} s",
            "seconds": secs}
    return base, parity


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    from tiled_online_softmax_causal_amd import VARIANTS
    ap.add_argument("--variant", default="auto", choices=list(VARIANTS))
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--entry", default="fa_fwd_ws", choices=("fa_fwd_ws", "fa_fwd"),
                    help="the C entry point timed (fa_fwd_ws: with the scheduling workspace)")
    ap.add_argument("--cold", action="store_true",
                    help="also time K launches each after a 1 GiB cache-evicting write (median reported)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of attention, run --steps plain device copies of MIB MiB (the "
                         "reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="store HBM bytes per launch for --workload from rocprofv3 --pmc counter CSVs "
                         "(attention run and --copy-calibration run), then exit")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size used for --copy-calibration")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.workload, *args.record_traffic, args.copy_mib)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(the forward pass shards over (batch, head) with no communication; run one process per GPU)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import tiled_online_softmax_causal_amd as fa
    from tiled_online_softmax_causal_amd.costmodel import algorithmic_bytes, attention_flops
    from workloads import uniform_qkv_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": args.steps}), flush=True)
        return

    B, H, S, D, causal, cpu_heads = WORKLOADS[args.workload]
    log(f"[bench] {fa.version()} on {torch.cuda.get_device_name(dev)}; workload {args.workload}")
    q, k, v = uniform_qkv_device(B, H, S, D, seed=args.seed, dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    scale = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32).item())
    variant = fa.VARIANTS[args.variant]
    if variant == fa.FA_VARIANT_AUTO:
        variant = fa.select_variant(B, H, S, D, fa.FA_DTYPE_BF16)
    stream = torch.cuda.current_stream(dev)
    use_ws = args.entry == "fa_fwd_ws"
    if use_ws and args.variant != "auto":
        raise SystemExit("--entry fa_fwd_ws runs the automatic variant")
    ws = torch.zeros(fa.fwd_workspace_bytes(), dtype=torch.uint8, device=dev) if use_ws else None
    # what the library does with the workspace: balance when the ping-pong grid is
    # resident over whole XCDs with at least 8 heads per XCD
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    n_items = B * H * math.ceil(S / 256)
    balanced = (use_ws and variant in (fa.FA_VARIANT_MFMA_B256, fa.FA_VARIANT_MFMA_B256_K128)
                and (B * H) % 8 == 0 and B * H >= 64 and cus % 8 == 0 and n_items > cus)

    # fa_fwd for the automatic variant, fa_fwd_variant for an explicit one
    call_variant = "auto" if args.variant == "auto" else variant

    def step():
        if use_ws:
            fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse, stream=stream, workspace=ws)
        else:
            fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse, variant=call_variant, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    flops = attention_flops(B, H, S, D, causal)
    nbytes = algorithmic_bytes(B, H, S, D, 2)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    log(f"[bench] {ms_per_step:.4f} ms/step (wall), kernel {kernel_ms:.4f} ms (events), "
        f"{achieved:.1f} TFLOP/s = {100 * achieved / PEAK_BF16_TFLOPS:.1f}% of bf16 peak, "
        f"{nbytes / (kernel_ms * 1e-3) / 1e9:.1f} GB/s effective")

    traffic = measured_traffic(args.workload, fa.kernel_name(variant, D, causal, balanced))
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": fa.kernel_name(variant, D, causal, balanced), "kernel_ms": round(kernel_ms, 5),
                "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
                "effective_hbm_gbs": round(nbytes / (kernel_ms * 1e-3) / 1e9, 1),
                "hbm_frac": round(nbytes / (kernel_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": args.workload.replace("_", " "), "batch": B, "heads": H, "seq_len": S,
                   "head_dim": D, "causal": causal, "layout": "[B,H,S,D] contiguous",
                   "inputs": f"uniform(-0.8,0.8) seed {args.seed}, scale fp32(1/sqrt({D}))",
                   "variant": [n for n, c in fa.VARIANTS.items() if c == variant][0],
                   "entry": args.entry, "schedule": "balanced" if balanced else "static",
                   "parallelism": "single GPU"},
        "roofline": roofline,
    }
    if args.cold:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        times = []
        for i in range(args.steps):
            scratch.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del scratch
        cold_ms = sorted(times)[len(times) // 2]
        result["cold"] = {"evict_bytes": 1 << 30, "launches": args.steps, "kernel_ms_median": round(cold_ms, 5),
                          "kernel_ms_min": round(min(times), 5),
                          "tflops": round(flops / (cold_ms * 1e-3) / 1e12, 2),
                          "effective_hbm_gbs": round(nbytes / (cold_ms * 1e-3) / 1e9, 1)}
        log(f"[bench] cold: median {cold_ms:.4f} ms over {args.steps} launches, "
            f"{result['cold']['effective_hbm_gbs']} GB/s effective")
    # One more step after the timed ones, into outputs filled with NaN and with
    # the same workspace: the parity check below reads this step's outputs, so it
    # shows that a call in the timed configuration computes every row (a skipped
    # work item would leave NaN), and that the workspace comes back zeroed.
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    step()
    torch.cuda.synchronize()
    unwritten = int((~torch.isfinite(o)).sum().item()) + int((~torch.isfinite(lse)).sum().item())
    ws_clean = True if ws is None else int(ws.count_nonzero().item()) == 0
    log(f"[bench] poisoned check step: {unwritten} non-finite outputs, workspace zero: {ws_clean}")

    if not args.no_cpu_baseline:
        log(f"[bench] oracle on {cpu_heads} whole heads (CPU baseline + parity)")
        base, parity = cpu_baseline(q, k, v, o, lse, cpu_heads, causal, scale)
        log(f"[bench] oracle {base['seconds']:.2f} s on {base['cores']} threads; parity {parity}")
        base.pop("seconds")
        result["cpu_baseline"] = base
        parity["checked_step"] = "after the timed steps, into NaN-filled outputs, same workspace"
        parity["non_finite_outputs"] = unwritten
        parity["workspace_left_zero"] = ws_clean
        parity["ok"] = parity["ok"] and unwritten == 0 and ws_clean
        result["parity"] = parity
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
