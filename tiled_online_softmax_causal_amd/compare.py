"""Measured comparison of the tiled and the dense attention forward on one MI355X.

    python -m tiled_online_softmax_causal_amd.compare [--seq 1024,4096,16384,32768]
        [--batch 1] [--heads 32] [--dim 128] [--paths flash,dense] [--variants auto]
        [--steps 5] [--warmup 2]
    python -m tiled_online_softmax_causal_amd.compare --traffic FETCH.csv WRITE.csv \\
        COPY_FETCH.csv COPY_WRITE.csv --calls N

The first form times both GPU paths -- fa_fwd (tiled, online softmax) and
fa_dense_fwd (score and probability matrices through HBM) -- at each sequence
length on seeded uniform(-0.8, 0.8) bf16 inputs, causal, and prints one JSON
line per (S, path) with the measured time, TFLOP/s, effective GB/s of the
compulsory bytes, and the logical bytes of the aiml.sh page's model
(run-output.txt, hbm_traffic_sweep: b1 h32 d128, S = 1024 ... 32768) for the
same shape.  --variants times the tiled path once per kernel variant (the
tilings of fa_fwd_variant: mfma_b256_k128, mfma_b256, mfma_b128, ...).  The
path "bwd" times fa_bwd (the forward's O and LSE and a seeded dO resident);
its TFLOP/s count the five products of the gradient, 2.5x the forward's flops,
and "executed_tflops" the seven its two kernels run (each recomputes P and
dP).  The second form turns rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
counter files of such a run into measured HBM bytes per call of each path,
scaled by the counters of a plain device copy of known size
(bench.py --copy-calibration).

    python -m tiled_online_softmax_causal_amd.compare --auto-check N [--shape-seed 7]

times each matrix-core tiling (mfma_b256_k128, mfma_b128, split; fa_fwd_variant)
on N seeded random causal bf16 shapes (B in 1..8, H in 4..64, S log-uniform in
128..16384, d 64 or 128) and prints one JSON line per shape with the tiling the
automatic choice (fa_fwd) takes and its time over the fastest tiling's.
"""
from __future__ import annotations

import argparse
import csv
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12


def _path_of(kernel_name: str):
    if "attn_fwd" in kernel_name:
        return "flash"
    if "dense_" in kernel_name:
        return "dense"
    if "attn_bwd" in kernel_name:
        return "bwd"
    return None


def _counter_kib(path: str) -> dict:
    """Sum of a counter (KiB) over each path's dispatches, and the dispatch counts."""
    tot, n = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = _path_of(r["Kernel_Name"])
            if key is None:
                continue
            tot[key] = tot.get(key, 0.0) + float(r["Counter_Value"])
            n[key] = n.get(key, 0) + 1
    return {k: (tot[k], n[k]) for k in tot}


def _copy_kib(path: str) -> float:
    """Mean of a counter (KiB) over the plain device copies (rocclr copyBuffer)."""
    with open(path) as f:
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(f) if "copyBuffer" in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no copy dispatches in {path}")
    return sum(vals) / len(vals)


def traffic(fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str, calls: int,
            copy_mib: int = 1024) -> dict:
    """HBM bytes per call of each path, each counter scaled by its plain-copy reading."""
    f_fac = copy_mib * 1024 / _copy_kib(copy_fetch_csv)
    w_fac = copy_mib * 1024 / _copy_kib(copy_write_csv)
    fetch, write = _counter_kib(fetch_csv), _counter_kib(write_csv)
    out = {"fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)}
    for p in sorted(set(fetch) | set(write)):
        rd = fetch.get(p, (0.0, 0))[0] * 1024 * f_fac / calls
        wr = write.get(p, (0.0, 0))[0] * 1024 * w_fac / calls
        out[p] = {"read_bytes": int(rd), "write_bytes": int(wr), "total_bytes": int(rd + wr),
                  "dispatches_per_call": fetch.get(p, (0, 0))[1] / calls}
    return out


def _dispatch_kib(path: str) -> list:
    """(dispatch id, path, KiB) of each counted dispatch, in dispatch order."""
    with open(path) as f:
        rows = [(int(r["Dispatch_Id"]), _path_of(r["Kernel_Name"]), float(r["Counter_Value"])) for r in csv.DictReader(f)]
    return sorted(r for r in rows if r[1] is not None)


def traffic_by_call(fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str,
                    copy_mib: int = 1024) -> list:
    """HBM bytes of each call, in call order, for a run of one call per path at each
    sequence length (compare.py --steps 1 --warmup 0): every tiled dispatch opens a call,
    and the dense dispatches after it (one per kernel and head chunk) belong to it."""
    f_fac = copy_mib * 1024 / _copy_kib(copy_fetch_csv)
    w_fac = copy_mib * 1024 / _copy_kib(copy_write_csv)
    calls = []
    for rows, key, fac in ((_dispatch_kib(fetch_csv), "read_bytes", f_fac), (_dispatch_kib(write_csv), "write_bytes", w_fac)):
        i = -1
        for _, p, kib in rows:
            if p == "flash":
                i += 1
            if i < 0:
                raise SystemExit(f"a {p} dispatch before the first tiled one")
            if i == len(calls):
                calls.append({})
            d = calls[i].setdefault(p, {"read_bytes": 0.0, "write_bytes": 0.0, "dispatches": 0})
            d[key] += kib * 1024 * fac
            if key == "read_bytes":
                d["dispatches"] += 1
    for c in calls:
        for d in c.values():
            d["read_bytes"], d["write_bytes"] = int(d["read_bytes"]), int(d["write_bytes"])
            d["total_bytes"] = d["read_bytes"] + d["write_bytes"]
    return calls


def page_grid() -> list:
    """The 48 sequence lengths of the reduced-order model's profile curves, rounded."""
    from tiled_online_softmax_causal_amd.costmodel import page_profile_seqs

    return [int(round(s)) for s in page_profile_seqs()]


def clock(grbm_csv: str, n_xcd: int = 8) -> dict:
    """Mean GPU clock (GHz) over each path's dispatches: GRBM_GUI_ACTIVE, the cycles the
    graphics engine is busy, summed over the n_xcd XCDs, divided by the dispatch's duration."""
    acc = {}
    with open(grbm_csv) as f:
        for r in csv.DictReader(f):
            key = _path_of(r["Kernel_Name"])
            if key is None or r["Counter_Name"] != "GRBM_GUI_ACTIVE":
                continue
            ns = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            if ns <= 0:
                continue
            ghz = float(r["Counter_Value"]) / n_xcd / ns
            s, n = acc.get(key, (0.0, 0))
            acc[key] = (s + ghz, n + 1)
    return {k: {"ghz": round(s / n, 3), "dispatches": n} for k, (s, n) in sorted(acc.items())}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--seq", default="1024,4096,16384,32768",
                    help="comma list of sequence lengths, or 'grid48': the model's 48-point profile grid")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--heads", type=int, default=32)
    ap.add_argument("--dim", type=int, default=128)
    ap.add_argument("--paths", default="flash,dense")
    ap.add_argument("--variants", default="auto", help="comma list of tiled-path variants (fa_fwd_variant)")
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--max-workspace-gib", type=float, default=64.0,
                    help="workspace of the dense path; heads are processed in chunks that fit")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"))
    ap.add_argument("--calls", type=int, default=1, help="attention calls per path in the profiled run")
    ap.add_argument("--per-call", action="store_true",
                    help="with --traffic: one line per call (one call per path at each --seq length)")
    ap.add_argument("--inputs", choices=("uniform", "zeros"), default="uniform",
                    help="uniform(-0.8, 0.8) (the workload) or all-zero Q, K, V: the same instructions with "
                         "no switching in the matrix-core operands, to separate power from issue limits")
    ap.add_argument("--auto-check", type=int, default=0, metavar="N",
                    help="time the automatic choice against each matrix-core tiling on N random shapes")
    ap.add_argument("--shape-seed", type=int, default=7)
    ap.add_argument("--clock", metavar="GRBM_CSV",
                    help="rocprofv3 --pmc GRBM_GUI_ACTIVE counter file -> mean GPU clock of each path's kernels")
    args = ap.parse_args()
    if args.clock:
        print(json.dumps(clock(args.clock)))
        return
    if args.auto_check:
        auto_check(args.auto_check, args.shape_seed)
        return
    seqs = page_grid() if args.seq == "grid48" else [int(s) for s in args.seq.split(",")]
    if args.traffic and args.per_call:
        calls = traffic_by_call(*args.traffic)
        if len(calls) != len(seqs):
            raise SystemExit(f"{len(calls)} calls in the counter files, {len(seqs)} lengths in --seq")
        for S, c in zip(seqs, calls):
            print(json.dumps({"seq_len": S, **c}))
        return
    if args.traffic:
        print(json.dumps(traffic(*args.traffic, calls=args.calls)))
        return

    import torch

    import tiled_online_softmax_causal_amd as fa
    from tiled_online_softmax_causal_amd.costmodel import algorithmic_bytes, attention_flops, page_logical_traffic
    from workloads import uniform_qkv_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, D = args.batch, args.heads, args.dim
    runs = []
    for path in args.paths.split(","):
        runs += [(path, v) for v in args.variants.split(",")] if path == "flash" else [(path, None)]
    for v in args.variants.split(","):
        if v not in fa.VARIANTS:
            raise SystemExit(f"unknown variant {v}; one of {sorted(fa.VARIANTS)}")
    for S in seqs:
        q, k, v = uniform_qkv_device(B, H, S, D, seed=42, dtype=torch.bfloat16, device=dev)
        if args.inputs == "zeros":
            for t in (q, k, v):
                t.zero_()
        scale = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32).item())
        model = page_logical_traffic(S, num_heads=B * H, head_dim=D)
        for path, variant in runs:
            ws = None
            if path == "bwd":
                o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
                do, _, _ = uniform_qkv_device(B, H, S, D, seed=1042, low=-1.0, high=1.0, dtype=torch.bfloat16,
                                              device=dev)
                ws = torch.empty(B * H * S, dtype=torch.float32, device=dev)
            if path == "dense":
                per_head = fa.dense_workspace_bytes(S)
                n = max(1, min(B * H, int(args.max_workspace_gib * 2**30) // per_head))
                ws = torch.empty(n * per_head, dtype=torch.uint8, device=dev)

            def call():
                if path == "bwd":
                    return fa.bwd(q, k, v, o, lse, do, causal=True, scale=scale, workspace=ws)
                if path == "dense":
                    return fa.dense_fwd(q, k, v, causal=True, scale=scale, workspace=ws)
                return fa.fwd(q, k, v, causal=True, scale=scale, variant=variant)

            for _ in range(args.warmup):
                call()
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            for _ in range(args.steps):
                call()
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / args.steps
            flops = attention_flops(B, H, S, D, True) * (2.5 if path == "bwd" else 1.0)
            # bwd reads Q, K, V, O, dO and writes dQ, dK, dV (plus LSE and delta)
            nbytes = algorithmic_bytes(B, H, S, D, 2) * (2 if path == "bwd" else 1)
            print(json.dumps({
                "path": path, "variant": variant, "inputs": args.inputs, "batch": B, "heads": H, "seq_len": S, "head_dim": D, "causal": True,
                "ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                "pct_of_peak": round(100 * flops / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
                "compulsory_bytes": nbytes, "effective_gbs": round(nbytes / ms / 1e6, 1),
                "executed_tflops": round(flops * 1.4 / ms / 1e9, 1) if path == "bwd" else None,
                "dense_workspace_heads": None if (ws is None or path != "dense") else ws.numel() // fa.dense_workspace_bytes(S),
                "page_model_mb": {"standard_total": round(model["standard_total_bytes"] / 1e6, 2),
                                  "tiled_logical": round(model["tiled_logical_bytes"] / 1e6, 2),
                                  "qkvo_compulsory": round(model["qkvo_bytes"] / 1e6, 2)},
            }), flush=True)
            del ws
            torch.cuda.empty_cache()
        del q, k, v
        torch.cuda.empty_cache()


def auto_check(n: int, seed: int):
    """The automatic choice (fa_fwd) against each matrix-core tiling on n seeded random shapes."""
    import random

    import torch

    import tiled_online_softmax_causal_amd as fa
    from tiled_online_softmax_causal_amd.costmodel import attention_flops
    from workloads import uniform_qkv_device

    rng = random.Random(seed)
    shapes = []
    while len(shapes) < n:
        D = rng.choice([64, 128])
        B = rng.choice([1, 1, 2, 4, 8])
        H = rng.choice([4, 8, 12, 16, 24, 32, 48, 64])
        S = int(2 ** rng.uniform(math.log2(128), math.log2(16384)))
        if B * H * S * D <= 2**29:  # at most 1 GiB per bf16 tensor
            shapes.append((B, H, S, D))
    tilings = ["mfma_b256_k128", "mfma_b128", "split"]
    names = {v: k for k, v in fa.VARIANTS.items()}
    us_all = []
    for B, H, S, D in shapes:
        q, k, v = uniform_qkv_device(B, H, S, D, seed=42, dtype=torch.bfloat16, device="cuda")
        scale = float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32).item())
        flops = attention_flops(B, H, S, D, True)
        reps = max(3, min(50, int(4e14 / (flops * 1e3 + 1))))
        us = {}
        order = tilings[len(us_all) % 3:] + tilings[:len(us_all) % 3]  # rotate: no tiling always first
        for var in order:
            # warm up for about 30 ms: under load the clock takes a few ms to settle
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                fa.fwd(q, k, v, causal=True, scale=scale, variant=var)
            e1.record()
            torch.cuda.synchronize()
            per_call = max(e0.elapsed_time(e1) / 3, 1e-3)
            for _ in range(min(200, int(30.0 / per_call))):
                fa.fwd(q, k, v, causal=True, scale=scale, variant=var)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fa.fwd(q, k, v, causal=True, scale=scale, variant=var)
            e1.record()
            torch.cuda.synchronize()
            us[var] = e0.elapsed_time(e1) / reps * 1e3
        us_all.append(us)
        best = min(tilings, key=us.get)
        # fa_fwd runs exactly the chosen tiling's kernel and schedule, so the
        # choice is judged on that tiling's own timing
        choice = names.get(fa.select_variant(B, H, S, D), "?")
        print(json.dumps({"shape": [B, H, S, D], "us": {k_: round(x, 1) for k_, x in us.items()},
                          "auto_variant": choice, "fastest_tiling": best,
                          "choice_over_fastest": round(us[choice] / us[best], 3) if choice in us else None}),
              flush=True)
        del q, k, v
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
