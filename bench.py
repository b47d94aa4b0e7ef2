"""W12 GEMM benchmark on one MI355X.

Workload (one step): the MLP GEMMs at hidden size 5120 - gate and up
(17408 x 5120) and down (5120 x 17408) - as exact W12 GEMMs with fp32
accumulation and BF16 output, at M = 1 and M = 32 activation rows: six GEMM
calls per step. Weights are synthetic per-output-channel Gaussians (per-row
lognormal scales, 1e-4 outliers x 2^12, 1e-4 zeros), encoded on the GPU
before timing; activations are BF16 N(0, 1). Every input is resident in HBM
before the timed region. Each step rotates through R encoded copies of each
matrix (R * 401 MB well above the 256 MB last-level cache), so weights
stream from HBM, as in the pages' cold-L2 measurements.

Prints one JSON line: value = packed W12 bytes (1.5 B per weight) streamed
per second over the whole step, plus per-call figures, the roofline entry of
the dominant kernel and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W12 GEMM achieved HBM GB/s (% of peak) and µs/call at M=1 and M=32"
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "w12_gemm_mlp5120_pmc_traffic.md")
GEMM_SOURCES = ["lossless_compressed_weight_amd/csrc/w12_gemm.hip", "lossless_compressed_weight_amd/csrc/w12_api.hip",
                "lossless_compressed_weight_amd/csrc/w12_internal.h"]
PEAK_GBS = 8000.0
MS = (1, 32)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copies", type=int, default=4, help="encoded copies of each matrix to rotate through")
    ap.add_argument("--cpu-rows", type=int, default=0, help="rows of each matrix in the CPU oracle sample (0: all)")
    ap.add_argument("--cpu-passes", type=int, default=2, help="passes of the oracle over its sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--ms", type=str, default=None, help="comma-separated M values (default 1,32)")
    ap.add_argument("--probe-sweep", type=str, default=None,
                    help="run only the read-bandwidth probe over its parameter grid; JSON lines to this file")
    return ap.parse_args()


PROBE_REGION = 17408 * 5120 * 3 // 2   # bytes of one packed 17408 x 5120 W12 matrix
PROBE_REGIONS = 16                     # 2.1 GB rotated, far above the 256 MB last-level cache


def probe_time(w12, buf, nbytes, grid, block, loads, mode, ws, stream, reps=12, warm=2, stamps=None):
    """Per-launch times (us) of the probe reading `nbytes`, each launch on the
    next of the buffer's regions (so no launch finds its bytes in a cache)."""
    import torch
    nreg = buf.numel() // nbytes
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(warm + reps):
        view = buf[(i % nreg) * nbytes:]
        if i >= warm:
            ev[i - warm][0].record(stream)
        w12.w12_probe_read(view, nbytes, grid, block, loads, mode, stamps if i == warm + reps - 1 else None, ws,
                           stream)
        if i >= warm:
            ev[i - warm][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def probe_sweep(path):
    """Read-bandwidth probe over workgroups per CU, waves per workgroup, loads
    in flight per lane and the work distribution, on 134 MB reads (one packed
    17408 x 5120 matrix) rotated over 2.1 GB; then the best setting on one
    1.17 GB read (the packed LM head) and with per-workgroup time stamps."""
    import torch
    from lossless_compressed_weight_amd import w12
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    buf = torch.zeros(PROBE_REGION * PROBE_REGIONS, dtype=torch.uint8, device=dev)
    ws = torch.zeros(w12.PROBE_WS_BYTES, dtype=torch.uint8, device=dev)
    out = open(path, "w")
    best = None
    for mode in (w12.PROBE_STATIC, w12.PROBE_DYNAMIC, w12.PROBE_STRIDE):
        for block in (256, 512, 1024):
            for wgpc in (1, 2, 4):
                for loads in (1, 2, 4, 8):
                    t = probe_time(w12, buf, PROBE_REGION, 256 * wgpc, block, loads, mode, ws, stream)
                    med = float(np.median(t))
                    rec = {"mode": mode, "block": block, "wg_per_cu": wgpc, "loads": loads,
                           "us_median": round(med, 3), "us_min": round(min(t), 3),
                           "gbs": round(PROBE_REGION / med / 1e3, 1)}
                    out.write(json.dumps(rec) + "\n")
                    out.flush()
                    if best is None or med < best[0]:
                        best = (med, rec)
    print(f"# probe best on 134 MB: {best[1]}", file=sys.stderr, flush=True)
    # time stamps: spread of workgroup start and end times for each mode at the best occupancy
    b = best[1]
    for mode in (w12.PROBE_STATIC, w12.PROBE_DYNAMIC, w12.PROBE_STRIDE):
        grid = 256 * b["wg_per_cu"]
        st = torch.zeros(3 * grid, dtype=torch.int64, device=dev)
        t = probe_time(w12, buf, PROBE_REGION, grid, b["block"], b["loads"], mode, ws, stream, stamps=st)
        a = st.cpu().numpy().reshape(grid, 3).astype(np.int64)
        t0 = a[:, 0].min()
        start, end = (a[:, 0] - t0) * 0.01, (a[:, 1] - t0) * 0.01   # 100 MHz counter -> us
        per_xcd = {int(x): round(float(end[a[:, 2] == x].max()), 3) for x in np.unique(a[:, 2])}
        rec = {"stamps_mode": mode, "grid": grid, "block": b["block"], "loads": b["loads"],
               "us_median": round(float(np.median(t)), 3),
               "start_us": [round(float(np.percentile(start, q)), 3) for q in (0, 50, 100)],
               "end_us": [round(float(np.percentile(end, q)), 3) for q in (0, 10, 50, 90, 100)],
               "last_end_per_xcd_us": per_xcd}
        out.write(json.dumps(rec) + "\n")
        out.flush()
    # one LM-head-sized read
    big = 151936 * 5120 * 3 // 2
    big -= big % 16
    for mode in (w12.PROBE_STATIC, w12.PROBE_DYNAMIC):
        t = probe_time(w12, buf, big, 256 * b["wg_per_cu"], b["block"], b["loads"], mode, ws, stream, reps=4)
        rec = {"lm_head_bytes": big, "mode": mode, "us_median": round(float(np.median(t)), 3),
               "gbs": round(big / float(np.median(t)) / 1e3, 1)}
        out.write(json.dumps(rec) + "\n")
    out.close()


def main():
    args = parse()
    if args.probe_sweep:
        probe_sweep(args.probe_sweep)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the W12 GEMM shards along output channels with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    from lossless_compressed_weight_amd import w12

    ms = tuple(int(v) for v in args.ms.split(",")) if args.ms else MS
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    wl = synth.WORKLOADS[1]
    t0 = time.time()
    mats_host = [(spec.name, synth.workload_matrix(1, i)) for i, spec in enumerate(wl.matrices)]
    print(f"# generated weights in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    encoded = []   # per matrix: list of R W12Matrix copies
    for name, w in mats_host:
        wd = torch.from_numpy(w.view(np.int16)).to(dev)
        mat = w12.encode(wd)
        del wd
        copies = [mat] + [w12.W12Matrix(mat.n, mat.k, mat.records.clone(), mat.e_top.clone(),
                                        mat.row_ptr.clone(), mat.esc.clone(), mat.n_esc)
                          for _ in range(args.copies - 1)]
        encoded.append(copies)
    torch.cuda.synchronize()
    print(f"# encoded {len(encoded)} matrices x {args.copies} copies", file=sys.stderr, flush=True)

    xs_host = {m: synth.make_activations(m, 17408, seed=synth.activation_seed(1, 0, m)) for m in ms}
    calls = []     # (m, matrix index, x view, y, ws)
    for m in ms:
        for i, (name, w) in enumerate(mats_host):
            n, k = w.shape
            x = torch.from_numpy(xs_host[m][:, :k].copy().view(np.int16)).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            ws = w12.new_workspace(w12.OP_GEMM, n, k, m, dev)
            calls.append((m, i, x, y, ws))
    stream = torch.cuda.current_stream()

    def run_step(step, events=None):
        c = step % args.copies
        for j, (m, i, x, y, ws) in enumerate(calls):
            if events is not None:
                events[j][0].record(stream)
            w12.w12_gemm(encoded[i][c], x, y, ws, stream)
            if events is not None:
                events[j][1].record(stream)

    for s in range(args.warmup):
        run_step(s)
    torch.cuda.synchronize()

    # timed region: K steps back to back (the whole-step figure)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        run_step(args.warmup + s)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # second timed region: K more steps with HIP events around every call on
    # the launch stream (per-call figures and the roofline entry)
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in calls]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        run_step(args.warmup + args.steps + s, ev[s])
    torch.cuda.synchronize()

    per_call = []
    packed_step = 0
    for j, (m, i, x, y, ws) in enumerate(calls):
        name, w = mats_host[i]
        n, k = w.shape
        t = [ev[s][j][0].elapsed_time(ev[s][j][1]) * 1e3 for s in range(args.steps)]  # us
        mat = encoded[i][0]
        packed = n * k * 3 // 2
        algo = packed + n + 4 * (n + 1) + 8 * mat.n_esc + 2 * m * k + 2 * m * n
        med = float(np.median(t))
        per_call.append({"m": m, "matrix": name, "n": n, "k": k, "us_median": round(med, 3),
                         "us_p10": round(float(np.percentile(t, 10)), 3),
                         "us_p90": round(float(np.percentile(t, 90)), 3),
                         "us_mean": round(float(np.mean(t)), 3),
                         "packed_gbs": round(packed / med / 1e3, 1),
                         "pct_peak_packed": round(100 * packed / med / 1e3 / PEAK_GBS, 2),
                         "algo_bytes": algo, "n_esc": mat.n_esc,
                         "path": "gemv" if m <= 2 else "mfma"})
        packed_step += packed
    value = packed_step / (ms_per_step * 1e-3) / 1e9

    # dominant kernel: the GEMM path taking the most time per step
    by_path = {}
    for pc in per_call:
        by_path.setdefault(pc["path"], []).append(pc)
    dom_path = max(by_path, key=lambda p: sum(pc["us_mean"] for pc in by_path[p]))
    dom = by_path[dom_path]
    algo_bytes = sum(pc["algo_bytes"] for pc in dom)
    dur_us = sum(pc["us_mean"] for pc in dom)
    achieved = algo_bytes / dur_us / 1e3
    traffic = measured_traffic(dom_path)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBS, 4),
                "traffic": traffic, "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                "algo_bytes_per_call": round(algo_bytes / len(dom)),
                "kernel": (f"w12_gemm {dom_path} path (M={dom[0]['m']}, gate/up/down), mean of per-call HIP events"
                           + (" (one call = k_xpose + k_mfma)" if dom_path == "mfma" else " (one call = k_gemv)"))}

    cpu = None
    if not args.no_cpu:
        import oracle as o
        sub = [(name, w[: args.cpu_rows] if args.cpu_rows > 0 else w) for name, w in mats_host]
        encs = [o.encode(w) for name, w in sub]
        cpu = cpu_baseline(sub, encs, {m: xs_host[m] for m in ms}, args.cpu_rows, args.cpu_passes)

    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "MLP W12 GEMMs at hidden 5120: gate/up 17408x5120, down 5120x17408; "
                                  f"M in {list(ms)}; fp32 accumulate, BF16 out; {args.copies} rotating copies",
                      "global_batch": list(ms), "seq_len": 1, "parallelism": "none"},
           "pct_peak": round(100 * value / PEAK_GBS, 2),
           "per_call": per_call, "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


def measured_traffic(path):
    """HBM bytes per call of `path` ("gemv" or "mfma") from the committed
    rocprofv3 counter summary, or None when the GEMM sources have changed
    since those counters were taken."""
    import hashlib
    try:
        line = next(l for l in open(TRAFFIC_PROFILE) if l.startswith("traffic_json: "))
        rec = json.loads(line[len("traffic_json: "):])
        h = hashlib.sha256()
        for f in GEMM_SOURCES:
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return int(rec["bytes_per_call"][path])
    except (OSError, StopIteration, KeyError, ValueError):
        return None


def cpu_baseline(sub, encs, xs, rows, passes):
    """The oracle (NumPy decode of the records + float64 matmul) over the
    sample (the first `rows` rows of each matrix, all rows if 0), for each M,
    `passes` times: packed GB/s of that work."""
    import oracle as o
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t_total = 0.0
    bytes_total = 0
    for _ in range(passes):
        for (name, w), enc in zip(sub, encs):
            for m, x in xs.items():
                t0 = time.perf_counter()
                wd = o.decode(enc)
                o.gemm_ref(x[:, : w.shape[1]], wd)
                t_total += time.perf_counter() - t0
                bytes_total += w.shape[0] * w.shape[1] * 3 // 2
    what = "all rows" if rows <= 0 else f"first {rows} rows"
    return {"value": round(bytes_total / t_total / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{what} of gate, up and down at M in {list(xs)}, {passes} passes: oracle decode of the "
                      f"records + float64 matmul ({t_total:.1f} s)"}


if __name__ == "__main__":
    main()
