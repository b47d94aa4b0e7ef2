"""W12 GEMM benchmark on one MI355X.

Workload (one step, the metric's own): the MLP GEMMs at hidden size 5120 -
gate and up (17408 x 5120) and down (5120 x 17408) - as exact W12 GEMMs with
fp32 accumulation and BF16 output, at M = 1 and M = 32 activation rows: six
GEMM calls per step. Weights are synthetic per-output-channel Gaussians
(per-row lognormal scales, 1e-4 outliers x 2^12, 1e-4 zeros), encoded on the
GPU before timing; activations are BF16 N(0, 1). Every input is resident in
HBM before the timed region. Each call reads the next of R encoded copies of
its matrix (R * 134 MB at least twice the 256 MB last-level cache), so
weights stream from HBM, as in the pages' cold-L2 measurements.

Prints one JSON line:
  value          packed W12 bytes (1.5 B per weight) per second over the whole step
  per_call       each (matrix, M): microseconds per call, measured over calls of
                 that shape issued back to back between one pair of HIP events
                 (each call on the next copy), and the kernel the library ran
  roofline       the kernel taking the most time per step: algorithmic bytes per
                 call / its per-call time, against 8 TB/s; traffic = measured
                 HBM bytes per call from the committed counter profile
  roofline_by_kernel   the same for every kernel the step runs
  probe          a plain 16-byte read of 134 MB (the same load the kernels use),
                 best of a few launch shapes: the read ceiling on this device
  workloads      the other workloads of the pages' configs, timed the same way
  cpu_baseline   the oracle (NumPy decode + float64 matmul) on the host cores
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W12 GEMM achieved HBM GB/s (% of peak) and µs/call at M=1 and M=32"
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "w12_gemm_mlp5120_pmc_traffic.md")
GEMM_SOURCES = ["lossless_compressed_weight_amd/csrc/w12_gemm.hip",
                "lossless_compressed_weight_amd/csrc/w12_gemm_mx.hip",
                "lossless_compressed_weight_amd/csrc/w12_api.hip",
                "lossless_compressed_weight_amd/csrc/w12_internal.h"]
PEAK_GBS = 8000.0
MS = (1, 32)
COPIES = 5

PROBE_REGION = 17408 * 5120 * 3 // 2   # bytes of one packed 17408 x 5120 W12 matrix
PROBE_REGIONS = 16                     # 2.1 GB rotated, far above the 256 MB last-level cache
# (mode, block, grid, loads, piece bytes): the best launch shapes of the probe sweep
PROBE_SHAPES = [(2, 512, 1024, 1, 0), (3, 256, 512, 4, 16384), (3, 512, 256, 4, 32768), (2, 1024, 256, 2, 0)]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copies", type=int, default=COPIES, help="encoded copies of each matrix to rotate through")
    ap.add_argument("--cpu-rows", type=int, default=2048, help="rows of each matrix in the CPU oracle sample")
    ap.add_argument("--cpu-passes", type=int, default=2, help="passes of the oracle over its sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the other configs' workloads")
    ap.add_argument("--ms", type=str, default=None, help="comma-separated M values (default 1,32)")
    ap.add_argument("--cpu-only", type=int, default=0, help="(internal) print the CPU oracle baseline with N threads")
    ap.add_argument("--probe-sweep", type=str, default=None,
                    help="run only the read-bandwidth probe over its parameter grid; JSON lines to this file")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers
def copies_of(w12, mat, r):
    return [mat] + [w12.W12Matrix(mat.n, mat.k, mat.records.clone(), mat.e_top.clone(), mat.row_ptr.clone(),
                                  mat.esc.clone(), mat.n_esc) for _ in range(r - 1)]


def algo_bytes(mat, m, argmax=False):
    """Bytes a call must move: packed records, e_top, row pointers, escapes,
    activations, and outputs (BF16 y, or M (index, value) pairs for the argmax)."""
    return (mat.n * mat.k * 3 // 2 + mat.n + 4 * (mat.n + 1) + 8 * mat.n_esc + 2 * m * mat.k
            + (8 * m if argmax else 2 * m * mat.n))


def back_to_back_us(torch, stream, call, n, warm=3):
    """Microseconds per call of `call(i)` for i = 0 .. n-1 issued back to back
    between one pair of HIP events on the launch stream."""
    for i in range(warm):
        call(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(n):
        call(warm + i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def measured_traffic():
    """HBM bytes per call of each kernel class from the committed rocprofv3
    counter summary, or None when the GEMM sources changed since."""
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
        return rec["bytes_per_call"]
    except (OSError, StopIteration, KeyError, ValueError):
        return None


def gemm_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# ------------------------------------------------------------------ probe
def probe_time(w12, buf, nbytes, grid, block, loads, mode, ws, stream, reps=12, warm=2, stamps=None, piece=0):
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
                           stream, piece=piece)
        if i >= warm:
            ev[i - warm][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def probe_ceiling(torch, w12, dev, stream):
    """Best per-launch time of the read probe on 134 MB over a few launch
    shapes, back to back with one event pair (as the GEMM calls are timed)."""
    buf = torch.zeros(PROBE_REGION * PROBE_REGIONS, dtype=torch.uint8, device=dev)
    ws = torch.zeros(w12.PROBE_WS_BYTES, dtype=torch.uint8, device=dev)
    best = None
    for mode, block, grid, loads, piece in PROBE_SHAPES:
        def call(i):
            w12.w12_probe_read(buf[(i % PROBE_REGIONS) * PROBE_REGION:], PROBE_REGION, grid, block, loads, mode,
                               None, ws, stream, piece=piece)
        us = back_to_back_us(torch, stream, call, 32)
        if best is None or us < best[0]:
            best = (us, {"mode": ["static", "dynamic", "stride", "pieces"][mode], "block": block, "grid": grid,
                         "loads": loads, "piece": piece})
    del buf
    us, shape = best
    return {"us_per_read": round(us, 3), "bytes": PROBE_REGION, "gbs": round(PROBE_REGION / us / 1e3, 1),
            "pct_peak": round(100 * PROBE_REGION / us / 1e3 / PEAK_GBS, 2), "shape": shape}


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
    for mode in (w12.PROBE_STATIC, w12.PROBE_DYNAMIC, w12.PROBE_STRIDE, w12.PROBE_PIECES):
        for block in (256, 512, 1024):
            for wgpc in (1, 2, 4):
                for loads in (1, 2, 4, 8):
                    piece = 32768 if mode == w12.PROBE_PIECES else 0
                    t = probe_time(w12, buf, PROBE_REGION, 256 * wgpc, block, loads, mode, ws, stream, piece=piece)
                    med = float(np.median(t))
                    rec = {"mode": mode, "block": block, "wg_per_cu": wgpc, "loads": loads, "piece": piece,
                           "us_median": round(med, 3), "us_min": round(min(t), 3),
                           "gbs": round(PROBE_REGION / med / 1e3, 1)}
                    out.write(json.dumps(rec) + "\n")
                    out.flush()
                    if best is None or med < best[0]:
                        best = (med, rec)
    print(f"# probe best on 134 MB: {best[1]}", file=sys.stderr, flush=True)
    b = best[1]
    for mode in (w12.PROBE_STATIC, w12.PROBE_STRIDE, w12.PROBE_PIECES):
        grid = 256 * b["wg_per_cu"]
        st = torch.zeros(3 * grid, dtype=torch.int64, device=dev)
        t = probe_time(w12, buf, PROBE_REGION, grid, b["block"], b["loads"], mode, ws, stream, stamps=st,
                       piece=32768)
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
    big = 151936 * 5120 * 3 // 2
    big -= big % 16
    for mode in (w12.PROBE_STATIC, w12.PROBE_STRIDE):
        t = probe_time(w12, buf, big, 256 * b["wg_per_cu"], b["block"], b["loads"], mode, ws, stream, reps=4)
        rec = {"lm_head_bytes": big, "mode": mode, "us_median": round(float(np.median(t)), 3),
               "gbs": round(big / float(np.median(t)) / 1e3, 1)}
        out.write(json.dumps(rec) + "\n")
    out.close()


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline_run(rows, passes):
    """The oracle (NumPy decode of the records + float64 matmul) over the first
    `rows` rows of gate, up and down at M = 1 and 32, `passes` times: packed
    GB/s of that work, and the BLAS threads it used."""
    import oracle as o
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    sub = [synth.workload_matrix(1, i, rows=slice(0, rows)) for i in range(3)]
    encs = [o.encode(w) for w in sub]
    xs = {m: synth.make_activations(m, 17408, seed=synth.activation_seed(1, 0, m)) for m in MS}
    t_total, nbytes = 0.0, 0
    for _ in range(passes):
        for w, enc in zip(sub, encs):
            for m, x in xs.items():
                t0 = time.perf_counter()
                wd = o.decode(enc)
                o.gemm_ref(x[:, : w.shape[1]], wd)
                t_total += time.perf_counter() - t0
                nbytes += w.shape[0] * w.shape[1] * 3 // 2
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} rows of gate, up and down at M in {list(MS)}, {passes} passes: oracle decode "
                      f"of the records + float64 matmul ({t_total:.1f} s)"}


def cpu_baseline(rows, passes):
    """All host cores in this process; one thread in a child process (BLAS
    thread count fixed before NumPy loads)."""
    allc = cpu_baseline_run(rows, passes)
    allc["os_cpu_count"] = os.cpu_count()
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--cpu-only", "1", "--cpu-rows",
                            str(rows), "--cpu-passes", "1"], env=env, capture_output=True, text=True, timeout=600)
        allc["single_thread"] = json.loads(r.stdout.strip().splitlines()[-1])
    except (subprocess.SubprocessError, ValueError, IndexError) as e:  # pragma: no cover
        allc["single_thread"] = {"error": str(e)}
    return allc


# ------------------------------------------------------------------ workloads
def time_shape(torch, w12, stream, mats, x, y, ws, reps, op="gemm", q_flags=0):
    """us per call of one shape, back to back, each call on the next copy."""
    if op == "gemm":
        call = lambda i: w12.w12_gemm(mats[i % len(mats)], x, y, ws, stream)
    elif op == "q8":
        call = lambda i: w12.w12_gemm_q8(mats[i % len(mats)], x, y, q_flags, ws, stream)
    else:
        call = lambda i: w12.w12_lmhead_argmax(mats[i % len(mats)], x, y[0], y[1], ws, stream)
    return back_to_back_us(torch, stream, call, reps)


def workloads(torch, w12, synth, dev, stream, reps):
    """The other configs (parity-test workloads), each call timed back to back."""
    out = {}
    # config 0: one 1024 x 1024 matrix, M = 1 (L2-resident and launch-bound)
    w = synth.workload_matrix(0, 0)
    mats = copies_of(w12, w12.encode(torch.from_numpy(w.view(np.int16)).to(dev)), 4)
    x = torch.from_numpy(synth.make_activations(1, 1024, seed=synth.activation_seed(0, 0, 1)).view(np.int16)).to(dev)
    y = torch.empty((1, 1024), dtype=torch.bfloat16, device=dev)
    ws = w12.new_workspace(w12.OP_GEMM, 1024, 1024, 1, dev)
    us = time_shape(torch, w12, stream, mats, x, y, ws, 64)
    out["config0_1024x1024_m1"] = {"us": round(us, 3), "kernel": w12.plan_info(mats[0], w12.OP_GEMM, 1)["kernel_name"],
                                   "note": "1.6 MB stays in L2; launch-bound"}
    del mats
    # config 2: one decoder layer's seven GEMMs back to back at M = 32 and 64
    wl = synth.WORKLOADS[2]
    layer, wts = [], {}
    for i, spec in enumerate(wl.matrices):
        wts[spec.name] = torch.from_numpy(synth.workload_matrix(2, i).view(np.int16)).to(dev)
        layer.append(copies_of(w12, w12.encode(wts[spec.name]), 3))
    packed = sum(c[0].n * c[0].k * 3 // 2 for c in layer)
    for m in (32, 64):
        xs = {k: torch.from_numpy(synth.make_activations(m, k, seed=synth.activation_seed(2, 0, m)).view(np.int16)).to(dev)
              for k in (5120, 6144, 17408)}
        ys = [torch.empty((m, c[0].n), dtype=torch.bfloat16, device=dev) for c in layer]
        wss = [w12.new_workspace(w12.OP_GEMM, c[0].n, c[0].k, m, dev) for c in layer]
        per = {}
        for li, (spec, c) in enumerate(zip(wl.matrices, layer)):
            us = time_shape(torch, w12, stream, c, xs[c[0].k], ys[li], wss[li], reps)
            per[spec.name] = {"us": round(us, 2), "kernel": w12.plan_info(c[0], w12.OP_GEMM, m)["kernel_name"]}

        def step(r):
            for li, c in enumerate(layer):
                w12.w12_gemm(c[r % len(c)], xs[c[0].k], ys[li], wss[li], stream)
        lay = back_to_back_us(torch, stream, step, reps)
        out[f"config2_layer_m{m}"] = {"layer_us": round(lay, 1), "packed_gbs": round(packed / lay / 1e3, 1),
                                      "pct_peak": round(100 * packed / lay / 1e3 / PEAK_GBS, 2), "per_gemm": per}
    del layer
    out.update(fused_layer(torch, w12, synth, dev, stream, reps, wts, packed))
    del wts
    # config 3: LM head fused with the argmax at M = 1, 16, 32
    w = synth.workload_matrix(3, 0)
    mat = w12.encode(torch.from_numpy(w.view(np.int16)).to(dev))
    del w
    mats = copies_of(w12, mat, 2)
    bounds = [w12.certify_bounds(c) for c in mats]
    packed = mat.n * mat.k * 3 // 2
    for m in (1, 16, 32):
        x = torch.from_numpy(synth.make_activations(m, 5120, seed=synth.activation_seed(3, 0, m)).view(np.int16)).to(dev)
        idx = torch.empty(m, dtype=torch.int32, device=dev)
        mx = torch.empty(m, dtype=torch.float32, device=dev)
        ws = w12.new_workspace(w12.OP_LMHEAD_ARGMAX, mat.n, mat.k, m, dev)
        us = time_shape(torch, w12, stream, mats, x, (idx, mx), ws, max(4, reps // 3), op="argmax")
        out[f"config3_lmhead_argmax_m{m}"] = {
            "us": round(us, 2), "packed_gbs": round(packed / us / 1e3, 1),
            "pct_peak": round(100 * packed / us / 1e3 / PEAK_GBS, 2),
            "kernel": w12.plan_info(mat, w12.OP_LMHEAD_ARGMAX, m)["kernel_name"]}
        # the certified head on the same inputs: Q pass + bounds + rescoring
        sv = torch.empty(m, dtype=torch.int32, device=dev)
        wsc = w12.new_workspace(w12.OP_LMHEAD_CERTIFIED, mat.n, mat.k, m, dev)
        uc = back_to_back_us(torch, stream, lambda i: w12.w12_lmhead_argmax_certified(
            mats[i % len(mats)], bounds[i % len(mats)], x, idx, mx, sv, wsc, stream), max(4, reps // 3))
        cidx = idx.clone()
        w12.w12_lmhead_argmax(mat, x, idx, mx, ws, stream)
        out[f"config3_lmhead_certified_m{m}"] = {
            "us": round(uc, 2), "speedup_vs_fused_head": round(us / uc, 3),
            "survivors_max": int(sv.max()), "fallback": bool(int(sv.max()) > w12.CERT_MAX_SURVIVORS),
            "same_indices_as_fused_head": bool(torch.equal(cidx, idx))}
    del mats, mat, bounds
    # config 4: escape stress, exact GEMM and the two Q sources at M = 32; the
    # same Q sources on the normal gate matrix of config 1 for comparison
    for wl_i, i, tag in [(4, j, f"config4_{spec.name}_m32") for j, spec in enumerate(synth.WORKLOADS[4].matrices)] + \
            [(1, 0, "config1_gate_q_sources_m32")]:
        spec = synth.WORKLOADS[wl_i].matrices[i]
        wi = synth.workload_matrix(wl_i, i)
        mat = w12.encode(torch.from_numpy(wi.view(np.int16)).to(dev))
        del wi
        mats = copies_of(w12, mat, 4)
        x = torch.from_numpy(synth.make_activations(32, spec.k, seed=synth.activation_seed(wl_i, i, 32))
                             .view(np.int16)).to(dev)
        y = torch.empty((32, spec.n), dtype=torch.bfloat16, device=dev)
        ws = w12.new_workspace(w12.OP_GEMM, spec.n, spec.k, 32, dev)
        ue = time_shape(torch, w12, stream, mats, x, y, ws, max(4, reps // 2))
        uq = time_shape(torch, w12, stream, mats, x, y, ws, reps, op="q8")
        uqe = time_shape(torch, w12, stream, mats, x, y, ws, max(4, reps // 2), op="q8", q_flags=w12.Q8_APPLY_ESCAPES)
        out[tag] = {"n": spec.n, "k": spec.k, "n_esc": mat.n_esc,
                    "exact_us": round(ue, 2), "exact_kernel": w12.plan_info(mat, w12.OP_GEMM, 32)["kernel_name"],
                    "exact_fixup_kernel": bool(w12.plan_info(mat, w12.OP_GEMM, 32)["fixup"]),
                    "q_view_us": round(uq, 2), "q_view_gbs": round(spec.n * spec.k / uq / 1e3, 1),
                    "q_view_escapes_us": round(uqe, 2),
                    "q_kernel": w12.plan_info(mat, w12.OP_GEMM_Q8, 32)["kernel_name"]}
        out[tag].update(q_source_agreement(torch, w12, mat, x))
        del mats, mat
    return out


def fused_layer(torch, w12, synth, dev, stream, reps, wts, packed):
    """The same layer with q|k|v and gate|up encoded as row concatenations
    (four GEMMs instead of seven), issued eagerly and replayed as one HIP graph
    per weight copy."""
    groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    fused = [copies_of(w12, w12.encode(torch.cat([wts[p] for p in g])), 3) for g in groups]
    out = {}
    for m in (32, 64):
        xs = {k: torch.from_numpy(synth.make_activations(m, k, seed=synth.activation_seed(2, 0, m)).view(np.int16)).to(dev)
              for k in (5120, 6144, 17408)}
        ys = [torch.empty((m, c[0].n), dtype=torch.bfloat16, device=dev) for c in fused]
        wss = [w12.new_workspace(w12.OP_GEMM, c[0].n, c[0].k, m, dev) for c in fused]
        per = {}
        for gi, (g, c) in enumerate(zip(groups, fused)):
            us = time_shape(torch, w12, stream, c, xs[c[0].k], ys[gi], wss[gi], reps)
            per["|".join(g)] = {"us": round(us, 2), "kernel": w12.plan_info(c[0], w12.OP_GEMM, m)["kernel_name"]}

        def layer(r, st=stream):
            for gi, c in enumerate(fused):
                w12.w12_gemm(c[r % len(c)], xs[c[0].k], ys[gi], wss[gi], st)
        eager = back_to_back_us(torch, stream, layer, reps)
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            layer(0, side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        for r in range(3):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layer(r, torch.cuda.current_stream())
            graphs.append(g)
        torch.cuda.synchronize()
        graph_us = back_to_back_us(torch, stream, lambda r: graphs[r % 3].replay(), reps)
        out[f"config2_fused_layer_m{m}"] = {
            "gemms": 4, "layer_us": round(eager, 1), "packed_gbs": round(packed / eager / 1e3, 1),
            "graph_layer_us": round(graph_us, 1), "graph_packed_gbs": round(packed / graph_us / 1e3, 1),
            "graph_pct_peak": round(100 * packed / graph_us / 1e3 / PEAK_GBS, 2), "per_gemm": per}
        del graphs
    return out


def q_source_agreement(torch, w12, mat, x):
    """Per activation row, does the argmax over the N outputs of a Q source
    equal that of the exact GEMM? For the 8-bit view alone and the view with
    the escapes applied, beside the bytes each source reads per call."""
    m, n, k = x.shape[0], mat.n, mat.k
    ye = w12.gemm(mat, x, torch.float32).argmax(dim=1)
    yq = w12.gemm_q8(mat, x, torch.float32).argmax(dim=1)
    yqe = w12.gemm_q8(mat, x, torch.float32, apply_escapes=True).argmax(dim=1)
    act = 2 * m * k + 2 * m * n
    return {"agree_q_view": round(float((yq == ye).float().mean()), 4),
            "agree_q_view_escapes": round(float((yqe == ye).float().mean()), 4),
            "bytes_exact": algo_bytes(mat, m), "bytes_q_view": n * k + n + act,
            "bytes_q_view_escapes": n * k + n + 4 * (n + 1) + 8 * mat.n_esc + act}


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.cpu_only:
        print(json.dumps(cpu_baseline_run(args.cpu_rows, args.cpu_passes)), flush=True)
        return
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
    stream = torch.cuda.current_stream()
    wl = synth.WORKLOADS[1]
    t0 = time.time()
    encoded, names = [], []
    for i, spec in enumerate(wl.matrices):
        w = synth.workload_matrix(1, i)
        mat = w12.encode(torch.from_numpy(w.view(np.int16)).to(dev))
        encoded.append(copies_of(w12, mat, args.copies))
        names.append(spec.name)
        del w
    torch.cuda.synchronize()
    print(f"# config 1 generated and encoded ({args.copies} copies) in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)

    calls = []     # (m, matrix index, x, y, ws)
    for m in ms:
        for i, copies in enumerate(encoded):
            n, k = copies[0].n, copies[0].k
            x = torch.from_numpy(synth.make_activations(m, k, seed=synth.activation_seed(1, i, m)).view(np.int16)).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            ws = w12.new_workspace(w12.OP_GEMM, n, k, m, dev)
            calls.append((m, i, x, y, ws))
    uses = [0] * len(encoded)

    def run_step(_):
        for m, i, x, y, ws in calls:
            c = encoded[i]
            w12.w12_gemm(c[uses[i] % len(c)], x, y, ws, stream)
            uses[i] += 1

    # timed region: K steps back to back (the whole-step figure)
    for s in range(args.warmup):
        run_step(s)
    ms_per_step = back_to_back_us(torch, stream, run_step, args.steps, warm=0) / 1e3
    packed_step = sum(encoded[i][0].n * encoded[i][0].k * 3 // 2 for _, i, _, _, _ in calls)
    value = packed_step / (ms_per_step * 1e-3) / 1e9

    # per call: each shape back to back (each call on the next copy)
    per_call = []
    for m, i, x, y, ws in calls:
        c = encoded[i]
        us = time_shape(torch, w12, stream, c, x, y, ws, max(args.steps, 10))
        plan = w12.plan_info(c[0], w12.OP_GEMM, m)
        packed = c[0].n * c[0].k * 3 // 2
        per_call.append({"m": m, "matrix": names[i], "n": c[0].n, "k": c[0].k, "us": round(us, 3),
                         "packed_gbs": round(packed / us / 1e3, 1),
                         "pct_peak_packed": round(100 * packed / us / 1e3 / PEAK_GBS, 2),
                         "algo_bytes": algo_bytes(c[0], m), "n_esc": c[0].n_esc,
                         "kernel": plan["kernel_name"], "grid": plan["grid"], "prepass": plan["prepass"]})

    probe = probe_ceiling(torch, w12, dev, stream)
    for pc in per_call:
        pc["pct_probe"] = round(100 * probe["us_per_read"] / pc["us"] * (pc["n"] * pc["k"] * 3 // 2) / probe["bytes"],
                                2)

    # roofline: every kernel class of the step, and the one taking the most time
    traffic = measured_traffic()
    by_kernel = {}
    for pc in per_call:
        by_kernel.setdefault(pc["kernel"], []).append(pc)
    rl_all = []
    for kern, pcs in by_kernel.items():
        algo = sum(pc["algo_bytes"] for pc in pcs)
        dur = sum(pc["us"] for pc in pcs)
        achieved = algo / dur / 1e3
        rl_all.append({"bound": "hbm", "kernel": kern, "achieved": round(achieved, 1), "peak": PEAK_GBS,
                       "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                       "frac_of_probe": round(achieved / probe["gbs"], 4),
                       "traffic": (int(traffic[kern]) if traffic and kern in traffic else None),
                       "algo_bytes_per_call": round(algo / len(pcs)), "us_per_call": round(dur / len(pcs), 3),
                       "calls": [f"{pc['matrix']} M={pc['m']}" for pc in pcs],
                       "prepass_in_call": bool(pcs[0]["prepass"])})
    dom = max(rl_all, key=lambda r: r["us_per_call"] * len(r["calls"]))
    roofline = {k: dom[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roofline.update({"kernel": dom["kernel"], "frac_of_probe": dom["frac_of_probe"],
                     "algo_bytes_per_call": dom["algo_bytes_per_call"], "us_per_call": dom["us_per_call"],
                     "calls": dom["calls"], "prepass_in_call": dom["prepass_in_call"],
                     "timing": "per-call time = back-to-back calls between one HIP event pair on the launch stream",
                     "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)"})

    # M scan (SpecPilot Appendix E: W12 time flat in the activation rows): gate and down of config 1
    # at every M the library takes, each with the kernel the library chooses
    m_scan = None
    if not args.no_workloads:
        m_scan = []
        for i in (0, 2):
            c = encoded[i]
            n, k = c[0].n, c[0].k
            for m in (1, 2, 3, 4, 8, 16, 24, 32, 48, 64):
                x = torch.from_numpy(synth.make_activations(m, k, seed=synth.activation_seed(1, i, m)).view(np.int16)).to(dev)
                y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                ws = w12.new_workspace(w12.OP_GEMM, n, k, m, dev)
                us = time_shape(torch, w12, stream, c, x, y, ws, max(args.steps, 10))
                plan = w12.plan_info(c[0], w12.OP_GEMM, m)
                m_scan.append({"matrix": names[i], "m": m, "us": round(us, 2),
                               "packed_gbs": round(n * k * 3 // 2 / us / 1e3, 1), "kernel": plan["kernel_name"],
                               "prepass": plan["prepass"]})

    extra = None
    if not args.no_workloads:
        del encoded
        torch.cuda.empty_cache()
        t1 = time.time()
        extra = workloads(torch, w12, synth, dev, stream, max(args.steps, 9))
        print(f"# other workloads in {time.time() - t1:.1f}s", file=sys.stderr, flush=True)

    cpu = None if args.no_cpu else cpu_baseline(args.cpu_rows, args.cpu_passes)

    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "MLP W12 GEMMs at hidden 5120: gate/up 17408x5120, down 5120x17408; "
                                  f"M in {list(ms)}; fp32 accumulate, BF16 out; {args.copies} rotating copies",
                      "global_batch": list(ms), "seq_len": 1, "parallelism": "none"},
           "pct_peak": round(100 * value / PEAK_GBS, 2),
           "per_call": per_call, "roofline": roofline, "roofline_by_kernel": rl_all, "probe": probe,
           "m_scan": m_scan, "workloads": extra, "cpu_baseline": cpu, "gemm_sources_sha256": gemm_sources_sha256()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
