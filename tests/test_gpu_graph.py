"""The GEMM entry points under HIP graph capture.

A call allocates nothing, issues no memset and leaves its workspace counters
at zero, so a captured sequence of calls replays like the eager calls. Each
replay is checked against the eager results bit for bit, with eager calls and
synchronizations between the replays."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev16, log, w12

pytestmark = pytest.mark.gpu


def test_captured_calls_replay_like_eager_calls():
    w = synth.workload_matrix(0, 0)                      # 1024 x 1024
    mat = w12.encode(dev16(w))
    n, k = w.shape
    cases = []
    for m in (1, 5, 32):
        x = dev16(synth.make_activations(m, k, seed=300 + m))
        cases.append(dict(
            m=m, x=x,
            y=torch.empty((m, n), dtype=torch.float32, device="cuda"),
            yq=torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
            idx=torch.empty(m, dtype=torch.int32, device="cuda"),
            mx=torch.empty(m, dtype=torch.float32, device="cuda"),
            ws=w12.new_workspace(w12.OP_GEMM, n, k, m),
            wsq=w12.new_workspace(w12.OP_GEMM_Q8, n, k, m),
            wsa=w12.new_workspace(w12.OP_LMHEAD_ARGMAX, n, k, m)))

    def calls():
        for c in cases:
            w12.w12_gemm(mat, c["x"], c["y"], c["ws"])
            w12.w12_gemm_q8(mat, c["x"], c["yq"], w12.Q8_APPLY_ESCAPES, c["wsq"])
            w12.w12_lmhead_argmax(mat, c["x"], c["idx"], c["mx"], c["wsa"])

    def outputs():
        return [t.clone() for c in cases for t in (c["y"], c["yq"], c["idx"], c["mx"])]

    calls()
    torch.cuda.synchronize()
    eager = outputs()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    for r in range(3):
        for c in cases:                                   # stale values must not survive a replay
            for key in ("y", "yq", "idx", "mx"):
                c[key].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"[graph] replay {r}")
        for a, b in zip(outputs(), eager):
            assert torch.equal(a, b), f"replay {r} differs from the eager calls"
        calls()                                           # eager work between replays
        torch.cuda.synchronize()
    for c in cases:
        for key in ("ws", "wsq", "wsa"):
            counters = c[key][: w12.WS_COUNTER_BYTES].view(torch.int32)
            assert int(counters.abs().sum()) == 0, f"{key} counters not back at zero (M={c['m']})"
    assert np.isfinite(eager[0].cpu().numpy()).all()
