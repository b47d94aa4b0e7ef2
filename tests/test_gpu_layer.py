"""One decoder layer's linears with fewer launches (SpecPilot Appendix F,
Table A7, where a persistent cross-GEMM W12 kernel was closed as slower; here
the launches are cut instead): q|k|v and gate|up, which share their inputs,
encoded as row concatenations (N = 8192 and N = 34816 at K = 5120), and the
layer's four GEMMs captured in one HIP graph.

W12 encodes every row on its own (window, records of 16 rows, per-row escape
lists; SpecPilot section 4.1), so a row concatenation encodes to the parts'
bytes laid end to end; the fused outputs are checked against the fp64 oracle
of each part."""
import functools

import numpy as np
import pytest
import torch

import synth
from gpu_util import check_bf16, check_bf16_value, check_f32, dev16, download, host16, log, o, w12

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "o", "gate", "up", "down")
GROUPS = {"qkv": ("q", "k", "v"), "o": ("o",), "gate_up": ("gate", "up"), "down": ("down",)}


@functools.lru_cache(maxsize=1)
def _weights():
    return {name: synth.workload_matrix(2, i) for i, name in enumerate(NAMES)}


@functools.lru_cache(maxsize=1)
def _fused():
    w = _weights()
    return {g: w12.encode(dev16(np.concatenate([w[p] for p in parts]))) for g, parts in GROUPS.items()}


def test_row_concatenation_encodes_as_its_parts():
    w = _weights()
    for g, parts in GROUPS.items():
        if len(parts) == 1:
            continue
        log(f"[layer] encode {g} = {'|'.join(parts)}")
        fused = download(_fused()[g])
        sep = [download(w12.encode(dev16(w[p]))) for p in parts]
        assert np.array_equal(fused[0], np.concatenate([s[0] for s in sep]))      # records
        assert np.array_equal(fused[1], np.concatenate([s[1] for s in sep]))      # e_top
        offs = np.cumsum([0] + [int(s[2][-1]) for s in sep[:-1]])
        rp = np.concatenate([sep[0][2][:1]] + [s[2][1:] + np.uint32(off) for s, off in zip(sep, offs)])
        assert np.array_equal(fused[2], rp)                                       # row pointers
        assert np.array_equal(fused[3], np.concatenate([s[3] for s in sep]))      # escapes


def _inputs(m):
    return {k: synth.make_activations(m, k, seed=synth.activation_seed(2, 0, m) + k) for k in (5120, 6144, 17408)}


def _check_group(g, x, y_f32, y_bf16):
    """Each part's columns of a fused output against the oracle of that part
    (y_f32 may be None: then the BF16 output is checked on its own)."""
    w = _weights()
    col = 0
    for p in GROUPS[g]:
        n = w[p].shape[0]
        y64 = o.gemm_ref(x, w[p])
        if y_f32 is not None:
            check_f32(y_f32[:, col:col + n], y64, f"{g}/{p}")
            check_bf16(y_bf16[:, col:col + n], y_f32[:, col:col + n], y64, f"{g}/{p} bf16")
        else:
            check_bf16_value(y_bf16[:, col:col + n], y64, f"{g}/{p} bf16")
        col += n


@pytest.mark.parametrize("m", [4, 16, 32, 64])
def test_fused_layer_matches_oracle(m):
    xs = _inputs(m)
    for g, mat in _fused().items():
        log(f"[layer] {g} {mat.n}x{mat.k} M={m} kernel {w12.plan_info(mat, w12.OP_GEMM, m)['kernel_name']}")
        xd = dev16(xs[mat.k])
        yf = w12.gemm(mat, xd, torch.float32).cpu().numpy()
        yb = host16(w12.gemm(mat, xd, torch.bfloat16))
        _check_group(g, xs[mat.k], yf, yb)


def test_fused_layer_graph_replays():
    """The four GEMMs of the layer captured in one graph: every replay equals
    the eager calls bit for bit and the fp64 oracle within the tolerance."""
    m = 32
    mats = _fused()
    xs = {k: dev16(v) for k, v in _inputs(m).items()}
    ys = {g: torch.empty((m, mat.n), dtype=torch.bfloat16, device="cuda") for g, mat in mats.items()}
    wss = {g: w12.new_workspace(w12.OP_GEMM, mat.n, mat.k, m) for g, mat in mats.items()}

    def layer():
        for g, mat in mats.items():
            w12.w12_gemm(mat, xs[mat.k], ys[g], wss[g])

    layer()
    torch.cuda.synchronize()
    eager = {g: y.clone() for g, y in ys.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    torch.cuda.synchronize()
    for r in range(3):
        for y in ys.values():
            y.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        log(f"[layer graph] replay {r}")
        for g in mats:
            assert torch.equal(ys[g].view(torch.int16), eager[g].view(torch.int16)), f"replay {r}: {g}"
        layer()
        torch.cuda.synchronize()
    xh = _inputs(m)
    for g, mat in mats.items():
        _check_group(g, xh[mat.k], None, host16(ys[g]))
    for g, ws in wss.items():
        assert int(ws[: w12.WS_COUNTER_BYTES].view(torch.int32).abs().sum()) == 0, g
