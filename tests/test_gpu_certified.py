"""Certified argmax LM head against the oracle (SpecPilot section 4.1, the
certified LM head paragraph; section 4.3, zero-copy Q pass).

What is unique is checked exactly: the per-row bounds (float64 sums rounded
up: never below the oracle's value, at most a float step above), and the
argmax index away from near ties, which must equal the oracle's and the full
fused head's. Which rows survive the certificate is not unique (it depends on
the fp32 Q logits); their count must lie between the oracle's survivors
without any rounding allowance and those with twice (plus a hair) the
allowance, which holds whenever the GPU's Q logits are within the allowance
of the exact Q-copy products."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from gpu_util import check_f32, dev16, log, o, w12

pytestmark = pytest.mark.gpu

CHUNK = 2048
THREADS = max(1, min(8, os.cpu_count() or 1))


def _oracle(w: np.ndarray, x: np.ndarray):
    """Chunked oracle: exact logits, Q-copy logits and the per-row bounds."""
    n = w.shape[0]
    y = np.empty((x.shape[0], n))
    yq = np.empty_like(y)
    r = np.empty(n)
    a = np.empty(n)

    def work(c):
        lo, hi = c
        enc = o.encode(w[lo:hi])
        with np.errstate(invalid="ignore", over="ignore"):
            y[:, lo:hi] = o.gemm_ref(x, w[lo:hi])
            yq[:, lo:hi] = o.gemm_ref(x, o.q_view_escapes_bits(enc))
        r[lo:hi], a[lo:hi] = o.certify_bounds(enc)
    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(work, [(i, min(i + CHUNK, n)) for i in range(0, n, CHUNK)]))
    return y, yq, r, a


def _check_bounds(mat, r, a):
    b = w12.certify_bounds(mat).cpu().numpy().astype(np.float64)
    fin = np.isfinite(r)
    assert np.array_equal(np.isinf(b[:, 0]), ~fin) and np.array_equal(np.isinf(b[:, 1]), ~fin)
    for got, want, name in ((b[fin, 0], r[fin], "r"), (b[fin, 1], a[fin], "a")):
        assert np.all(got >= want), f"{name} below the oracle"
        assert np.all(got <= want * (1 + 2.0 ** -21)), f"{name} more than a float step above the oracle"
    return w12.certify_bounds(mat)


def _check_call(mat, bounds, x, y, yq, r, a, what, expect_fallback=False):
    m = x.shape[0]
    xd = dev16(x)
    idx, mx, sv = w12.lmhead_argmax_certified(mat, bounds, xd)
    fidx, fmx = w12.lmhead_argmax(mat, xd)
    idx, mx, sv = idx.cpu().numpy().astype(np.int64), mx.cpu().numpy(), sv.cpu().numpy()
    fidx = fidx.cpu().numpy().astype(np.int64)
    ridx, margin = o.argmax_ref(y)
    far = margin >= 1e-3
    assert np.array_equal(idx[far], ridx[far]), f"{what}: certified argmax differs from the oracle"
    assert np.array_equal(idx[far], fidx[far]), f"{what}: certified argmax differs from the full head"
    best = y[np.arange(m), ridx]
    fin = np.isfinite(best)
    scale = np.maximum(np.abs(best), 1e-3 * np.abs(y).max(axis=1))
    assert np.all(np.abs(mx[far & fin] - best[far & fin]) <= 2e-3 * scale[far & fin]), f"{what}: max logit"
    c = o.certify_slack(mat.k)
    for i in range(m):
        xn = float(np.linalg.norm(o.bf16_to_f64(x[i])))
        lo = len(o.certified_survivors(yq[i], r, a, xn, 0.0))
        hi = len(o.certified_survivors(yq[i], r, a, xn, 2.1 * c))
        assert lo <= sv[i] <= hi, f"{what}: row {i} kept {sv[i]} rows, oracle range [{lo}, {hi}]"
    fell_back = bool((sv > w12.CERT_MAX_SURVIVORS).any())
    assert expect_fallback is None or fell_back == expect_fallback, f"{what}: fallback {fell_back}"
    if fell_back:                      # the full head's answer, bit for bit
        assert np.array_equal(idx, fidx) and np.array_equal(mx.view(np.uint32), fmx.cpu().numpy().view(np.uint32))
    log(f"  {what}: survivors per row {sv.min()}..{sv.max()}, near ties {int((~far).sum())}")
    return sv


def _infinite():
    w = synth.workload_matrix(0, 0).copy()
    w[5, 17] = 0x7F80      # +inf (its logit is +inf: x[:, 17] = 1 below)
    w[300, 900] = 0xFF80   # -inf
    w[700, 100] = 0x7F80   # +inf
    return w


CASES = {
    "config0": lambda: synth.workload_matrix(0, 0),
    "ragged_48": lambda: synth.workload_matrix(0, 0)[:48],
    "stress_rows": lambda: synth.workload_matrix(4, 0, rows=slice(0, 512)),
    "lm_head_rows": lambda: synth.workload_matrix(3, 0, rows=slice(0, 4096)),
    # K = 17408: the norm of x takes several passes of the bound kernel's loads
    "wide_k": lambda: synth.workload_matrix(1, 2, rows=slice(0, 512)),
}


@pytest.mark.parametrize("name", list(CASES.keys()))
def test_certified_head_small(name):
    w = CASES[name]()
    log(f"[certified] {name} {w.shape}")
    ms = (1, 3, 16, 33, 64)
    xs = [synth.make_activations(m, w.shape[1], seed=900 + m) for m in ms]
    y, yq, r, a = _oracle(w, np.concatenate(xs))
    mat = w12.encode(dev16(w))
    bounds = _check_bounds(mat, r, a)
    row = 0
    for m, x in zip(ms, xs):
        _check_call(mat, bounds, x, y[row:row + m], yq[row:row + m], r, a, f"{name} M={m}", expect_fallback=None)
        row += m


def test_certified_bounds_of_nan_rows():
    w = synth.workload_matrix(0, 0)[:64].copy()
    w[3, 9] = 0x7FC1       # NaN
    w[40, 0] = 0xFFC0      # NaN, sign bit set
    _, _, r, a = _oracle(w, synth.make_activations(1, 1024, seed=1))
    assert np.isinf(r[[3, 40]]).all() and np.isfinite(np.delete(r, [3, 40])).all()
    _check_bounds(w12.encode(dev16(w)), r, a)


def test_certified_head_infinite_rows():
    """Rows holding inf can never be ruled out (infinite bound); the answer
    equals the full head's: the lowest row with a +inf logit."""
    w = _infinite()
    x = synth.make_activations(8, 1024, seed=8)
    x[:, 17] = 0x3F80
    y, yq, r, a = _oracle(w, x)
    assert np.isinf(r[[5, 300, 700]]).all()
    mat = w12.encode(dev16(w))
    bounds = _check_bounds(mat, r, a)
    idx, mx, sv = w12.lmhead_argmax_certified(mat, bounds, dev16(x))
    fidx, fmx = w12.lmhead_argmax(mat, dev16(x))
    assert idx.cpu().numpy().tolist() == [5] * 8 and torch.equal(idx, fidx)
    assert np.all(np.isposinf(mx.cpu().numpy())) and np.all(np.isposinf(fmx.cpu().numpy()))
    assert int(sv.min()) >= 3                       # the three infinite rows always survive


@pytest.mark.parametrize("m", [4, 20])
def test_certified_head_falls_back_when_too_many_survive(m):
    """Identical rows: every logit ties, every row survives (1024 > cap), so
    the full head runs (the fused argmax up to 16 activation rows, the
    two-pass one beyond) and the lowest index wins; then a normal call on the
    same workspace is certified again (the state was cleared)."""
    base = synth.workload_matrix(0, 0)
    w = np.tile(base[7:8], (1024, 1))
    x = synth.make_activations(m, 1024, seed=5)
    y, yq, r, a = _oracle(w, x)
    mat = w12.encode(dev16(w))
    bounds = _check_bounds(mat, r, a)
    ws = w12.new_workspace(w12.OP_LMHEAD_CERTIFIED, 1024, 1024, m)
    idx = torch.empty(m, dtype=torch.int32, device="cuda")
    mx = torch.empty(m, dtype=torch.float32, device="cuda")
    sv = torch.empty(m, dtype=torch.int32, device="cuda")
    for rep in range(2):
        w12.w12_lmhead_argmax_certified(mat, bounds, dev16(x), idx, mx, sv, ws)
        assert idx.cpu().numpy().tolist() == [0] * m
        assert sv.cpu().numpy().tolist() == [1024] * m
        # the maximum is the tied logit itself, within the oracle's tolerance
        check_f32(mx.cpu().numpy()[:, None], y[:, :1], f"fallback M={m} max")
    mat2 = w12.encode(dev16(base))
    y2, yq2, r2, a2 = _oracle(base, x)
    b2 = w12.certify_bounds(mat2)
    w12.w12_lmhead_argmax_certified(mat2, b2, dev16(x), idx, mx, sv, ws)
    ridx, margin = o.argmax_ref(y2)
    far = margin >= 1e-3
    assert np.array_equal(idx.cpu().numpy()[far], ridx[far])
    assert int(sv.max()) <= w12.CERT_MAX_SURVIVORS


LM_MS = (1, 16, 32)


@pytest.fixture(scope="module")
def lm_head():
    """The LM head workload 151936 x 5120: encoded once, with the oracle's
    logits, Q-copy logits and bounds for M = 1, 16, 32 computed in one pass."""
    w = synth.workload_matrix(3, 0)
    xs = {m: synth.make_activations(m, 5120, seed=synth.activation_seed(3, 0, m)) for m in LM_MS}
    log("[certified] lm head 151936x5120: oracle")
    y, yq, r, a = _oracle(w, np.concatenate([xs[m] for m in LM_MS]))
    mat = w12.encode(dev16(w))
    del w
    bounds = _check_bounds(mat, r, a)
    out, row = {}, 0
    for m in LM_MS:
        out[m] = (xs[m], y[row:row + m], yq[row:row + m])
        row += m
    return mat, bounds, r, a, out


@pytest.mark.parametrize("m", LM_MS)
def test_certified_lm_head_151936_full(lm_head, m):
    mat, bounds, r, a, data = lm_head
    x, y, yq = data[m]
    _check_call(mat, bounds, x, y, yq, r, a, f"lm head M={m}")


def test_certified_workspace_reused_across_sizes():
    """One workspace, sized for the largest call, serves calls of different M
    in any order: the state that accumulates sits at a fixed place and every
    call leaves it clear."""
    w = synth.workload_matrix(3, 0, rows=slice(0, 4096))
    mat = w12.encode(dev16(w))
    bounds = w12.certify_bounds(mat)
    ws = w12.new_workspace(w12.OP_LMHEAD_CERTIFIED, 4096, 5120, 64)
    for m in (33, 3, 64, 1, 17, 64):
        x = synth.make_activations(m, 5120, seed=1300 + m)
        idx = torch.empty(m, dtype=torch.int32, device="cuda")
        mx = torch.empty(m, dtype=torch.float32, device="cuda")
        w12.w12_lmhead_argmax_certified(mat, bounds, dev16(x), idx, mx, None, ws)
        ridx, margin = o.argmax_ref(o.gemm_ref(x, w))
        far = margin >= 1e-3
        assert np.array_equal(idx.cpu().numpy()[far], ridx[far]), f"M={m}"
    assert int(ws[: w12.WS_COUNTER_BYTES].view(torch.int32).abs().sum()) == 0
