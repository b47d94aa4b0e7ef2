"""The MFMA stream kernel (W12_KERNEL_MFMA_STREAM) against the oracle.

SpecPilot section 4.1 / Figure 5b: the exact W12 GEMM, escapes restoring the
exact weights, the reduction over K split in a fixed order. In this kernel the
escapes' exact BF16 values are substituted into the decoded weights before the
MFMA; entries beyond a wave's list capacity are corrected after the stream.
Every case here forces the kernel (test hook W12_TUNE_PATH = 3), so it runs
on matrices the library would send elsewhere too (dense escapes, M <= 2).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import check_bf16, check_f32, dev16, gemm_both, log, o, w12

pytestmark = pytest.mark.gpu

STREAM = 3


@pytest.fixture(autouse=True)
def _force_stream():
    w12.set_tuning(w12.TUNE_PATH, STREAM)
    yield
    w12.set_tuning(w12.TUNE_PATH, 0)
    w12.set_tuning(w12.TUNE_GRID, 0)


def _skewed():
    """Sparse overall (about 1.4 escapes per row) but with one 64-row tile
    whose rows are a quarter escapes: that tile's waves overflow their
    substitution lists."""
    w = synth.workload_matrix(1, 0, rows=slice(0, 1024)).copy()
    rng = np.random.default_rng(77)
    hit = rng.random((64, w.shape[1])) < 0.25
    blk = w[256:320]
    blk[hit] = (blk[hit].astype(np.uint32) + (20 << 7)).astype(np.uint16)   # exponent + 20: far above the window
    w[256:320] = blk
    return w


def _finite_patterns():
    w = synth.all_bf16_patterns(512).reshape(-1, 1024)
    w = w[np.isfinite(o.bf16_to_f64(w)).all(axis=1)]
    return w[: (w.shape[0] // 16) * 16]


def _mats():
    return {
        "config0": synth.workload_matrix(0, 0),                          # 1024 x 1024
        "ragged_rows": synth.workload_matrix(0, 0)[:48],                  # one tile of three 16-row blocks
        "single_record": synth.workload_matrix(0, 0)[:16, :512],
        "wide_k": synth.workload_matrix(1, 2, rows=slice(0, 256)),       # 256 x 17408
        "stress": synth.workload_matrix(4, 0, rows=slice(0, 512)),       # ~1% escapes: list overflow
        "skewed": _skewed(),
    }


MS = [1, 3, 8, 16, 17, 31, 32, 33, 48, 64]


@pytest.mark.parametrize("name", list(_mats().keys()))
@pytest.mark.parametrize("m", MS)
def test_stream_matches_fp64_oracle(name, m):
    w = _mats()[name]
    log(f"[stream] {name} {w.shape} M={m}")
    x = synth.make_activations(m, w.shape[1], seed=4000 + m)
    mat = w12.encode(dev16(w))
    plan = w12.plan_info(mat, w12.OP_GEMM, m)
    assert plan["kernel"] == w12.KERNEL_MFMA_STREAM and plan["prepass"] == 0
    yf, yb = gemm_both(mat, dev16(x))
    y64 = o.gemm_ref(x, w)
    check_f32(yf, y64, f"stream {name} M={m}")
    check_bf16(yb, yf, y64, f"stream {name} M={m}")


@pytest.mark.parametrize("grid", [1, 3, 7, 15, 50, 333, 1000])
@pytest.mark.parametrize("m", [4, 16, 40, 64])
def test_stream_any_grid(grid, m):
    """Every workgroup count splits K differently (split tiles whole-tile sized
    or single 16-row blocks, one to many sharers); all match the oracle and
    leave the counters at zero."""
    w = synth.workload_matrix(1, 0, rows=slice(0, 1024))[:, :2048]
    x = synth.make_activations(m, 2048, seed=70 + m)
    mat = w12.encode(dev16(w))
    w12.set_tuning(w12.TUNE_GRID, grid)
    ws = w12.new_workspace(w12.OP_GEMM, 1024, 2048, m)
    y = torch.empty((m, 1024), dtype=torch.float32, device="cuda")
    for rep in range(2):
        w12.w12_gemm(mat, dev16(x), y, ws)
        check_f32(y.cpu().numpy(), o.gemm_ref(x, w), f"stream grid={grid} M={m} rep={rep}")
    assert int(ws[: w12.WS_COUNTER_BYTES].view(torch.int32).abs().sum()) == 0


def _onehot_exact(w):
    enc = o.encode(w)
    esc_cols = np.unique(enc.esc["col"])
    cols = np.unique(np.concatenate([[0, 1, 63, 64, 511, 512, w.shape[1] - 1], esc_cols[:60]]))
    mat = w12.encode(dev16(w))
    for start in range(0, len(cols), 32):
        cc = cols[start:start + 32]
        x = np.zeros((len(cc), w.shape[1]), np.uint16)
        x[np.arange(len(cc)), cc] = 0x3F80
        y = w12.gemm(mat, dev16(x), torch.float32).cpu().numpy()
        want = o.bf16_to_f64(w[:, cc]).T
        assert np.array_equal(y.astype(np.float64), want), f"cols {cc}"


def test_stream_onehot_rows_reproduce_columns_exactly():
    """x = e_k makes y a column of W exactly: substituted escapes (zeros,
    subnormals, values far outside the window) and escapes past a wave's list
    capacity (dense stress rows) alike."""
    _onehot_exact(synth.workload_matrix(4, 0, rows=slice(0, 256))[:, :1024])
    _onehot_exact(_finite_patterns())
    _onehot_exact(_skewed()[192:384])


@pytest.mark.parametrize("m", [3, 16, 32, 64])
def test_stream_q8(m):
    w = synth.workload_matrix(4, 0, rows=slice(0, 512))
    enc = o.encode(w)
    x = synth.make_activations(m, w.shape[1], seed=600 + m)
    mat = w12.encode(dev16(w))
    yf, yb = gemm_both(mat, dev16(x), q=True)
    yq64 = o.gemm_q8_ref(x, enc)
    check_f32(yf, yq64, f"stream Q M={m}")
    check_bf16(yb, yf, yq64, f"stream Q M={m}")
    yfe, _ = gemm_both(mat, dev16(x), q=True, apply_escapes=True)
    qbits = o.q_view_bits(enc)
    rows = np.repeat(np.arange(enc.n), np.diff(enc.row_ptr.astype(np.int64)))
    qbits[rows, enc.esc["col"].astype(np.int64)] = enc.esc["bits"]
    check_f32(yfe, o.gemm_ref(x, qbits), f"stream Q+escapes M={m}")


def test_stream_and_helper_kernels_agree():
    """Both MFMA kernels on the same inputs: within the tolerance of each
    other (their fp32 summation orders differ)."""
    w = synth.workload_matrix(1, 1, rows=slice(0, 2048))
    x = synth.make_activations(32, w.shape[1], seed=5)
    mat = w12.encode(dev16(w))
    y64 = o.gemm_ref(x, w)
    out = {}
    for path in (2, 3):
        w12.set_tuning(w12.TUNE_PATH, path)
        out[path] = w12.gemm(mat, dev16(x), torch.float32).cpu().numpy()
        check_f32(out[path], y64, f"path={path}")
    s = np.maximum(np.abs(y64), 1e-3 * np.abs(y64).max(axis=1, keepdims=True))
    assert np.max(np.abs(out[2] - out[3]) / s) < 4e-3


@pytest.mark.parametrize("path", [1, 2, 3])
@pytest.mark.parametrize("scale_exp", [-100, 100])
def test_activation_range(path, scale_exp):
    """Activations scaled by 2^+-100: every kernel (GEMV and helper-wave MFMA
    accumulate w * 2^(127 - E_n) and scale at the end; the stream kernel
    accumulates true values) stays within the tolerance of the oracle."""
    w12.set_tuning(w12.TUNE_PATH, path)
    w = synth.workload_matrix(0, 0)
    m = 2 if path == 1 else 32
    x = synth.make_activations(m, 1024, seed=31)
    e = (x.astype(np.int64) >> 7) & 0xFF
    ok = (e > 0) & (e + scale_exp >= 1) & (e + scale_exp <= 254)
    xs = np.where(ok, x.astype(np.int64) + (scale_exp << 7), 0).astype(np.uint16)   # x * 2^scale_exp, exactly
    mat = w12.encode(dev16(w))
    yf, yb = gemm_both(mat, dev16(xs))
    y64 = o.gemm_ref(xs, w)
    check_f32(yf, y64, f"path={path} x*2^{scale_exp}")


@pytest.mark.parametrize("path", [1, 2, 3])
def test_non_finite_weights(path):
    """inf and NaN weights (escapes holding their raw bits) propagate as in
    IEEE arithmetic: every output the float64 oracle makes NaN or infinite is
    NaN or the same infinity, the rest stay within the tolerance."""
    w12.set_tuning(w12.TUNE_PATH, path)
    w = synth.workload_matrix(0, 0).copy()
    w[5, 17] = 0x7F80      # +inf
    w[300, 900] = 0xFF80   # -inf
    w[301, 3] = 0x7FC1     # NaN
    w[700, 100] = 0x7F80
    w[700, 101] = 0xFF80   # inf - inf in one row: NaN
    m = 2 if path == 1 else 17
    x = synth.make_activations(m, 1024, seed=8)
    x[:, 17] = 0x3F80      # keep the row-5 product +inf (x > 0)
    mat = w12.encode(dev16(w))
    yf = w12.gemm(mat, dev16(x), torch.float32).cpu().numpy().astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        y64 = o.gemm_ref(x, w)
    nan = np.isnan(y64)
    assert nan.any() and np.array_equal(np.isnan(yf), nan)
    inf = np.isinf(y64)
    assert inf.any() and np.array_equal(yf[inf], y64[inf])
    fin = ~(nan | inf)
    rows_ok = fin.all(axis=0)
    check_f32(yf[:, rows_ok], y64[:, rows_ok], f"finite rows path={path}")
