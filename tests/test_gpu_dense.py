"""The dense-escape path against the oracle: the GEMM without escape work,
then the fix-up kernel applying y = (A - CN) + CP per output (SpecPilot
section 4.1: the sparse per-channel list restores the exact weights; here the
list is dense, about 55 escapes per row in the escape-stress workload).

The library takes this path above 8 escapes per row; W12_TUNE_PATH = 4 forces
it on any matrix with escapes."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import check_bf16, check_f32, dev16, gemm_both, log, o, w12

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_hooks():
    yield
    w12.set_tuning(w12.TUNE_PATH, 0)


def _stress(rows=512, cols=None):
    w = synth.workload_matrix(4, 0, rows=slice(0, max(rows, 256)))[:rows]
    return w if cols is None else w[:, :cols]


@pytest.mark.parametrize("m", [1, 2, 3, 16, 32, 33, 64])
def test_dense_path_chosen_and_matches_oracle(m):
    w = _stress()
    enc = o.encode(w)
    assert enc.n_esc > 8 * w.shape[0]
    mat = w12.encode(dev16(w))
    for op, flags in ((w12.OP_GEMM, 0), (w12.OP_GEMM_Q8, w12.Q8_APPLY_ESCAPES)):
        assert w12.plan_info(mat, op, m, flags)["fixup"] == 1
    assert w12.plan_info(mat, w12.OP_GEMM_Q8, m)["fixup"] == 0          # view only: no escapes to apply
    assert w12.plan_info(mat, w12.OP_LMHEAD_ARGMAX, m)["fixup"] == 0
    x = synth.make_activations(m, w.shape[1], seed=7000 + m)
    log(f"[dense] stress {w.shape} M={m}")
    yf, yb = gemm_both(mat, dev16(x))
    y64 = o.gemm_ref(x, w)
    check_f32(yf, y64, f"dense exact M={m}")
    check_bf16(yb, yf, y64, f"dense exact M={m}")
    yqf, yqb = gemm_both(mat, dev16(x), q=True, apply_escapes=True)
    yq64 = o.gemm_ref(x, o.q_view_escapes_bits(enc))
    check_f32(yqf, yq64, f"dense Q+escapes M={m}")
    check_bf16(yqb, yqf, yq64, f"dense Q+escapes M={m}")


@pytest.mark.parametrize("name,rows,cols", [("config0", 1024, 1024), ("ragged_48", 48, 1024),
                                            ("single_record", 16, 512), ("wide_k", 256, 17408)])
@pytest.mark.parametrize("m", [1, 5, 32, 64])
def test_forced_dense_path_on_sparse_escapes(name, rows, cols, m):
    if name == "wide_k":
        w = synth.workload_matrix(1, 2, rows=slice(0, 256))
    else:
        w = synth.workload_matrix(0, 0)[:rows, :cols]
    w12.set_tuning(w12.TUNE_PATH, w12.PATH_DENSE)
    mat = w12.encode(dev16(w))
    assert w12.plan_info(mat, w12.OP_GEMM, m)["fixup"] == 1
    x = synth.make_activations(m, w.shape[1], seed=7100 + m)
    yf, yb = gemm_both(mat, dev16(x))
    y64 = o.gemm_ref(x, w)
    check_f32(yf, y64, f"forced dense {name} M={m}")
    check_bf16(yb, yf, y64, f"forced dense {name} M={m}")


def test_dense_onehot_rows_reproduce_columns_exactly():
    """x = e_k: A holds the placeholder, CN cancels it exactly and CP adds the
    exact weight, so y is the weight column bit for bit (zeros, subnormals,
    far outliers included)."""
    w = _stress(256, 1024)
    enc = o.encode(w)
    mat = w12.encode(dev16(w))
    cols = np.unique(np.concatenate([[0, 1, 511, 512, 1023], np.unique(enc.esc["col"])[:59]]))
    qv = o.q_view_escapes_bits(enc)
    for start in range(0, len(cols), 32):
        cc = cols[start:start + 32]
        x = np.zeros((len(cc), w.shape[1]), np.uint16)
        x[np.arange(len(cc)), cc] = 0x3F80
        y = w12.gemm(mat, dev16(x), torch.float32).cpu().numpy()
        assert np.array_equal(y.astype(np.float64), o.bf16_to_f64(w[:, cc]).T), f"cols {cc}"
        # the Q pass with escapes through the same fix-up: the Q view with the
        # escapes' exact values, column for column
        yq = w12.gemm_q8(mat, dev16(x), torch.float32, apply_escapes=True).cpu().numpy()
        assert np.array_equal(yq.astype(np.float64), o.bf16_to_f64(qv[:, cc]).T), f"Q cols {cc}"


def test_dense_non_finite_weights():
    w12.set_tuning(w12.TUNE_PATH, w12.PATH_DENSE)
    w = synth.workload_matrix(0, 0).copy()
    w[5, 17] = 0x7F80
    w[300, 900] = 0xFF80
    w[301, 3] = 0x7FC1
    x = synth.make_activations(8, 1024, seed=8)
    x[:, 17] = 0x3F80
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
    check_f32(yf[:, rows_ok], y64[:, rows_ok], "dense finite rows")


def test_dense_path_workspace_reuse_and_strides():
    """The dense path inside one workspace shared with other calls and sizes,
    with strided x and y; the counters end at zero."""
    w = _stress()
    mat = w12.encode(dev16(w))
    n, k = w.shape
    ws = w12.new_workspace(w12.OP_GEMM, n, k, 64)
    for rep in range(2):
        for m in (64, 3, 17):
            xfull = synth.make_activations(m, k + 64, seed=rep * 10 + m)
            xd = dev16(xfull)[:, :k]
            y = torch.full((m, n + 16), -7.0, dtype=torch.float32, device="cuda")
            w12.w12_gemm(mat, xd, y[:, :n], ws)
            yh = y.cpu().numpy()
            check_f32(yh[:, :n], o.gemm_ref(xfull[:, :k], w), f"reuse rep={rep} M={m}")
            assert np.all(yh[:, n:] == -7.0)
    torch.cuda.synchronize()
    assert int(ws[: w12.WS_COUNTER_BYTES].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("m", [1, 32])
def test_dense_path_escape_lists_beyond_one_lds_piece(m):
    """Many escapes per row on a tall matrix: the slices per row are capped so
    that the fix-up's lanes stay within one pass of the device, so each
    workgroup takes 32 or more rows and more than the 2048 escape entries that
    one LDS piece holds; the lists are walked across several pieces, with
    slices that straddle a piece boundary."""
    n, k = 20480, 2048
    w = synth.workload_matrix(3, 0, rows=slice(0, n))[:, :k].copy()
    rng = np.random.default_rng(11)
    hit = rng.random(w.shape) < 0.06
    e = (w >> 7) & 0xFF
    # outliers 2^12 above their neighbours (exponent field + 12, exact): escapes
    w = np.where(hit & (e > 0) & (e < 240), w + (12 << 7), w).astype(np.uint16)
    mat = w12.encode(dev16(w))
    assert mat.n_esc > 100 * n                       # > 3200 entries in any 32 rows
    assert w12.plan_info(mat, w12.OP_GEMM, m)["fixup"] == 1
    x = synth.make_activations(m, k, seed=7300 + m)
    log(f"[dense] {n}x{k} n_esc={mat.n_esc} M={m}")
    yf, yb = gemm_both(mat, dev16(x))
    y64 = o.gemm_ref(x, w)
    check_f32(yf, y64, f"dense pieces M={m}")
    check_bf16(yb, yf, y64, f"dense pieces M={m}")
