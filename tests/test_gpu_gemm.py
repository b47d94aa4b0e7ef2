"""GPU GEMM, Q pass and LM-head argmax against the oracle's float64 products.

SpecPilot section 4.1 / Figure 5b (exact W12 GEMM with the escape fix-up and
a deterministic split of the reduction), section 4.3 (Q pass over the 8-bit
view with the midpoint rule), Appendix E (W12 LM head; here fused with an
argmax whose ties go to the lowest index)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import argmax_logits_f32, check_bf16, check_f32, dev16, gemm_both, host16, log, o, upload, w12

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_tuning():
    yield
    w12.set_tuning(w12.TUNE_PATH, 0)
    w12.set_tuning(w12.TUNE_GRID, 0)


def _mats():
    return {
        "config0": synth.workload_matrix(0, 0),                          # 1024 x 1024
        "ragged_rows": synth.workload_matrix(0, 0)[:48],                  # last GEMV tile has 48 rows
        "single_record": synth.workload_matrix(0, 0)[:16, :512],
        "wide_k": synth.workload_matrix(1, 2, rows=slice(0, 256)),       # 256 x 17408
        "stress": synth.workload_matrix(4, 0, rows=slice(0, 512)),       # ~1% escapes, bimodal rows
    }


MS = [1, 2, 3, 4, 7, 8, 15, 16, 17, 31, 32, 33, 48, 63, 64]


@pytest.mark.parametrize("name", list(_mats().keys()))
@pytest.mark.parametrize("m", MS)
def test_gemm_matches_fp64_oracle(name, m):
    w = _mats()[name]
    log(f"[gemm] {name} {w.shape} M={m}")
    x = synth.make_activations(m, w.shape[1], seed=1000 + m)
    mat = w12.encode(dev16(w))
    yf, yb = gemm_both(mat, dev16(x))
    y64 = o.gemm_ref(x, w)
    check_f32(yf, y64, f"{name} M={m}")
    check_bf16(yb, yf, y64, f"{name} M={m}")


@pytest.mark.parametrize("name", ["config0", "wide_k", "stress"])
@pytest.mark.parametrize("m", [2, 5, 9, 15, 16])
def test_forced_gemv_matches_oracle(name, m):
    """The GEMV kernel runs M = 1 by default; forced, it serves every M up to 16."""
    w = _mats()[name]
    log(f"[gemv forced] {name} {w.shape} M={m}")
    x = synth.make_activations(m, w.shape[1], seed=2000 + m)
    mat = w12.encode(dev16(w))
    w12.set_tuning(w12.TUNE_PATH, 1)
    yf, yb = gemm_both(mat, dev16(x))
    y64 = o.gemm_ref(x, w)
    check_f32(yf, y64, f"gemv {name} M={m}")
    check_bf16(yb, yf, y64, f"gemv {name} M={m}")


@pytest.mark.parametrize("grid", [1, 3, 7, 15, 50, 1000])
@pytest.mark.parametrize("m", [1, 5, 16, 40])
@pytest.mark.parametrize("path", [0, 1])
def test_split_reduction_any_grid(grid, m, path):
    """Every workgroup count splits K differently (partial tiles reduced in a
    fixed order; at 15 workgroups the MFMA kernel's split tiles are single
    16-row blocks); all must match the oracle. path 1 forces the GEMV kernel."""
    if path == 1 and m > 16:
        pytest.skip("the GEMV kernel serves M <= 16")
    w = synth.workload_matrix(0, 0)
    x = synth.make_activations(m, 1024, seed=7 + m)
    mat = w12.encode(dev16(w))
    w12.set_tuning(w12.TUNE_GRID, grid)
    w12.set_tuning(w12.TUNE_PATH, path)
    yf, yb = gemm_both(mat, dev16(x))
    check_f32(yf, o.gemm_ref(x, w), f"grid={grid} M={m} path={path}")


@pytest.mark.parametrize("n,k,m", [
    (6144, 512, 1), (6144, 512, 32),   # 96 tiles: two equal sharers per tile (192 workgroups)
    (5120, 512, 2), (5120, 512, 20),   # 80 tiles, two units each: capped at 160 workgroups
    (5120, 1024, 48), (5120, 1024, 64),  # 160 tiles of 32 rows: whole tiles, no exchange
    (4096, 1024, 16),                  # 64 tiles: four sharers per tile
])
def test_default_grid_for_fewer_tiles_than_cus(n, k, m):
    """With fewer tiles than compute units the library picks the grid by the
    tile count (equal sharers per tile, or whole tiles on fewer workgroups):
    each such plan matches the oracle."""
    w = synth.make_weights(n, k, synth.WORKLOADS[0], seed=n + k)
    log(f"[default grid] {n}x{k} M={m}")
    x = synth.make_activations(m, k, seed=31 + m)
    mat = w12.encode(dev16(w))
    yf, yb = gemm_both(mat, dev16(x))
    y64 = o.gemm_ref(x, w)
    check_f32(yf, y64, f"{n}x{k} M={m}")
    check_bf16(yb, yf, y64, f"{n}x{k} M={m}")


@pytest.mark.parametrize("n,k,m", [
    (12784, 5120, 32),   # 200 tiles of 64 rows on 200 workgroups; the last tile has 48 rows
    (16368, 1024, 32),   # 256 tiles on 256 workgroups; the last tile has 48 rows
    (4112, 5120, 64),    # 257 blocks in 129 tiles of 32 rows; the last tile has 16 rows
    (16336, 4096, 8),    # 256 whole tiles on 256 workgroups; the last tile has 16 rows
    (16336, 4096, 1),
])
@pytest.mark.parametrize("path", [0, 3])
def test_whole_tiles_reaching_past_n(n, k, m, path):
    """Plans whose whole tiles already cover every row, with a last tile cut
    short by N: no rows are left for split tiles, and every output matches
    (the library's kernel choice, and the stream kernel forced)."""
    w12.set_tuning(w12.TUNE_PATH, path)
    w = synth.make_weights(n, k, synth.WORKLOADS[0], seed=n + 3 * k)
    log(f"[whole tiles past N] {n}x{k} M={m} path={path}")
    x = synth.make_activations(m, k, seed=53 + m)
    mat = w12.encode(dev16(w))
    yf, yb = gemm_both(mat, dev16(x))
    y64 = o.gemm_ref(x, w)
    check_f32(yf, y64, f"{n}x{k} M={m}")
    check_bf16(yb, yf, y64, f"{n}x{k} M={m}")


def test_gemv_and_mfma_paths_agree_at_m16():
    w = synth.workload_matrix(0, 0)
    x = synth.make_activations(16, 1024, seed=99)
    mat = w12.encode(dev16(w))
    y64 = o.gemm_ref(x, w)
    out = {}
    for path in (1, 2):
        w12.set_tuning(w12.TUNE_PATH, path)
        out[path] = w12.gemm(mat, dev16(x), torch.float32).cpu().numpy()
        check_f32(out[path], y64, f"path={path}")
    assert np.max(np.abs(out[1] - out[2]) / np.maximum(np.abs(y64), 1e-3 * np.abs(y64).max())) < 2 * 2e-3


def _onehot_case(w, big_scale):
    enc = o.encode(w)
    esc_cols = np.unique(enc.esc["col"])
    cols = np.unique(np.concatenate([[0, 1, 511, 512, w.shape[1] - 1], esc_cols[:40]]))
    mat = w12.encode(dev16(w))
    for start in range(0, len(cols), 32):
        cc = cols[start:start + 32]
        x = np.zeros((len(cc), w.shape[1]), np.uint16)
        scale = np.ones(len(cc))
        for i, c in enumerate(cc):
            x[i, c] = 0x3F80
            if big_scale and i % 3 == 0:
                x[i, c] = 0x4300                                          # 128.0
                scale[i] = 128.0
        y = w12.gemm(mat, dev16(x), torch.float32).cpu().numpy()
        want = scale[:, None] * o.bf16_to_f64(w[:, cc]).T
        assert np.array_equal(y.astype(np.float64), want), f"cols {cc}"


def test_onehot_rows_reproduce_columns_exactly():
    """x = e_k (or 128 e_k) makes y a column of W: exact, escape columns
    included (the fix-up removes the placeholder and adds the exact weight)."""
    _onehot_case(synth.workload_matrix(4, 0, rows=slice(0, 256))[:, :1024], big_scale=True)
    # every finite BF16 pattern, zeros and subnormals included (x = 1 only: a
    # larger factor would overflow fp32 on the largest patterns)
    w = synth.all_bf16_patterns(512).reshape(-1, 1024)
    w = w[np.isfinite(o.bf16_to_f64(w)).all(axis=1)]
    _onehot_case(w[: (w.shape[0] // 16) * 16], big_scale=False)


@pytest.mark.parametrize("grid", [0, 5, 333])
def test_workspace_reuse_across_calls(grid):
    """Split tiles count their workgroups in the workspace and reset the count:
    one workspace serves many calls, ops and sizes in a row."""
    w12.set_tuning(w12.TUNE_GRID, grid)
    w = synth.workload_matrix(0, 0)
    mat = w12.encode(dev16(w))
    big = max(w12.workspace_bytes(op, 1024, 1024, m) for op in (w12.OP_GEMM, w12.OP_GEMM_Q8, w12.OP_LMHEAD_ARGMAX)
              for m in (1, 7, 16, 33, 64))
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    ref = o.encode(w)
    for rep in range(3):
        for m in (1, 7, 16, 33, 64):
            x = synth.make_activations(m, 1024, seed=rep * 100 + m)
            y = torch.empty((m, 1024), dtype=torch.float32, device="cuda")
            w12.w12_gemm(mat, dev16(x), y, ws)
            check_f32(y.cpu().numpy(), o.gemm_ref(x, w), f"reuse grid={grid} rep={rep} M={m}")
            w12.w12_gemm_q8(mat, dev16(x), y, 0, ws)
            check_f32(y.cpu().numpy(), o.gemm_q8_ref(x, ref), f"reuse Q grid={grid} rep={rep} M={m}")
            idx = torch.empty(m, dtype=torch.int32, device="cuda")
            w12.w12_lmhead_argmax(mat, dev16(x), idx, None, ws)
            ridx, margin = o.argmax_ref(o.gemm_ref(x, w))
            far = margin >= 1e-3
            assert np.array_equal(idx.cpu().numpy()[far], ridx[far])
    torch.cuda.synchronize()
    assert int(ws[: w12.WS_COUNTER_BYTES].view(torch.int32).abs().sum()) == 0   # counters back at zero


def test_deterministic_repeats():
    w = synth.workload_matrix(4, 0, rows=slice(0, 1024))
    mat = w12.encode(dev16(w))
    for m in (1, 8, 32, 64):
        x = dev16(synth.make_activations(m, w.shape[1], seed=m))
        a = w12.gemm(mat, x, torch.float32)
        b = w12.gemm(mat, x, torch.float32)
        assert torch.equal(a, b)
        qa = w12.gemm_q8(mat, x, torch.float32)
        qb = w12.gemm_q8(mat, x, torch.float32)
        assert torch.equal(qa, qb)


def test_deterministic_repeats_whole_tiles():
    """17408 x 5120 (272 whole tiles): the helper-wave kernel at every M from
    3 (its streaming waves' fixed share of columns, the split tiles' exchange)
    and the GEMV below; repeated calls, over two copies of the matrix, give
    the same bits."""
    w = synth.workload_matrix(1, 0)
    mat = w12.encode(dev16(w))
    mat2 = w12.W12Matrix(mat.n, mat.k, mat.records.clone(), mat.e_top.clone(), mat.row_ptr.clone(),
                         mat.esc.clone(), mat.n_esc)
    for m in (1, 3, 16, 17, 32, 64):
        log(f"[repeats] 17408x5120 M={m} {w12.plan_info(mat, w12.OP_GEMM, m)['kernel_name']}")
        x = dev16(synth.make_activations(m, w.shape[1], seed=40 + m))
        a = w12.gemm(mat, x, torch.float32)
        for rep in range(2):
            assert torch.equal(w12.gemm(mat2 if rep else mat, x, torch.float32), a)
            assert torch.equal(w12.gemm_q8(mat, x, torch.float32, apply_escapes=True),
                               w12.gemm_q8(mat2, x, torch.float32, apply_escapes=True))


@pytest.mark.parametrize("path", [0, 2, 3])
def test_strided_activations_and_outputs(path):
    """x and y with row strides past K and N, on the library's choice and on
    each MFMA kernel forced (both read row-major x themselves up to 16 rows,
    the stream kernel at every M)."""
    w = synth.workload_matrix(0, 0)
    mat = w12.encode(dev16(w))
    old = w12.set_tuning(w12.TUNE_PATH, path)
    try:
        for m in (3, 16, 20, 32):
            xfull = synth.make_activations(m, 1024 + 64, seed=m)
            xd = dev16(xfull)[:, :1024]                                   # ldx = 1088
            y = torch.full((m, 1024 + 32), -7.0, dtype=torch.float32, device="cuda")
            ws = w12.new_workspace(w12.OP_GEMM, 1024, 1024, m)
            w12.w12_gemm(mat, xd, y[:, :1024], ws)
            yh = y.cpu().numpy()
            check_f32(yh[:, :1024], o.gemm_ref(xfull[:, :1024], w), f"strided M={m} path {path}")
            assert np.all(yh[:, 1024:] == -7.0)                           # nothing written past N
    finally:
        w12.set_tuning(w12.TUNE_PATH, old)


@pytest.mark.parametrize("m", [1, 8, 16, 32])
def test_q8_matches_oracle_view(m):
    w = synth.workload_matrix(4, 0, rows=slice(0, 512))
    enc = o.encode(w)
    x = synth.make_activations(m, w.shape[1], seed=300 + m)
    mat = w12.encode(dev16(w))
    yf, yb = gemm_both(mat, dev16(x), q=True)
    yq64 = o.gemm_q8_ref(x, enc)
    check_f32(yf, yq64, f"Q M={m}")
    check_bf16(yb, yf, yq64, f"Q M={m}")
    # with escapes applied the Q pass differs from the Q view only at escapes
    yfe, _ = gemm_both(mat, dev16(x), q=True, apply_escapes=True)
    qbits = o.q_view_bits(enc)
    rows = np.repeat(np.arange(enc.n), np.diff(enc.row_ptr.astype(np.int64)))
    qbits[rows, enc.esc["col"].astype(np.int64)] = enc.esc["bits"]
    check_f32(yfe, o.gemm_ref(x, qbits), f"Q+escapes M={m}")


def test_q8_equals_exact_when_low_bits_are_midpoint():
    w = (synth.plain_gaussian(256, 1024, seed=12) & 0xFFF0) | 0x0008
    enc = o.encode(w)
    keep = np.ones(w.shape[0], bool)
    rows = np.repeat(np.arange(enc.n), np.diff(enc.row_ptr.astype(np.int64)))
    keep[rows] = False                                                   # rows without escapes
    w = w[keep][: (keep.sum() // 16) * 16]
    assert o.encode(w).n_esc == 0
    mat = w12.encode(dev16(w))
    for m in (1, 32):
        x = dev16(synth.make_activations(m, 1024, seed=m))
        assert torch.equal(w12.gemm(mat, x, torch.float32), w12.gemm_q8(mat, x, torch.float32))


@pytest.mark.parametrize("m", [1, 4, 16, 32, 64])
def test_lmhead_argmax_small(m):
    rng = np.random.default_rng(m)
    w = synth.workload_matrix(3, 0, rows=slice(0, 2048))
    x = synth.make_activations(m, w.shape[1], seed=500 + m)
    mat = w12.encode(dev16(w))
    idx, mx = w12.lmhead_argmax(mat, dev16(x))
    yf = argmax_logits_f32(mat, dev16(x)).cpu().numpy()
    idx = idx.cpu().numpy()
    mx = mx.cpu().numpy()
    # the fused argmax is the argmax of the same kernel's fp32 logits
    assert np.array_equal(idx, np.argmax(yf, axis=1))
    assert np.array_equal(mx, yf[np.arange(m), idx])
    # and the oracle's, away from near-ties
    ridx, margin = o.argmax_ref(o.gemm_ref(x, w))
    far = margin >= 1e-3
    assert np.array_equal(idx[far], ridx[far])
    del rng


@pytest.mark.parametrize("m", [1, 2, 3, 16, 17, 32, 33, 48, 64])
def test_lmhead_argmax_whole_tiles(m):
    """Enough rows that every workgroup also owns whole tiles (the per-lane and
    per-tile argmax folds), with exact ties planted in different whole tiles:
    the lowest row must win."""
    n, k = 20480, 1024
    w = synth.workload_matrix(3, 0, rows=slice(0, n))[:, :k].copy()
    x = synth.make_activations(m, k, seed=900 + m)
    # row 9000 scaled by 2^14 (exponent field + 14, exact) leads for many
    # activation rows; rows 3000 and 15000 (other whole tiles and workgroups,
    # which add up K in the same order) copy it
    e = (w[9000] >> 7) & 0xFF
    w[9000] = np.where((e > 0) & (e < 240), w[9000] + (14 << 7), w[9000]).astype(np.uint16)
    w[3000] = w[9000]
    w[15000] = w[9000]
    log(f"[argmax whole tiles] {n}x{k} M={m}")
    mat = w12.encode(dev16(w))
    idx, mx = w12.lmhead_argmax(mat, dev16(x))
    yf = argmax_logits_f32(mat, dev16(x)).cpu().numpy()
    idx = idx.cpu().numpy().astype(np.int64)
    assert np.array_equal(idx, np.argmax(yf, axis=1))
    assert np.array_equal(mx.cpu().numpy().view(np.uint32), yf[np.arange(m), idx].view(np.uint32))
    y64 = o.gemm_ref(x, w)
    ridx, margin = o.argmax_ref(y64)
    far = margin >= 1e-3
    assert np.array_equal(idx[far], ridx[far])
    # where the planted rows lead, the lowest of the three wins
    lead = np.isin(ridx, [3000, 9000, 15000])
    assert lead.sum() >= 1 if m > 2 else True
    assert np.all(idx[lead] == 3000)


@pytest.mark.parametrize("m", [2, 20])
def test_lmhead_argmax_planted_ties_and_negatives(m):
    """All-negative logits, exact ties (lowest index wins) and -0 vs +0; at
    M = 20 through the stored-logits pass, whose workgroup reads pieces past
    the 64 columns of a row (they re-read the row's last piece, unused)."""
    k = 512
    w = np.zeros((64, k), np.uint16)
    w[:, 0] = 0xBF80                                                     # every logit = -x0
    w[10, 0] = 0xBF00                                                    # -0.5: the max for x0 > 0
    w[40, 0] = 0xBF00                                                    # tie with row 10
    mat = w12.encode(dev16(w))
    x = np.zeros((m, k), np.uint16)
    x[0::2, 0] = 0x4000                                                  # 2.0
    x[1::2, 0] = 0x0000                                                  # all logits +-0 -> row 0
    idx, mx = w12.lmhead_argmax(mat, dev16(x))
    assert idx.cpu().tolist() == [10, 0] * (m // 2)
    assert mx.cpu().tolist() == [-1.0, 0.0] * (m // 2)


def test_oracle_encoded_records_drive_the_gemm():
    """The GEMM reads the oracle's bytes as well as the GPU encoder's."""
    w = synth.workload_matrix(0, 0)
    x = synth.make_activations(32, 1024, seed=4)
    y_gpu_enc = w12.gemm(w12.encode(dev16(w)), dev16(x), torch.float32)
    y_orc_enc = w12.gemm(upload(o.encode(w)), dev16(x), torch.float32)
    assert torch.equal(y_gpu_enc, y_orc_enc)
    log(f"max |y| {float(y_gpu_enc.abs().max()):.3f}; bits {host16(y_gpu_enc.to(torch.bfloat16))[0, :2]}")
