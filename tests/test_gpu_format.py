"""GPU encode and decode against the oracle: byte-exact records, window tops,
CSR row pointers and escape entries; bit-exact round trips (SpecPilot section
4.1: every decoded tensor must equal the checkpoint bit for bit)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev16, download, host16, log, o, strip_records, upload, w12

pytestmark = pytest.mark.gpu


def _edge_matrices():
    rng = np.random.default_rng(5)
    allpat = synth.all_bf16_patterns(512)                               # 128 x 512, every pattern
    zeros = np.zeros((16, 1024), np.uint16)                             # all escapes, +0
    negz = np.full((16, 512), 0x8000, np.uint16)                        # -0
    sub = rng.integers(0, 0x80, size=(32, 512)).astype(np.uint16)       # subnormals and zeros
    tied = np.tile(np.array([100 << 7, 116 << 7], np.uint16), (16, 256))  # every row tied
    inwin = (0x3F80 | rng.integers(0, 0x80, size=(48, 1024))).astype(np.uint16)
    specials = synth.random_bits((64, 1536), 21)
    specials[:, ::7] = 0x7F80
    specials[:, 3::11] = 0xFFC1
    return {"all_patterns": allpat, "zeros": zeros, "neg_zero": negz, "subnormal": sub, "tied": tied,
            "all_in_window": inwin, "specials": specials,
            "config0": synth.workload_matrix(0, 0),
            "plain_gaussian": synth.plain_gaussian(256, 5120, seed=3),
            "stress_rows": synth.workload_matrix(4, 0, rows=slice(0, 512))}


@pytest.mark.parametrize("name", list(_edge_matrices().keys()))
def test_encode_matches_oracle_bytes(name):
    w = _edge_matrices()[name]
    log(f"[encode parity] {name} {w.shape}")
    ref = o.encode(w)
    mat = w12.encode(dev16(w))
    torch.cuda.synchronize()
    rec, e_top, row_ptr, esc = download(mat)
    assert np.array_equal(e_top, ref.e_top)
    assert np.array_equal(row_ptr, ref.row_ptr)
    assert mat.n_esc == ref.n_esc
    assert np.array_equal(esc, ref.esc)
    assert np.array_equal(rec, ref.records)


@pytest.mark.parametrize("name", list(_edge_matrices().keys()))
def test_roundtrip_and_oracle_records_decode(name):
    w = _edge_matrices()[name]
    log(f"[decode] {name} {w.shape}")
    wd = dev16(w)
    mat = w12.encode(wd)
    assert torch.equal(w12.decode(mat).view(torch.int16), wd)
    # the GPU decoder on the oracle's bytes restores the original too
    assert np.array_equal(host16(w12.decode(upload(o.encode(w)))), w)


def test_validate_accepts_good_and_rejects_corrupt():
    w = synth.workload_matrix(0, 0)
    mat = w12.encode(dev16(w))
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    assert w12.w12_validate(mat, ws) == w12.OK
    bad = w12.W12Matrix(mat.n, mat.k, mat.records, mat.e_top.clone(), mat.row_ptr, mat.esc, mat.n_esc)
    bad.e_top[3] = 5
    assert w12.w12_validate(bad, ws) == w12.E_CORRUPT
    if mat.n_esc >= 2:
        esc = mat.esc.clone()
        e = esc.cpu().numpy().view(o.ESC_DTYPE).copy()
        e["col"][0] = mat.k + 1
        bad = w12.W12Matrix(mat.n, mat.k, mat.records, mat.e_top, mat.row_ptr,
                            torch.from_numpy(e.view(np.int64)).cuda(), mat.n_esc)
        assert w12.w12_validate(bad, ws) == w12.E_CORRUPT


WORKLOAD_MATRICES = [(wl, mi) for wl in (1, 2, 3, 4) for mi in range(len(synth.WORKLOADS[wl].matrices))
                     if not (wl == 2 and mi in (4, 5, 6))]  # config 2's MLP matrices are config 1's shapes


@pytest.mark.parametrize("wl,mi", WORKLOAD_MATRICES)
def test_workload_encode_roundtrip_and_sampled_parity(wl, mi):
    spec = synth.WORKLOADS[wl].matrices[mi]
    log(f"[workload encode] config {wl} {spec.name} {spec.n}x{spec.k}")
    w = synth.workload_matrix(wl, mi)
    wd = dev16(w)
    mat = w12.encode(wd)
    assert torch.equal(w12.decode(mat).view(torch.int16), wd)
    rec, e_top, row_ptr, esc = download(mat)
    counts = np.diff(row_ptr.astype(np.int64))
    # sampled 16-row blocks, whole: first, last and spread ones
    nblk = spec.n // 16
    rng = np.random.default_rng(wl * 10 + mi)
    blocks = sorted(set([0, nblk - 1] + list(rng.choice(nblk, size=min(nblk, 6), replace=False))))
    for b in blocks:
        rows = slice(16 * b, 16 * b + 16)
        ref = o.encode(w[rows])
        assert np.array_equal(e_top[rows], ref.e_top), b
        assert np.array_equal(counts[rows], np.diff(ref.row_ptr.astype(np.int64))), b
        assert np.array_equal(strip_records(rec, spec.k, [b]), ref.records), b
        got = esc[row_ptr[16 * b]:row_ptr[16 * b + 16]]
        assert np.array_equal(got, ref.esc), b
    # every row's window top and escape count, from the oracle's window rule
    step = max(1, spec.n // 2048)
    sample = w[::step]
    assert np.array_equal(e_top[::step], o.window_tops(sample).astype(np.uint8))
    frac = mat.n_esc / w.size
    log(f"  n_esc={mat.n_esc} fraction={frac:.3e} bits/weight={o.bits_per_weight(spec.n, spec.k, mat.n_esc):.4f}")
    assert mat.nbytes() == o.encoded_nbytes(spec.n, spec.k, mat.n_esc)
