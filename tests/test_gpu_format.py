"""GPU encode and decode against the oracle: byte-exact records, window tops,
CSR row pointers and escape entries; bit-exact round trips (SpecPilot section
4.1: every decoded tensor must equal the checkpoint bit for bit)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from gpu_util import dev16, download, host16, log, o, upload, w12

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


WORKLOAD_MATRICES = [(wl, mi) for wl in (1, 2, 3, 4) for mi in range(len(synth.WORKLOADS[wl].matrices))]
CHUNK = 2048
THREADS = max(1, min(16, os.cpu_count() or 1))


def _compare_chunk(w, r0, r1, rec, e_top, row_ptr, esc, per_block):
    """Mismatch text for rows [r0, r1) against the oracle's encoding of those rows, or ''."""
    ref = o.encode(w[r0:r1])
    if not np.array_equal(e_top[r0:r1], ref.e_top):
        bad = np.nonzero(e_top[r0:r1] != ref.e_top)[0]
        return f"e_top differs at rows {(r0 + bad[:8]).tolist()}"
    if not np.array_equal(row_ptr[r0:r1 + 1] - row_ptr[r0], ref.row_ptr):
        return f"escape row pointers differ in rows [{r0}, {r1})"
    if not np.array_equal(esc[row_ptr[r0]:row_ptr[r1]], ref.esc):
        return f"escape entries differ in rows [{r0}, {r1})"
    if not np.array_equal(rec[r0 // 16 * per_block:r1 // 16 * per_block], ref.records):
        return f"record bytes differ in rows [{r0}, {r1})"
    return ""


@pytest.mark.parametrize("wl,mi", WORKLOAD_MATRICES)
def test_workload_encode_full_parity(wl, mi):
    """Every window top, escape row pointer, escape entry and record byte of
    the GPU encoding equals the oracle's (computed over 2048-row chunks in a
    thread pool: plain oracle calls on row ranges, which the format encodes
    independently), and the GPU decode restores every weight bit for bit."""
    spec = synth.WORKLOADS[wl].matrices[mi]
    log(f"[workload encode] config {wl} {spec.name} {spec.n}x{spec.k}")
    w = synth.workload_matrix(wl, mi)
    wd = dev16(w)
    mat = w12.encode(wd)
    assert torch.equal(w12.decode(mat).view(torch.int16), wd)
    del wd
    rec, e_top, row_ptr, esc = download(mat)
    per_block = (spec.k // 512) * 12288
    chunks = [(r, min(r + CHUNK, spec.n)) for r in range(0, spec.n, CHUNK)]
    with ThreadPoolExecutor(THREADS) as ex:
        errs = list(ex.map(lambda c: _compare_chunk(w, c[0], c[1], rec, e_top, row_ptr, esc, per_block), chunks))
    bad = [e for e in errs if e]
    assert not bad, bad[:4]
    assert int(row_ptr[0]) == 0 and int(row_ptr[-1]) == mat.n_esc
    frac = mat.n_esc / w.size
    log(f"  n_esc={mat.n_esc} fraction={frac:.3e} bits/weight={o.bits_per_weight(spec.n, spec.k, mat.n_esc):.4f}")
    assert mat.nbytes() == o.encoded_nbytes(spec.n, spec.k, mat.n_esc)


def test_encode_never_writes_past_escape_capacity():
    """A buffer smaller than the escape count gets the list's prefix and not
    one byte more; records and the CSR row pointers are unaffected."""
    w = synth.workload_matrix(4, 0, rows=slice(0, 256))[:64]
    ref = o.encode(w)
    assert ref.n_esc > 40
    wd = dev16(w)
    e_top = torch.empty(64, dtype=torch.uint8, device="cuda")
    row_ptr = torch.empty(65, dtype=torch.int32, device="cuda")
    ws = w12.new_workspace(w12.OP_ENCODE_PLAN, 64, w.shape[1])
    assert w12.w12_encode_plan(wd, e_top, row_ptr, ws) == ref.n_esc
    cap = ref.n_esc - 37
    records = torch.empty(ref.records.size, dtype=torch.uint8, device="cuda")
    esc = torch.full((ref.n_esc + 8,), -1, dtype=torch.int64, device="cuda")
    w12.w12_encode(wd, e_top, row_ptr, records, esc, n_esc=cap)
    got = esc.cpu().numpy()
    assert np.array_equal(got[:cap].view(o.ESC_DTYPE), ref.esc[:cap])
    assert np.all(got[cap:] == -1)
    assert np.array_equal(records.cpu().numpy(), ref.records)
    assert np.array_equal(row_ptr.cpu().numpy().view(np.uint32), ref.row_ptr)
