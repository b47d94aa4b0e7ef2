"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (default workgroup count, one call per matrix and M).

Workloads (shapes and weight distributions of SpecPilot, arXiv 2611.02501,
section 4.1 and Appendix E, with synthetic per-channel Gaussian weights):
  * the MLP GEMMs at hidden 5120 (gate/up 17408x5120, down 5120x17408) at
    M = 1, 4, 8, 16, 32;
  * one decoder layer's seven linears at M = 32 and 64;
  * the LM head 151936x5120 fused with the argmax at M = 1, 16, 32;
  * the Q pass and escape stress on the MLP shapes at M = 32 (1e-2 outliers,
    10% bimodal rows): full escape lists and records against the oracle, the
    exact and Q outputs, and the per-row top-1 agreement of Q and exact.

Every output is compared: the oracle's float64 products are computed over
row chunks of W in a thread pool (plain oracle calls; chunking only splits
the rows of W^T).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from gpu_util import REL, argmax_logits_f32, check_bf16, check_f32, dev16, download, gemm_both, log, o, w12

pytestmark = pytest.mark.gpu

CHUNK = 2048
THREADS = max(1, min(8, os.cpu_count() or 1))


def _chunks(n):
    return [(r, min(r + CHUNK, n)) for r in range(0, n, CHUNK)]


def oracle_products(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """float64 X W^T, computed over row chunks of W (oracle gemm_ref per chunk)."""
    y = np.empty((x.shape[0], w.shape[0]), np.float64)

    def work(c):
        y[:, c[0]:c[1]] = o.gemm_ref(x, w[c[0]:c[1]])

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(work, _chunks(w.shape[0])))
    return y


def _activations(wl, mi, ms, k):
    return {m: synth.make_activations(m, k, seed=synth.activation_seed(wl, mi, m)) for m in ms}


def _gemm_full_check(wl, mi, ms):
    spec = synth.WORKLOADS[wl].matrices[mi]
    log(f"[workload gemm] config {wl} {spec.name} {spec.n}x{spec.k} M={list(ms)}")
    w = synth.workload_matrix(wl, mi)
    mat = w12.encode(dev16(w))
    xs = _activations(wl, mi, ms, spec.k)
    xall = np.concatenate([xs[m] for m in ms], axis=0)
    y64all = oracle_products(xall, w)
    row = 0
    for m in ms:
        log(f"  M={m}")
        xd = dev16(xs[m])
        yf, yb = gemm_both(mat, xd)
        y64 = y64all[row:row + m]
        row += m
        worst = check_f32(yf, y64, f"config {wl} {spec.name} M={m}")
        check_bf16(yb, yf, y64, f"config {wl} {spec.name} M={m}")
        # the same call again gives the same bits
        again = w12.gemm(mat, xd, torch.float32).cpu().numpy()
        assert np.array_equal(again.view(np.uint32), yf.view(np.uint32))
        log(f"    max scaled error {worst:.2e} (bound {REL})")


@pytest.mark.parametrize("mi", [0, 1, 2], ids=["gate", "up", "down"])
def test_mlp_hidden5120_full(mi):
    _gemm_full_check(1, mi, (1, 4, 8, 16, 32))


@pytest.mark.parametrize("mi", range(7), ids=["q", "k", "v", "o", "gate", "up", "down"])
def test_decoder_layer_hidden5120_full(mi):
    _gemm_full_check(2, mi, (32, 64))


LM_MS = (1, 16, 32)


@pytest.fixture(scope="module")
def lm_head():
    spec = synth.WORKLOADS[3].matrices[0]
    log(f"[lm head] generating {spec.n}x{spec.k}")
    w = synth.workload_matrix(3, 0)
    mat = w12.encode(dev16(w))
    torch.cuda.synchronize()
    xs = _activations(3, 0, LM_MS, spec.k)
    y64 = oracle_products(np.concatenate([xs[m] for m in LM_MS], axis=0), w)
    del w
    out, row = {}, 0
    for m in LM_MS:
        out[m] = (xs[m], y64[row:row + m])
        row += m
    return mat, out


@pytest.mark.parametrize("m", LM_MS)
def test_lm_head_151936_argmax_full(lm_head, m):
    mat, data = lm_head
    x, y64 = data[m]
    log(f"[lm head argmax] 151936x5120 M={m}")
    xd = dev16(x)
    idx, mx = w12.lmhead_argmax(mat, xd)
    yf = argmax_logits_f32(mat, xd).cpu().numpy()
    idx = idx.cpu().numpy().astype(np.int64)
    mx = mx.cpu().numpy()
    check_f32(yf, y64, f"lm head logits M={m}")
    # the fused argmax is the argmax (lowest index on ties) of the same fp32 logits
    assert np.array_equal(idx, np.argmax(yf, axis=1))
    assert np.array_equal(mx.view(np.uint32), yf[np.arange(m), idx].view(np.uint32))
    ridx, margin = o.argmax_ref(y64)
    near = margin < 1e-3
    assert np.array_equal(idx[~near], ridx[~near])
    log(f"  rows with top-2 margin < 1e-3: {int(near.sum())} of {m}"
        + (f" (indices {np.nonzero(near)[0].tolist()}, agree {int((idx[near] == ridx[near]).sum())})"
           if near.any() else ""))


def _oracle_stress(w, x):
    """Chunked oracle encode plus the exact and Q-view float64 products."""
    n = w.shape[0]
    yx = np.empty((x.shape[0], n), np.float64)
    yq = np.empty_like(yx)
    encs = {}

    def work(c):
        r0, r1 = c
        enc = o.encode(w[r0:r1])
        yx[:, r0:r1] = o.gemm_ref(x, w[r0:r1])
        yq[:, r0:r1] = o.gemm_q8_ref(x, enc)
        encs[c] = enc

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(work, _chunks(n)))
    return encs, yx, yq


@pytest.mark.parametrize("mi", [0, 1, 2], ids=["gate", "up", "down"])
def test_q_pass_escape_stress_full(mi):
    spec = synth.WORKLOADS[4].matrices[mi]
    m = 32
    log(f"[escape stress] {spec.name} {spec.n}x{spec.k} M={m}")
    w = synth.workload_matrix(4, mi)
    x = _activations(4, mi, (m,), spec.k)[m]
    mat = w12.encode(dev16(w))
    torch.cuda.synchronize()
    rec, e_top, row_ptr, esc = download(mat)
    encs, y64, yq64 = _oracle_stress(w, x)
    # encoder: every window top, row pointer, escape entry and record byte
    per_block = (spec.k // 512) * 12288
    for (r0, r1), enc in sorted(encs.items()):
        assert np.array_equal(e_top[r0:r1], enc.e_top), r0
        assert np.array_equal(row_ptr[r0:r1 + 1] - row_ptr[r0], enc.row_ptr), r0
        assert np.array_equal(esc[row_ptr[r0]:row_ptr[r1]], enc.esc), r0
        assert np.array_equal(rec[r0 // 16 * per_block:r1 // 16 * per_block], enc.records), r0
    assert mat.n_esc == sum(e.n_esc for e in encs.values())
    log(f"  n_esc={mat.n_esc} ({mat.n_esc / w.size:.3e} of the weights)")
    del w
    xd = dev16(x)
    yf, yb = gemm_both(mat, xd)
    check_f32(yf, y64, f"stress exact {spec.name}")
    check_bf16(yb, yf, y64, f"stress exact {spec.name}")
    qf, qb = gemm_both(mat, xd, q=True)
    check_f32(qf, yq64, f"stress Q {spec.name}")
    check_bf16(qb, qf, yq64, f"stress Q {spec.name}")
    # per-row top-1 agreement of the Q pass with the exact pass
    agree_gpu = float(np.mean(np.argmax(qf, axis=1) == np.argmax(yf, axis=1)))
    agree_orc = float(np.mean(np.argmax(yq64, axis=1) == np.argmax(y64, axis=1)))
    log(f"  Q-vs-exact top-1 agreement over {m} rows: GPU {agree_gpu:.3f}, oracle {agree_orc:.3f}")
    # with the escape list applied the Q pass differs from exact only in the low mantissa bits
    qe, _ = gemm_both(mat, xd, q=True, apply_escapes=True)
    agree_esc = float(np.mean(np.argmax(qe, axis=1) == np.argmax(yf, axis=1)))
    log(f"  Q pass with escapes applied: top-1 agreement {agree_esc:.3f}")
    # the GPU's Q argmax equals the oracle's Q argmax away from near ties
    ridx, margin = o.argmax_ref(yq64)
    far = margin >= 1e-3
    assert np.array_equal(np.argmax(qf, axis=1)[far], ridx[far])
