"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: exhaustive
round trips, brute force, closed forms written with float arithmetic instead
of bit fields, torch's BF16 rounding, hand-derived bytes and the pages'
published statistics (SpecPilot, arXiv 2611.02501, section 4.1, Figure 5,
section 4.3, Appendix E)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as o
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- BF16 rounding ----------------------------------------------------------------
def test_rne_matches_torch_on_fp32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    # random fp32 bit patterns of every class except NaN
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.f64_to_bf16_rne(x.astype(np.float64)), ref)


def test_rne_ties_and_edges():
    # midpoints between consecutive BF16 values go to the even mantissa
    lo = np.arange(0x3F80, 0x4000, dtype=np.uint16)
    a, b = o.bf16_to_f64(lo), o.bf16_to_f64(lo + 1)
    got = o.f64_to_bf16_rne((a + b) / 2)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    # just above the midpoint rounds up, just below rounds down
    assert np.array_equal(o.f64_to_bf16_rne(np.nextafter((a + b) / 2, np.inf)), lo + 1)
    assert np.array_equal(o.f64_to_bf16_rne(np.nextafter((a + b) / 2, -np.inf)), lo)
    # overflow: the largest finite BF16 is (2 - 2^-7) 2^127; its midpoint to 2^128 ties to inf
    big = (2 - 2 ** -7) * 2.0 ** 127
    assert o.f64_to_bf16_rne(np.array([big]))[0] == 0x7F7F
    assert o.f64_to_bf16_rne(np.array([(2 - 2 ** -8) * 2.0 ** 127]))[0] == 0x7F80
    assert o.f64_to_bf16_rne(np.array([-np.inf]))[0] == 0xFF80
    # subnormal BF16: spacing 2^-133, half the smallest subnormal ties to zero
    assert o.f64_to_bf16_rne(np.array([2.0 ** -134]))[0] == 0x0000
    assert o.f64_to_bf16_rne(np.array([3 * 2.0 ** -134]))[0] == 0x0002
    assert o.f64_to_bf16_rne(np.array([-0.0]))[0] == 0x8000
    # values exactly representable come back unchanged
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(o.bf16_to_f64(allb))
    assert np.array_equal(o.f64_to_bf16_rne(o.bf16_to_f64(allb[finite])), allb[finite])


def test_bf16_to_f64_closed_form():
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = o.bf16_to_f64(allb)
    for b in [0x0000, 0x8000, 0x0001, 0x007F, 0x0080, 0x3F80, 0xBFC0, 0x4049, 0x7F7F, 0x7F80, 0xFF80]:
        s, e, m = b >> 15, (b >> 7) & 0xFF, b & 0x7F
        if e == 255:
            want = -math.inf if s else math.inf
        elif e == 0:
            want = (-1) ** s * m * 2.0 ** (-133)
        else:
            want = (-1) ** s * (1 + m / 128) * 2.0 ** (e - 127)
        assert v[b] == want, hex(b)
    assert np.isnan(v[0x7FC0]) and np.isnan(v[0xFFC1])


# --- window choice -----------------------------------------------------------------
def _brute_window(row_bits):
    """Directly count, for every candidate top E in [16, 254], the normal
    weights whose exponent lies in [E-15, E]."""
    e = [(int(b) >> 7) & 0xFF for b in row_bits]
    normal = [1 <= x <= 254 for x in e]
    counts = {E: sum(1 for x, nm in zip(e, normal) if nm and E - 15 <= x <= E) for E in range(16, 255)}
    emax = max([x for x, nm in zip(e, normal) if nm], default=0)
    return counts, emax


def _adversarial_rows(rng, k):
    rows = []
    for _ in range(60):
        kind = rng.integers(0, 6)
        if kind == 0:   # two clusters exactly 16 binades apart: ties
            e = rng.choice([100, 116], size=k)
        elif kind == 1:  # uniform over all exponents, all classes
            e = rng.integers(0, 256, size=k)
        elif kind == 2:  # tiny exponents near the bottom of the normal range
            e = rng.integers(0, 20, size=k)
        elif kind == 3:  # wide spread
            e = rng.integers(60, 200, size=k)
        elif kind == 4:  # all zero / subnormal
            e = np.zeros(k, dtype=np.int64)
        else:            # gaussian-like
            e = np.clip(np.round(rng.normal(120, 3, size=k)), 0, 255).astype(np.int64)
        s = rng.integers(0, 2, size=k)
        m = rng.integers(0, 128, size=k)
        rows.append(((s << 15) | (e << 7) | m).astype(np.uint16))
    return np.stack(rows)


def test_window_against_brute_force():
    rng = np.random.default_rng(2)
    rows = np.concatenate([_adversarial_rows(rng, 64),
                           synth.random_bits((40, 64), 3),
                           synth.workload_matrix(0, 0)[:24, :64]])
    tops = o.window_tops(rows)
    for row, E in zip(rows, tops):
        counts, emax = _brute_window(row)
        best = max(counts.values())
        assert counts[int(E)] == best                    # the window covers the most weights
        cap = max(16, emax)
        assert 16 <= E <= cap
        # ties: the largest maximal top not above the cap
        assert all(counts[x] < best for x in range(int(E) + 1, cap + 1))


def test_window_all_escape_row_and_ties():
    zeros = np.zeros((1, 512), dtype=np.uint16)
    assert o.window_tops(zeros)[0] == 16
    # 256 weights at exponent 100 and 256 at 116: tops 100..115 hold 256, 116 holds 256 too
    row = np.array([[100 << 7] * 256 + [116 << 7] * 256], dtype=np.uint16)
    assert o.window_tops(row)[0] == 116
    # a narrow cluster (exponents 100..103): every top from 103 to 115 covers all
    # of it, and the tie goes to the largest normal exponent, 103; inf, NaN, zero
    # and subnormal weights in the row do not move that cap
    base = [(100 + i % 4) << 7 | (i % 128) for i in range(508)]
    row = np.array([base + [0x7F80, 0xFFC0, 0x0000, 0x0005]], dtype=np.uint16)
    assert o.window_tops(row)[0] == 103


# --- escapes and fields --------------------------------------------------------------
def _mixed_matrix():
    return np.concatenate([synth.all_bf16_patterns(512),
                           synth.workload_matrix(0, 0)[:128, :512],
                           synth.random_bits((128, 512), 9)])


def test_escape_set_closed_form():
    w = _mixed_matrix()
    enc = o.encode(w)
    e = (w.astype(np.int64) >> 7) & 0xFF
    E = enc.e_top.astype(np.int64)[:, None]
    expect = (e < E - 15) | (e > E) | (e == 0) | (e == 255)
    got = np.zeros_like(expect)
    rows = np.repeat(np.arange(w.shape[0]), np.diff(enc.row_ptr.astype(np.int64)))
    got[rows, enc.esc["col"].astype(np.int64)] = True
    assert np.array_equal(got, expect)
    # per row: escapes = K - (normal weights inside the chosen window)
    normal = (e >= 1) & (e <= 254)
    inwin = normal & (e >= E - 15) & (e <= E)
    assert np.array_equal(np.diff(enc.row_ptr.astype(np.int64)), w.shape[1] - inwin.sum(axis=1))
    # columns ascend within each row and escape bits are the original ones
    for n in range(w.shape[0]):
        a, b = enc.row_ptr[n], enc.row_ptr[n + 1]
        cols = enc.esc["col"][a:b].astype(np.int64)
        assert np.all(np.diff(cols) > 0)
        assert np.array_equal(enc.esc["bits"][a:b], w[n, cols])


def test_roundtrip_every_bf16_pattern():
    # SpecPilot section 4.1: every decoded tensor equals the original bit for bit
    w = _mixed_matrix()
    rng = np.random.default_rng(4)
    for trial in range(3):
        ww = w[rng.permutation(w.shape[0])] if trial else w
        enc = o.encode(ww)
        assert np.array_equal(o.decode(enc), ww)


def test_roundtrip_config_shapes():
    for wl, mi in [(0, 0), (4, 0), (4, 2)]:
        w = synth.workload_matrix(wl, mi, rows=slice(0, 256))
        assert np.array_equal(o.decode(o.encode(w)), w)


def test_view_and_b_values_closed_form():
    """The view byte of an in-window weight, read as a sign / 4-bit exponent
    offset / 3-bit mantissa minifloat with the row's window, is the weight
    truncated toward zero to 4 significant bits; adding the B nibble times
    2^(e-127-7) gives the weight back (section 4.1, Figure 5)."""
    w = synth.workload_matrix(0, 0)[:64]
    enc = o.encode(w)
    view, ml = o.unpack_records(enc.records, enc.n, enc.k)
    x = o.bf16_to_f64(w)
    esc = np.zeros(w.shape, bool)
    rows = np.repeat(np.arange(w.shape[0]), np.diff(enc.row_ptr.astype(np.int64)))
    esc[rows, enc.esc["col"].astype(np.int64)] = True
    E = enc.e_top.astype(np.float64)[:, None]
    v = view.astype(np.int64)
    sign = np.where(v >= 128, -1.0, 1.0)
    off = (v // 8) % 16
    mh = v % 8
    vval = sign * 2.0 ** (off + E - 15 - 127) * (1 + mh / 8)
    mag = np.abs(x)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    trunc = np.sign(x) * np.floor(mag / 2.0 ** (ex - 3)) * 2.0 ** (ex - 3)
    ok = ~esc
    assert np.array_equal(vval[ok], trunc[ok])
    assert np.array_equal((vval + sign * ml * 2.0 ** (off + E - 15 - 127 - 7))[ok], x[ok])


def test_placeholders_are_nearest_in_window_values():
    w = _mixed_matrix()
    enc = o.encode(w)
    rows = np.repeat(np.arange(w.shape[0]), np.diff(enc.row_ptr.astype(np.int64)))
    E = enc.e_top.astype(np.int64)[rows]
    ph = o.bf16_to_f64(enc.esc["ph"])
    big = (2 - 2 ** -7) * 2.0 ** (E - 127)       # largest in-window magnitude
    small = 2.0 ** (E - 15 - 127)                 # smallest in-window magnitude
    val = o.bf16_to_f64(enc.esc["bits"])
    sign = np.where(enc.esc["bits"] >= 0x8000, -1.0, 1.0)
    above = np.isnan(val) | (np.abs(val) > big)
    assert np.array_equal(ph, np.where(above, sign * big, sign * small))


def test_layout_golden_record():
    g = _golden("layout_v1.json")
    w = np.full((16, 512), int(g["base_bits"], 16), dtype=np.uint16)
    for ov in g["overrides"]:
        w[ov["r"], ov["c"]] = int(ov["bits"], 16)
    enc = o.encode(w)
    for item in g["e_top"]:
        assert enc.e_top[item["r"]] == item["value"], item["why"]
    for item in g["view_bytes"] + g["b_bytes"]:
        assert enc.records[item["pos"]] == int(item["value"], 16), item["why"]
    got = [(int(np.searchsorted(enc.row_ptr, i, side="right") - 1), int(e["col"]), int(e["bits"]), int(e["ph"]))
           for i, e in enumerate(enc.esc)]
    want = [(x["r"], x["col"], int(x["bits"], 16), int(x["ph"], 16)) for x in g["escapes"]]
    assert got == want


def test_record_geometry_matches_pages():
    g = _golden("pages_w12_facts.json")
    assert o.REC_BYTES == g["record_bytes"]["value"]
    assert o.REC_ROWS * o.REC_COLS == g["record_weights"]["value"]
    assert o.REC_VIEW_BYTES == g["view_bytes"]["value"]
    num, den = g["view_fraction"]["value"]
    assert Fraction(o.REC_VIEW_BYTES, o.REC_BYTES) == Fraction(num, den)
    assert o.WINDOW == g["window_binades"]["value"]
    # 1 sign + 4 offset + 7 mantissa bits; the view is A + E = 8 bits
    assert 1 + 4 + 7 == g["bits_in_window"]["value"] and 1 + 3 + 4 == g["view_bits"]["value"]
    # the record stores exactly 12 bits per weight
    assert o.REC_BYTES * 8 == 12 * o.REC_ROWS * o.REC_COLS


def test_escape_fraction_and_size_orders_of_magnitude():
    """Well-behaved per-channel weights escape at ~1e-4 and cost ~12.01 bits
    (Figure 5, section 4.1, Appendix E)."""
    g = _golden("pages_w12_facts.json")
    w = synth.plain_gaussian(1024, 5120, seed=11)
    enc = o.encode(w)
    frac = enc.n_esc / w.size
    assert 1e-5 < frac < g["escape_fraction_upper"]["value"]
    bpw = o.bits_per_weight(1024, 5120, enc.n_esc)
    lo, hi = g["bits_per_weight_dense_models"]["value"]
    assert 12.0 < bpw < hi + 0.005 and abs(bpw - lo) < 0.01
    # sizes: the closed form equals the arrays' actual byte counts
    actual = enc.records.nbytes + enc.e_top.nbytes + enc.row_ptr.nbytes + enc.esc.nbytes
    assert actual == o.encoded_nbytes(1024, 5120, enc.n_esc)
    # the pages' converted-layer shrink is 12/16 up to metadata and escapes
    a, b = g["converted_gb"]["value"]
    assert abs(b / a - 12 / 16) < 0.01


# --- products -------------------------------------------------------------------------
def test_gemm_ref_equals_exact_rational_sum():
    rng = np.random.default_rng(5)
    w = synth.workload_matrix(0, 0)[:16, :512][:, :48]
    x = synth.make_activations(3, 48, seed=6)
    y = o.gemm_ref(x, w)
    exact = o.gemm_exact_sum(x, w)
    xa, wa = np.abs(o.bf16_to_f64(x)), np.abs(o.bf16_to_f64(w))
    bound = 48 * 2.0 ** -53 * (xa @ wa.T)
    for i in range(3):
        for j in range(16):
            assert abs(Fraction(float(y[i, j])) - exact[i][j]) <= Fraction(float(bound[i, j]))
    # a planted case with an exactly known answer
    xs = np.array([[0x3F80, 0x4000, 0xC040]], dtype=np.uint16)     # 1, 2, -3
    ws = np.array([[0x3F00, 0x3E80, 0x3F80]], dtype=np.uint16)     # 0.5, 0.25, 1
    assert o.gemm_ref(xs, ws)[0, 0] == 0.5 + 0.5 - 3.0
    del rng


def test_gemm_onehot_rows_reproduce_weights():
    w = synth.workload_matrix(0, 0)[:64]
    k = w.shape[1]
    cols = [0, 1, 37, 511, 512, 1023]
    x = np.zeros((len(cols), k), dtype=np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = 0x3F80 if i % 2 == 0 else 0x4100      # 1.0 or 8.0
    y = o.gemm_ref(x, w)
    for i, c in enumerate(cols):
        scale = 1.0 if i % 2 == 0 else 8.0
        assert np.array_equal(y[i], scale * o.bf16_to_f64(w[:, c]))


def test_q_view_equals_exact_when_low_bits_are_midpoint():
    """If every weight is in its window and already has low nibble 1000, the
    Q view loses nothing (section 4.3, midpoint rule)."""
    w = synth.plain_gaussian(32, 1024, seed=12)
    w = (w & 0xFFF0) | 0x0008
    enc = o.encode(w)
    q = o.q_view_bits(enc)
    esc = np.zeros(w.shape, bool)
    rows = np.repeat(np.arange(w.shape[0]), np.diff(enc.row_ptr.astype(np.int64)))
    esc[rows, enc.esc["col"].astype(np.int64)] = True
    assert np.array_equal(q[~esc], w[~esc])
    x = synth.make_activations(4, 1024, seed=13)
    if enc.n_esc == 0:
        assert np.array_equal(o.gemm_q8_ref(x, enc), o.gemm_ref(x, w))


def test_q_view_closed_form():
    w = _mixed_matrix()
    enc = o.encode(w)
    q = o.bf16_to_f64(o.q_view_bits(enc))
    x = o.bf16_to_f64(w)
    view, _ = o.unpack_records(enc.records, enc.n, enc.k)
    E = enc.e_top.astype(np.float64)[:, None]
    v = view.astype(np.int64)
    sign = np.where(v >= 128, -1.0, 1.0)
    want = sign * 2.0 ** ((v // 8) % 16 + E - 15 - 127) * (1 + (v % 8) / 8 + 8 / 128)
    assert np.array_equal(q, want)
    # on in-window weights the Q value is within half of the dropped range
    esc = np.zeros(w.shape, bool)
    rows = np.repeat(np.arange(w.shape[0]), np.diff(enc.row_ptr.astype(np.int64)))
    esc[rows, enc.esc["col"].astype(np.int64)] = True
    ok = ~esc
    ulp4 = 2.0 ** ((v // 8) % 16 + E - 15 - 127 - 3)
    assert np.all(np.abs(q - x)[ok] <= (ulp4 / 2)[ok])


def test_gemm_q8_ref_brute_force():
    """The Q pass product on a tiny matrix with escapes: an exact rational sum
    over weights written from the view bytes by the midpoint rule, with each
    escape's placeholder in place of its value (section 4.3, zero-copy Q pass).
    """
    w = _mixed_matrix()[:16].copy()
    w[:, 40:] = synth.workload_matrix(0, 0)[:16, 40:512]
    enc = o.encode(w)
    assert enc.n_esc > 0
    view, _ = o.unpack_records(enc.records, enc.n, enc.k)
    cols = 48
    x = synth.make_activations(2, 512, seed=14)
    x[:, cols:] = 0
    xv = o.bf16_to_f64(x)
    want = [[Fraction(0)] * 16 for _ in range(2)]
    bound = np.zeros((2, 16))
    for n in range(16):
        E = int(enc.e_top[n])
        for c in range(cols):
            v = int(view[n, c])
            q = Fraction(-1 if v >= 128 else 1) * Fraction(2) ** ((v >> 3) % 16 + E - 15 - 127) * \
                (1 + Fraction(v % 8, 8) + Fraction(8, 128))
            for i in range(2):
                want[i][n] += Fraction(float(xv[i, c])) * q
                bound[i, n] += abs(float(xv[i, c]) * float(q))
    got = o.gemm_q8_ref(x, enc)
    for i in range(2):
        for n in range(16):
            err = abs(Fraction(float(got[i, n])) - want[i][n])
            assert err <= Fraction(cols * 2.0 ** -53 * bound[i, n]), (i, n)
    # the placeholders, not the escapes' own values, enter the Q product
    hit = enc.esc["col"] < cols
    assert np.any(enc.esc["bits"][hit] != enc.esc["ph"][hit])


def test_argmax_planted_winners():
    rng = np.random.default_rng(7)
    y = rng.normal(size=(5, 1000))
    winners = [3, 999, 0, 500, 42]
    for i, j in enumerate(winners):
        y[i, j] = y[i].max() + 0.25
    idx, margin = o.argmax_ref(y)
    assert list(idx) == winners
    assert np.allclose(margin, 0.25)
    tie = np.zeros((1, 8))
    tie[0, [2, 5]] = 1.0
    idx, margin = o.argmax_ref(tie)
    assert idx[0] == 2 and margin[0] == 0.0


# --- certified LM head (section 4.1, certified LM head paragraph) --------------
def test_certify_bounds_zero_when_low_bits_are_midpoint():
    """Every in-window weight already at the midpoint nibble and escapes
    restored exactly: the Q copy equals the weights, so r = 0, and a is twice
    the row norm (view and weights agree)."""
    w = synth.plain_gaussian(32, 1024, seed=12)
    w = (w & 0xFFF0) | 0x0008
    w[3, 7] = 0                       # an escape (zero) in a row
    w[5, 9] = w[5, 9] + (30 << 7)     # an escape far above the window
    enc = o.encode(w)
    assert enc.n_esc >= 2
    r, a = o.certify_bounds(enc)
    assert np.all(r == 0.0)
    wf = o.bf16_to_f64(w)
    clean = [i for i in range(32) if i not in (3, 5)]
    assert np.allclose(a[clean], 2 * np.sqrt((wf[clean] ** 2).sum(1)), rtol=1e-15)


def test_certify_bounds_closed_form_single_weight():
    """One weight off the midpoint by d nibble steps at exponent e: the Q copy
    differs only there, by d * 2^(e - 7), so r is that amount exactly."""
    base = np.full((16, 512), 0x3F88, np.uint16)     # 1.0625: exponent 127, nibble 8
    for d, (row, col) in zip((-8, -1, 1, 7), ((0, 0), (1, 100), (2, 511), (3, 250))):
        base[row, col] = 0x3F80 | (8 + d)            # nibble 8 + d
    base[4, 3] = 0x4088 | 0x3                        # exponent 129, nibble 11: d = 3
    enc = o.encode(base)
    assert enc.n_esc == 0
    r, _ = o.certify_bounds(enc)
    want = np.zeros(16)
    want[:4] = np.abs([-8, -1, 1, 7]) * 2.0 ** -7
    want[4] = 3 * 2.0 ** (2 - 7)
    assert np.array_equal(r, want)


def test_certify_bounds_cauchy_schwarz_and_non_finite():
    """|x.w - x.q| <= ||x|| r on random rows, with equality when x points along
    w - q; a row with inf or NaN gets infinite bounds."""
    w = synth.workload_matrix(0, 0)[:64].copy()
    w[10, 5] = 0x7F80
    w[11, 6] = 0x7FC1
    enc = o.encode(w)
    r, a = o.certify_bounds(enc)
    assert np.isinf(r[10]) and np.isinf(r[11]) and np.isinf(a[10]) and np.isinf(a[11])
    fin = np.isfinite(r)
    wf = o.bf16_to_f64(w)[fin]
    q = o.bf16_to_f64(o.q_view_escapes_bits(enc))[fin]
    rng = np.random.default_rng(3)
    for _ in range(20):
        x = rng.normal(size=1024)
        assert np.all(np.abs((wf - q) @ x) <= np.linalg.norm(x) * r[fin] * (1 + 1e-12))
    d = wf[0] - q[0]
    assert math.isclose(abs(d @ d), np.linalg.norm(d) * r[fin][0], rel_tol=1e-12)


def test_certified_survivors_keep_the_argmax():
    """The rows kept always include the true argmax; with a zero bound and no
    rounding allowance only the argmax survives (distinct logits)."""
    rng = np.random.default_rng(11)
    for trial in range(50):
        n = 300
        l = rng.normal(size=n) * 3
        r = np.abs(rng.normal(size=n)) * 0.02
        x_norm = 10.0
        err = rng.uniform(-1, 1, size=n) * x_norm * r          # any error within the bound
        lq = l - err
        keep = o.certified_survivors(lq, r, np.ones(n), x_norm, 0.0)
        assert int(np.argmax(l)) in keep
        assert len(o.certified_survivors(l, np.zeros(n), np.ones(n), x_norm, 0.0)) == 1
    # an infinite bound (non-finite row) is never ruled out and rules nothing out
    lq = np.array([1.0, 5.0, 2.0])
    keep = o.certified_survivors(lq, np.array([0.0, 0.0, np.inf]), np.ones(3), 1.0, 0.0)
    assert list(keep) == [1, 2]
    # a NaN logit (a row holding NaN) gives a NaN upper bound: kept, not dropped
    keep = o.certified_survivors(np.array([1.0, 5.0, np.nan]), np.array([0.0, 0.0, np.inf]), np.ones(3), 1.0, 0.0)
    assert list(keep) == [1, 2]
    assert o.certify_slack(5120) == pytest.approx(4 * 5120 * 2.0 ** -24, rel=1e-3)
