"""W12 oracle: a plain, slow CPU statement of what the W12 path computes.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP library (it imports neither the library nor its binding) and the
library never calls it.

Source: "SpecPilot: Autonomous Algorithm Discovery and Systems Optimization for
Speculative Decoding" (arXiv 2611.02501), section 4.1 "W12: A Lossless 12-bit
Weight Format" with Figure 5, section 4.3 "Two-Level Verification" (the
zero-copy Q pass), section 2.1 (the lossless criterion) and Appendix E "W12
Details"; the Korean review of the same paper restates the format in its
section 4.1. Where those pages leave a choice open, this module fixes it; each
such reading is named ``[reading Fx]`` in a comment and listed in the design
notes of the repository.

Everything is NumPy on uint16 BF16 bit patterns; floating point reference
values are float64.

Format v1 in one paragraph. For each output channel (row) n the encoder picks
the 16-binade window [E_n - 15, E_n] that holds the most normal weights. An
in-window weight is stored as sign s, 4-bit offset off = e - (E_n - 15) and its
7 mantissa bits split as mh (top 3) and ml (low 4): 12 bits. Plane A = {s, mh},
plane E = {off}, plane B = {ml}. A and E form one byte per weight, the 8-bit
view ``v = s<<7 | off<<3 | mh``. Every other weight (outside the window, zero,
subnormal, inf, NaN) is an escape: its planes hold a placeholder and a sparse
per-row list keeps its exact bits. Weights are packed into 12 KB records of
16 rows x 512 columns: 8 KB of view bytes, then 4 KB of B nibbles.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction

import numpy as np

# --- format v1 constants ----------------------------------------------------
# SpecPilot section 4.1: a record is 12 KB and covers 8192 weights (a 128 x 64
# tile on the pages' Hopper kernel); the 8-bit view fills its first 8 KB and
# plane B the last 4 KB (section 4.3: the view is the first two thirds).
# [reading F4] this build keeps the size, the weight count and the view-first
# order, and orients the tile as 16 rows x 512 columns.
REC_ROWS = 16
REC_COLS = 512
REC_VIEW_BYTES = REC_ROWS * REC_COLS          # one byte per weight
REC_B_BYTES = REC_ROWS * REC_COLS // 2        # one nibble per weight
REC_BYTES = REC_VIEW_BYTES + REC_B_BYTES      # 12288
WINDOW = 16                                   # binades per window (section 4.1)
E_TOP_MIN = 16                                # [reading F2] window bottom >= 1
E_TOP_MAX = 254                               # largest normal exponent
Q_MIDPOINT = 8                                # [reading F7] midpoint of 4 dropped bits

ESC_DTYPE = np.dtype([("col", "<u4"), ("bits", "<u2"), ("ph", "<u2")])


# --- BF16 helpers -------------------------------------------------------------
def fields(bits: np.ndarray):
    """Split BF16 patterns into sign, 8-bit exponent field and 7-bit mantissa."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    return b >> 15, (b >> 7) & 0xFF, b & 0x7F


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of each BF16 pattern (BF16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):              # NaN payloads convert as NaN
        return u.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to BF16, nearest with ties to even, in one step.

    BF16 has 8 significant bits and fp32's exponent range: in the binade
    [2^b, 2^(b+1)) its values are spaced 2^(b-7); below 2^-126 (subnormals)
    the spacing is 2^-133. Magnitudes that round to 2^128 or above become inf.
    NaN maps to the canonical quiet NaN 0x7FC0."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    finite = np.isfinite(ax)
    _, e = np.frexp(np.where(finite, ax, 0.0))    # ax = f * 2^e, f in [0.5, 1)
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(ax / spacing) * spacing            # np.rint rounds half to even
    r = np.where(finite & (r < 2.0 ** 128), r, np.inf)
    v = np.where(np.signbit(x), -r, r)
    out = (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[np.isnan(x)] = np.uint16(0x7FC0)
    return out


# --- window choice (section 4.1) ----------------------------------------------
def window_tops(bits: np.ndarray) -> np.ndarray:
    """E_n for every row: the top of the 16-binade window covering the most
    normal weights of that row (SpecPilot section 4.1).

    [reading F2] only normal weights (exponent field 1..254) count, and the
    window [E-15, E] must lie inside the normal range, so E >= 16.
    [reading F1] ties: among the tops E in [16, max(16, e_max)] (e_max is the
    row's largest normal exponent) that reach the largest count, take the
    largest E. A row with no normal weight gets E_n = 16."""
    _, e, _ = fields(bits)
    e = np.atleast_2d(e)
    n = e.shape[0]
    normal = (e >= 1) & (e <= E_TOP_MAX)
    # histogram h[n, j] of normal exponents j = 0..255
    rows = np.broadcast_to(np.arange(n, dtype=np.int64)[:, None], e.shape)
    h = np.bincount((rows * 256 + e)[normal], minlength=n * 256).reshape(n, 256)
    # count[n, E] = h[n, E-15] + ... + h[n, E] for E = 16..254
    csum = np.concatenate([np.zeros((n, 1), np.int64), np.cumsum(h, axis=1)], axis=1)
    tops = np.arange(E_TOP_MIN, E_TOP_MAX + 1)
    count = csum[:, tops + 1] - csum[:, tops + 1 - WINDOW]
    e_max = np.where(normal.any(axis=1), np.where(normal, e, 0).max(axis=1), 0)
    cap = np.maximum(E_TOP_MIN, e_max)
    count = np.where(tops[None, :] <= cap[:, None], count, -1)
    best = count.max(axis=1)
    # largest E attaining the best count
    last = count.shape[1] - 1 - np.argmax((count == best[:, None])[:, ::-1], axis=1)
    return tops[last].astype(np.int64)


# --- encode / decode -------------------------------------------------------------
@dataclass
class Encoded:
    n: int
    k: int
    records: np.ndarray   # uint8[(n/16) * (k/512) * 12288]
    e_top: np.ndarray     # uint8[n]
    row_ptr: np.ndarray   # uint32[n + 1]
    esc: np.ndarray       # ESC_DTYPE[n_esc]

    @property
    def n_esc(self) -> int:
        return int(self.esc.shape[0])


def logical_planes(bits: np.ndarray, e_top: np.ndarray):
    """Per-weight fields (s, off, mh, ml) and the escape mask, given E_n.

    SpecPilot section 4.1: an in-window weight keeps its sign, the offset
    e - (E_n - 15) and its seven mantissa bits. Weights outside the window,
    zeros and subnormals are escapes ([reading F8]: inf and NaN too).
    [reading F5] an escape's planes hold the in-window value nearest to it with
    its sign: the largest, (s, 15, 7, 15), for escapes above the window and for
    inf/NaN; the smallest, (s, 0, 0, 0), for everything else."""
    s, e, m = fields(bits)
    E = np.asarray(e_top, dtype=np.int64)[:, None]
    lo = E - (WINDOW - 1)
    normal = (e >= 1) & (e <= E_TOP_MAX)
    inwin = normal & (e >= lo) & (e <= E)
    above = (e == 255) | (normal & (e > E))
    off = np.where(inwin, e - lo, np.where(above, 15, 0))
    mh = np.where(inwin, m >> 4, np.where(above, 7, 0))
    ml = np.where(inwin, m & 0xF, np.where(above, 15, 0))
    return s, off, mh, ml, ~inwin


def view_byte(s, off, mh):
    """[reading F3] the 8-bit view (planes A and E): sign in bit 7, the
    exponent offset in bits 6..3, the top three mantissa bits in bits 2..0."""
    return ((s << 7) | (off << 3) | mh).astype(np.uint8)


def fields_to_bf16(s, off, mh, ml, e_top):
    """BF16 pattern of the in-window value with the given fields."""
    E = np.asarray(e_top, dtype=np.int64)[:, None]
    exp = off + E - (WINDOW - 1)
    return ((s << 15) | (exp << 7) | (mh << 4) | ml).astype(np.uint16)


def pack_records(view: np.ndarray, ml: np.ndarray) -> np.ndarray:
    """[reading F4] Physical record layout, format v1.

    Records cover 16 rows x 512 columns and are stored in (row block, column
    block) row-major order. Inside a record, row r and column c = 16*G + t
    (G = 0..31, t = 0..15):
      view byte at  (G*16 + r)*16 + t
      B nibble in   8192 + (G*16 + r)*8 + (t//8)*4 + (t%4),
                    high nibble if t%8 < 4, low nibble otherwise.
    So each 16-byte view group (one row, 16 consecutive columns) has an 8-byte
    B group at the same index, and a B byte holds the nibbles of columns t and
    t+4 of the same row."""
    n, k = view.shape
    nrb, nkb = n // REC_ROWS, k // REC_COLS
    # view: [rb, r, kb, G, t] -> [rb, kb, G, r, t]
    v = view.reshape(nrb, REC_ROWS, nkb, 32, 16).transpose(0, 2, 3, 1, 4)
    v = v.reshape(nrb, nkb, REC_VIEW_BYTES)
    # B: [rb, r, kb, G, t8, half, j] with t = 8*t8 + 4*half + j
    q = ml.astype(np.uint8).reshape(nrb, REC_ROWS, nkb, 32, 2, 2, 4)
    b = (q[..., 0, :] << 4) | q[..., 1, :]            # [rb, r, kb, G, t8, j]
    b = b.transpose(0, 2, 3, 1, 4, 5).reshape(nrb, nkb, REC_B_BYTES)
    return np.concatenate([v, b], axis=2).reshape(-1)


def unpack_records(records: np.ndarray, n: int, k: int):
    """Inverse of :func:`pack_records`: per-weight view bytes and B nibbles."""
    nrb, nkb = n // REC_ROWS, k // REC_COLS
    rec = np.asarray(records, dtype=np.uint8).reshape(nrb, nkb, REC_BYTES)
    v = rec[:, :, :REC_VIEW_BYTES].reshape(nrb, nkb, 32, REC_ROWS, 16)
    view = v.transpose(0, 3, 1, 2, 4).reshape(n, k)
    b = rec[:, :, REC_VIEW_BYTES:].reshape(nrb, nkb, 32, REC_ROWS, 2, 4)
    b = b.transpose(0, 3, 1, 2, 4, 5)                 # [rb, r, kb, G, t8, j]
    ml = np.stack([b >> 4, b & 0xF], axis=-2)         # [..., t8, half, j]
    return view, ml.reshape(n, k)


def check_shape(n: int, k: int):
    if n <= 0 or k <= 0 or n % REC_ROWS or k % REC_COLS:
        raise ValueError(f"W12 needs N % {REC_ROWS} == 0 and K % {REC_COLS} == 0, got {n}x{k}")


def encode(w_bits: np.ndarray) -> Encoded:
    """Encode a BF16 matrix [N, K] (one output channel per row) into W12."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    n, k = w.shape
    check_shape(n, k)
    e_top = window_tops(w)
    s, off, mh, ml, esc_mask = logical_planes(w, e_top)
    records = pack_records(view_byte(s, off, mh), ml)
    # [reading F6] CSR by row; entries in ascending column order
    rows, cols = np.nonzero(esc_mask)                 # row-major: columns ascend per row
    row_ptr = np.zeros(n + 1, dtype=np.uint32)
    row_ptr[1:] = np.cumsum(esc_mask.sum(axis=1)).astype(np.uint32)
    ph = fields_to_bf16(s, off, mh, ml, e_top)
    esc = np.empty(rows.shape[0], dtype=ESC_DTYPE)
    esc["col"] = cols
    esc["bits"] = w[rows, cols]
    esc["ph"] = ph[rows, cols]
    return Encoded(n, k, records, e_top.astype(np.uint8), row_ptr, esc)


def _escape_rows(enc: Encoded) -> np.ndarray:
    counts = np.diff(enc.row_ptr.astype(np.int64))
    return np.repeat(np.arange(enc.n), counts)


def decode(enc: Encoded) -> np.ndarray:
    """Exact decode: rebuild every weight from its fields, then restore the
    escapes from the list (SpecPilot section 4.1: every decoded tensor must
    equal the checkpoint bit for bit)."""
    view, ml = unpack_records(enc.records, enc.n, enc.k)
    view = view.astype(np.int64)
    s, off, mh = view >> 7, (view >> 3) & 0xF, view & 0x7
    w = fields_to_bf16(s, off, mh, ml.astype(np.int64), enc.e_top.astype(np.int64))
    w[_escape_rows(enc), enc.esc["col"].astype(np.int64)] = enc.esc["bits"]
    return w


def q_view_bits(enc: Encoded) -> np.ndarray:
    """Weights the Q pass sees (SpecPilot section 4.3, zero-copy Q pass): only
    the 8-bit view is read and the four dropped mantissa bits are set to
    their midpoint. [reading F7] the midpoint is binary 1000; escapes keep
    their placeholders (the escape list is not read)."""
    view, _ = unpack_records(enc.records, enc.n, enc.k)
    view = view.astype(np.int64)
    s, off, mh = view >> 7, (view >> 3) & 0xF, view & 0x7
    return fields_to_bf16(s, off, mh, np.full_like(view, Q_MIDPOINT), enc.e_top.astype(np.int64))


def encoded_nbytes(n: int, k: int, n_esc: int) -> int:
    """Bytes of an encoded matrix: records (12 bits per weight), e_top (1 B per
    row), row_ptr (4 B per row + 4) and 8 B per escape."""
    return n * k * 3 // 2 + n + 4 * (n + 1) + 8 * n_esc


def bits_per_weight(n: int, k: int, n_esc: int) -> float:
    return 8.0 * encoded_nbytes(n, k, n_esc) / (n * k)


# --- products ----------------------------------------------------------------------
def gemm_ref(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """Y = X W^T in float64 over the original weights: the exact pass's
    product, before any rounding to the output type."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(w_bits).T


def gemm_q8_ref(x_bits: np.ndarray, enc: Encoded) -> np.ndarray:
    """Y_q = X Wq^T in float64, Wq the Q pass's view of the weights."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(q_view_bits(enc)).T


def gemm_exact_sum(x_bits: np.ndarray, w_bits: np.ndarray) -> list:
    """Exact rational Y = X W^T by brute force (tiny, finite inputs only)."""
    x = [[Fraction(float(v)) for v in row] for row in bf16_to_f64(x_bits)]
    w = [[Fraction(float(v)) for v in row] for row in bf16_to_f64(w_bits)]
    return [[sum((a * b for a, b in zip(xr, wr)), Fraction(0)) for wr in w] for xr in x]


def argmax_ref(y: np.ndarray):
    """Per row: the lowest column index attaining the maximum and the gap
    between the two largest values ([reading F10]: ties go to the lowest index;
    the margin is in logit units)."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    idx = np.argmax(y, axis=1)
    if y.shape[1] > 1:
        top2 = -np.partition(-y, 1, axis=1)[:, :2]
        margin = top2[:, 0] - top2[:, 1]
    else:
        margin = np.full(y.shape[0], np.inf)
    return idx.astype(np.int64), margin


# --- certified LM head ------------------------------------------------------------
# SpecPilot section 4.1, the certified LM head paragraph: a Q copy of the head
# plus a per-row Cauchy-Schwarz bound on its error proves which vocabulary rows
# cannot be the argmax; only the rest are rescored with the exact weights, and
# the full head runs when too many remain. [reading F16] the Q copy is the
# zero-copy 8-bit view with the escapes applied (section 4.3), so the bound
# covers the four dropped mantissa bits of in-window weights only.
def q_view_escapes_bits(enc: Encoded) -> np.ndarray:
    """The 8-bit view with every escape replaced by its exact bits."""
    q = q_view_bits(enc)
    q[_escape_rows(enc), enc.esc["col"].astype(np.int64)] = enc.esc["bits"]
    return q


def certify_bounds(enc: Encoded):
    """Per row n: r_n = ||w_n - q_n||_2 (q: the view with escapes applied),
    and a_n = ||w_n||_2 + ||v_n||_2 (v: the view with the placeholders), the
    scale of the fp32 rounding allowance. A row holding inf or NaN gets
    r_n = a_n = +inf (it can never be ruled out)."""
    w = bf16_to_f64(decode(enc))
    v = bf16_to_f64(q_view_bits(enc))
    q = bf16_to_f64(q_view_escapes_bits(enc))
    bad = ~np.isfinite(w).all(axis=1)
    w = np.where(np.isfinite(w), w, 0.0)
    q = np.where(np.isfinite(q), q, 0.0)
    r = np.sqrt(np.sum((w - q) ** 2, axis=1))
    a = np.sqrt(np.sum(w ** 2, axis=1)) + np.sqrt(np.sum(v ** 2, axis=1))
    r[bad] = np.inf
    a[bad] = np.inf
    return r, a


def certify_slack(k: int) -> float:
    """[reading F16] the fp32 rounding allowance per unit of ||x|| a_n: four
    times gamma_K = K u / (1 - K u), u = 2^-24, which bounds the rounding
    error of any fp32 summation order of K products (and of the escape
    fix-up's terms, whose magnitudes a_n also covers) with room for a
    non-round-to-nearest accumulator."""
    u = 2.0 ** -24
    return 4.0 * k * u / (1.0 - k * u)


def certified_survivors(lq: np.ndarray, r: np.ndarray, a: np.ndarray, x_norm: float, slack: float) -> np.ndarray:
    """Rows whose logit may be the largest: row n is ruled out when its upper
    bound lq_n + ||x|| (r_n + slack a_n) is below the largest lower bound
    lq_j - ||x|| (r_j + slack a_j). lq: Q-copy logits of one activation row."""
    width = x_norm * (r + slack * a)
    lower = np.where(np.isfinite(width), lq - width, -np.inf)
    best_lower = np.max(lower[~np.isnan(lower)]) if np.any(~np.isnan(lower)) else -np.inf
    upper = lq + width
    return np.flatnonzero(~(upper < best_lower))
