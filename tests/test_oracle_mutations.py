"""Planted mistakes in the oracle: every one must make a pin fail.

Each case edits the oracle's source text (a plausible slip: a flipped tie
rule, an off-by-one window, swapped fields or nibbles applied consistently to
encode and decode so that the round trip still holds, a wrong midpoint, a
dropped escape restore, a truncation for a rounding...), loads the edited
source as a separate module, and runs the pins of ``test_oracle`` against it.
The case passes when at least one pin fails. The oracle itself is never
modified; the edits live only in the loaded copy, on the CPU.
"""
import inspect
import os
import sys
import types

import pytest

import test_oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "w12_ref.py")

# (case id, [(original text, replacement, expected occurrence count)])
MUTANTS = [
    ("window_tie_smallest_top", [(
        "last = count.shape[1] - 1 - np.argmax((count == best[:, None])[:, ::-1], axis=1)",
        "last = np.argmax(count == best[:, None], axis=1)", 1)]),
    ("window_15_binades", [(
        "count = csum[:, tops + 1] - csum[:, tops + 1 - WINDOW]",
        "count = csum[:, tops + 1] - csum[:, tops + 2 - WINDOW]", 1)]),
    ("window_top_not_capped", [(
        "count = np.where(tops[None, :] <= cap[:, None], count, -1)", "count = count", 1)]),
    ("window_cap_counts_inf_and_nan", [(
        "e_max = np.where(normal.any(axis=1), np.where(normal, e, 0).max(axis=1), 0)",
        "e_max = e.max(axis=1)", 1)]),
    ("window_one_binade_low_in_planes", [(
        "inwin = normal & (e >= lo) & (e <= E)", "inwin = normal & (e >= lo - 1) & (e <= E)", 1)]),
    ("inf_nan_get_small_placeholder", [(
        "above = (e == 255) | (normal & (e > E))", "above = normal & (e > E)", 1)]),
    ("above_placeholder_mantissa_zero", [(
        "mh = np.where(inwin, m >> 4, np.where(above, 7, 0))",
        "mh = np.where(inwin, m >> 4, 0)", 1)]),
    ("view_fields_swapped_consistently", [
        ("return ((s << 7) | (off << 3) | mh).astype(np.uint8)",
         "return ((s << 7) | (mh << 4) | off).astype(np.uint8)", 1),
        ("s, off, mh = view >> 7, (view >> 3) & 0xF, view & 0x7",
         "s, off, mh = view >> 7, view & 0xF, (view >> 4) & 0x7", 2)]),
    ("view_rows_and_groups_transposed_consistently", [
        ("v = view.reshape(nrb, REC_ROWS, nkb, 32, 16).transpose(0, 2, 3, 1, 4)",
         "v = view.reshape(nrb, REC_ROWS, nkb, 32, 16).transpose(0, 2, 1, 3, 4)", 1),
        ("v = rec[:, :, :REC_VIEW_BYTES].reshape(nrb, nkb, 32, REC_ROWS, 16)\n"
         "    view = v.transpose(0, 3, 1, 2, 4).reshape(n, k)",
         "v = rec[:, :, :REC_VIEW_BYTES].reshape(nrb, nkb, REC_ROWS, 32, 16)\n"
         "    view = v.transpose(0, 2, 1, 3, 4).reshape(n, k)", 1)]),
    ("b_nibbles_swapped_consistently", [
        ("b = (q[..., 0, :] << 4) | q[..., 1, :]", "b = (q[..., 1, :] << 4) | q[..., 0, :]", 1),
        ("ml = np.stack([b >> 4, b & 0xF], axis=-2)", "ml = np.stack([b & 0xF, b >> 4], axis=-2)", 1)]),
    ("exponent_rebuilt_one_low", [(
        "exp = off + E - (WINDOW - 1)", "exp = off + E - WINDOW", 1)]),
    ("decode_skips_escape_restore", [(
        'w[_escape_rows(enc), enc.esc["col"].astype(np.int64)] = enc.esc["bits"]', "pass", 1)]),
    ("row_ptr_shifted", [(
        "row_ptr[1:] = np.cumsum(esc_mask.sum(axis=1)).astype(np.uint32)",
        "row_ptr[1:] = np.concatenate([[0], np.cumsum(esc_mask.sum(axis=1))[:-1]]).astype(np.uint32)", 1)]),
    ("placeholder_holds_original_bits", [(
        'esc["ph"] = ph[rows, cols]', 'esc["ph"] = w[rows, cols]', 1)]),
    ("q_view_truncates_instead_of_midpoint", [(
        "np.full_like(view, Q_MIDPOINT)", "np.zeros_like(view)", 1)]),
    ("q_product_uses_exact_weights", [(
        "return bf16_to_f64(x_bits) @ bf16_to_f64(q_view_bits(enc)).T",
        "return bf16_to_f64(x_bits) @ bf16_to_f64(decode(enc)).T", 1)]),
    ("gemm_drops_weight_sign", [(
        "return bf16_to_f64(x_bits) @ bf16_to_f64(w_bits).T",
        "return bf16_to_f64(x_bits) @ np.abs(bf16_to_f64(w_bits)).T", 1)]),
    ("argmax_ties_to_highest_index", [(
        "idx = np.argmax(y, axis=1)", "idx = y.shape[1] - 1 - np.argmax(y[:, ::-1], axis=1)", 1)]),
    ("argmax_margin_to_smallest", [(
        "margin = top2[:, 0] - top2[:, 1]", "margin = top2[:, 0] - y.min(axis=1)", 1)]),
    ("rounding_truncates", [(
        "r = np.rint(ax / spacing) * spacing", "r = np.floor(ax / spacing) * spacing", 1)]),
    ("rounding_subnormal_spacing", [(
        "spacing = np.ldexp(1.0, np.maximum(e - 8, -133))",
        "spacing = np.ldexp(1.0, np.maximum(e - 8, -134))", 1)]),
    ("bf16_value_shift", [(
        "u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)",
        "u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)", 1)]),
    ("size_drops_row_ptr_sentinel", [(
        "4 * (n + 1)", "4 * n", 1)]),
    ("certify_q_copy_keeps_placeholders", [(
        "q = bf16_to_f64(q_view_escapes_bits(enc))", "q = bf16_to_f64(q_view_bits(enc))", 1)]),
    ("certify_bound_squared_norm", [(
        "r = np.sqrt(np.sum((w - q) ** 2, axis=1))", "r = np.sum((w - q) ** 2, axis=1)", 1)]),
    ("certify_non_finite_rows_bounded", [(
        "    r[bad] = np.inf\n", "", 1)]),
    ("survivors_lower_bound_sign", [(
        "lower = np.where(np.isfinite(width), lq - width, -np.inf)",
        "lower = np.where(np.isfinite(width), lq + width, -np.inf)", 1)]),
    ("survivors_nan_upper_dropped", [(
        "return np.flatnonzero(~(upper < best_lower))", "return np.flatnonzero(upper >= best_lower)", 1)]),
]

# cheap pins first; a mutant stops at the first pin it breaks
_SLOW = ("test_roundtrip_config_shapes", "test_rne_matches_torch_on_fp32_inputs",
         "test_escape_fraction_and_size_orders_of_magnitude")


def _pins():
    fns = [f for name, f in inspect.getmembers(test_oracle, inspect.isfunction)
           if name.startswith("test_") and f.__module__ == test_oracle.__name__]
    fns.sort(key=lambda f: (f.__name__ in _SLOW, inspect.getsourcelines(f)[1]))
    return fns


def _load(edits):
    src = open(SRC).read()
    for old, new, count in edits:
        assert src.count(old) == count, f"mutation site not found as expected: {old!r}"
        src = src.replace(old, new)
    name = "oracle_mutant"
    mod = types.ModuleType(name)
    mod.__file__ = SRC
    sys.modules[name] = mod          # dataclasses look the module up while the class is built
    try:
        exec(compile(src, SRC, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


def _failing_pin(mod, monkeypatch):
    monkeypatch.setattr(test_oracle, "o", mod)
    for fn in _pins():
        try:
            fn()
        except pytest.skip.Exception:
            continue
        except Exception:            # an assertion, or the mutant breaking a shape
            return fn.__name__
    return None


def test_unmutated_copy_passes_every_pin(monkeypatch):
    assert _failing_pin(_load([]), monkeypatch) is None


@pytest.mark.parametrize("edits", [m[1] for m in MUTANTS], ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(edits, monkeypatch):
    assert _failing_pin(_load(edits), monkeypatch) is not None, "no pin caught this mistake"
