"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one slip in a private copy of the oracle's source (never in
the oracle itself, never on the GPU), runs the pin suite of
test_oracle_pins.py against that copy, and requires at least one pin to fail.
The slips are the kinds a reader could make when writing the method from the
pages: a dropped term, a wrong sign or index, the scale applied to the wrong
operand, the group taken along the wrong axis, a wrong rounding mode, the
wrong code offset or nibble order.
"""
from __future__ import annotations

import inspect
import os
import types

import pytest

import tests.test_oracle_pins as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "awq_oracle.py")

# (name, text in the oracle, replacement)
MUTATIONS = [
    ("stat_max_not_mean", "col_sum = np.abs(X.astype(np.float64)).sum(axis=0)",
     "col_sum = np.abs(X.astype(np.float64)).max(axis=0) * N"),
    ("stat_no_abs", "col_sum = np.abs(X.astype(np.float64)).sum(axis=0)",
     "col_sum = X.astype(np.float64).sum(axis=0)"),
    ("stat_divides_by_n_minus_1", "return (col_sum / np.float64(N)).astype(np.float32)",
     "return (col_sum / np.float64(max(N - 1, 1))).astype(np.float32)"),
    ("scale_exponent_one_minus_alpha", "flat_o[j] = np.float32(math.pow(aj, al))",
     "flat_o[j] = np.float32(math.pow(aj, 1.0 - al))"),
    ("scale_inverted", "flat_o[j] = np.float32(math.pow(aj, al))",
     "flat_o[j] = np.float32(1.0 / math.pow(aj, al))"),
    ("qmax_without_minus_one", "qmax = np.float32(2 ** (bits - 1) - 1)", "qmax = np.float32(2 ** (bits - 1))"),
    ("group_along_columns", "m = np.abs(Wp).reshape(G, group, D_out).max(axis=1)",
     "m = np.abs(Wp).reshape(D_in // group, group, D_out).max(axis=1).max(axis=0, keepdims=True).repeat(G, 0)"),
    ("round_half_up", "q = np.rint(ratio)", "q = np.floor(ratio + np.float32(0.5))"),
    ("truncate_not_round", "q = np.rint(ratio)", "q = np.trunc(ratio)"),
    ("reciprocal_multiply", "ratio = (Wp / safe).astype(np.float32)",
     "ratio = (Wp * (np.float32(1.0) / safe)).astype(np.float32)"),
    ("loss_without_inverse_scale", "Xs = X64 / np.asarray(s, dtype=np.float64)[None, :]", "Xs = X64"),
    ("loss_scale_multiplied", "Xs = X64 / np.asarray(s, dtype=np.float64)[None, :]",
     "Xs = X64 * np.asarray(s, dtype=np.float64)[None, :]"),
    ("loss_sign", "E = Xs @ What - Y", "E = Xs @ What + Y"),
    ("loss_not_squared", "return float(np.sum(E * E))", "return float(np.sqrt(np.sum(E * E)))"),
    ("argmin_last_tie", "if losses[k] < losses[best]:", "if losses[k] <= losses[best]:"),
    ("pack_plain_order", "PACK_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)", "PACK_ORDER = (0, 1, 2, 3, 4, 5, 6, 7)"),
    ("pack_offset_seven", "def pack_int4(q: np.ndarray, offset: int = 8)", "def pack_int4(q: np.ndarray, offset: int = 7)"),
    ("pack_msb_first", "word |= nib[:, row, :].astype(np.uint64) << np.uint64(4 * slot)",
     "word |= nib[:, row, :].astype(np.uint64) << np.uint64(4 * (7 - slot))"),
    ("bf16_ties_up", "up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & np.uint64(1)) == 1))",
     "up = rest >= 0x8000"),
    ("stat_max_is_min", "return np.abs(X.astype(np.float64)).max(axis=0).astype(np.float32)",
     "return np.abs(X.astype(np.float64)).min(axis=0).astype(np.float32)"),
    ("stat_max_without_abs", "return np.abs(X.astype(np.float64)).max(axis=0).astype(np.float32)",
     "return X.astype(np.float64).max(axis=0).astype(np.float32)"),
    ("weight_stat_along_columns", "row_sum = np.abs(W.astype(np.float64)).sum(axis=1)",
     "row_sum = np.abs(W.astype(np.float64)).sum(axis=0)[: W.shape[0]]"),
    ("weight_stat_no_mean", "return (row_sum / np.float64(W.shape[1])).astype(np.float32)",
     "return row_sum.astype(np.float32)"),
    ("weight_term_exponent_alpha", "flat_o[j] = np.float32(math.pow(aj, al) / math.pow(bj, 1.0 - al))",
     "flat_o[j] = np.float32(math.pow(aj, al) / math.pow(bj, al))"),
    ("weight_term_multiplied", "flat_o[j] = np.float32(math.pow(aj, al) / math.pow(bj, 1.0 - al))",
     "flat_o[j] = np.float32(math.pow(aj, al) * math.pow(bj, 1.0 - al))"),
    ("clip_ratio_ignored", "mr = (np.float32(ratio) * m).astype(np.float32)", "mr = m"),
    ("clip_no_saturation", "    q = np.clip(q, -qmax, qmax)\n    return q.astype(np.int8), delta\n\n\ndef clip_search",
     "    return q.astype(np.int8), delta\n\n\ndef clip_search"),
    ("clip_error_without_inverse_scale", "D = What / s64[:, None] - W64", "D = What - W64"),
    ("clip_error_sums_columns", "errors[k, g, :] = np.sum(E * E, axis=0)",
     "errors[k, g, :] = np.sum(E * E)"),
    ("clip_error_other_group", "E = X64[:, rows] @ D[rows, :]",
     "E = X64[:, rows] @ D[slice(((g + 1) % G) * group, ((g + 1) % G + 1) * group), :]"),
    ("asym_range_without_zero", "lo = np.minimum(blocks.min(axis=1), np.float32(0.0))", "lo = blocks.min(axis=1)"),
    ("asym_signed_levels", "qu = np.float32(2 ** bits - 1)\n    G = D_in // group\n    blocks",
     "qu = np.float32(2 ** (bits - 1) - 1)\n    G = D_in // group\n    blocks"),
    ("asym_zero_truncated", "z = np.where(step > 0, np.rint((-lo / safe).astype(np.float32)), np.float32(0.0))",
     "z = np.where(step > 0, np.trunc((-lo / safe).astype(np.float32)), np.float32(0.0))"),
    ("asym_zero_not_added", "q = np.rint((Wp / sfull).astype(np.float32)) + zfull",
     "q = np.rint((Wp / sfull).astype(np.float32))"),
    ("asym_dequant_plus_zero", "return (q.astype(np.float64) - zf) * np.repeat(step.astype(np.float64), group, axis=0)",
     "return (q.astype(np.float64) + zf) * np.repeat(step.astype(np.float64), group, axis=0)"),
    ("f16_steps_ignored", "    if f16_steps:\n        delta = round_to_f16(delta)", "    if f16_steps:\n        pass"),
    ("f16_round_toward_zero", "        return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)",
     "        return (np.asarray(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFFE000)).view(np.float32)"),
    ("gemm_scale_not_inverse", "Xe = round_to_bf16((X * np.asarray(inv_s, dtype=np.float32)[None, :]).astype(np.float32))",
     "Xe = round_to_bf16((X / np.asarray(inv_s, dtype=np.float32)[None, :]).astype(np.float32))"),
]


def _pin_calls():
    """Every pin test of test_oracle_pins.py with each of its parameter sets."""
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != pins.__name__:
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            calls.append((name, fn, {}))
            continue
        argnames, values = marks[0].args[0], marks[0].args[1]
        argnames = [a.strip() for a in argnames.split(",")] if isinstance(argnames, str) else list(argnames)
        for v in values:
            v = v if isinstance(v, (tuple, list)) else (v,)
            calls.append((f"{name}{tuple(v)}", fn, dict(zip(argnames, v))))
    return calls


def _mutant(old: str, new: str) -> types.ModuleType:
    src = open(SRC_PATH).read()
    assert src.count(old) >= 1, f"mutation target not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC_PATH
    exec(compile(src.replace(old, new, 1), SRC_PATH + " (mutant)", "exec"), mod.__dict__)
    return mod


def test_unmutated_oracle_passes_every_pin(monkeypatch):
    monkeypatch.setattr(pins, "oracle", _mutant("PACK_ORDER", "PACK_ORDER"))
    for name, fn, kw in _pin_calls():
        fn(**kw)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, old, new):
    monkeypatch.setattr(pins, "oracle", _mutant(old, new))
    failed = []
    for pin, fn, kw in _pin_calls():
        try:
            with pytest.MonkeyPatch.context():
                fn(**kw)
        except AssertionError:
            failed.append(pin)
            break
    assert failed, f"no pin caught the planted mistake {name}"
