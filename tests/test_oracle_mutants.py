"""The oracle's pins are strong enough to catch plausible mistakes (CPU only).

Each case plants one mistake in a *copy* of the oracle -- a C source edit
compiled into a temporary library, or a replaced Python function -- and runs
the pin tests against it.  At least one pin must fail for every mistake.  The
real oracle is never modified.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, mutated text): each is a mistake a careful reader
# could plausibly make when writing the oracle from the pages.
C_MUTANTS = [
    ("nibble_order_reversed", "unsigned shift = (unsigned)(4 * (k % 8));",
     "unsigned shift = (unsigned)(4 * (7 - k % 8));"),
    ("nibble_mask_three_bits", "return (unsigned)((word >> shift) & 15u);",
     "return (unsigned)((word >> shift) & 7u);"),
    ("group_index_halved", "double s = scales[o * groups + k / group];",
     "double s = scales[o * groups + (k / group) / 2];"),
    ("bias_dropped", "return s * q + b;", "return s * q;"),
    ("bias_sign", "return s * q + b;", "return s * q - b;"),
    ("scale_on_bias", "return s * q + b;", "return s * (q + b);"),
    ("first_term_skipped",
     "double term = weight_at(codes, scales, biases, o, k, k_in, group) * x[k];",
     "double term = (k == 0) ? 0.0 : weight_at(codes, scales, biases, o, k, k_in, group) * x[k];"),
    ("gemm_output_transposed", "Y[t * n_out + o] = acc;", "Y[o * T + t] = acc;"),
    ("bf16_round_truncates", "double r = nearbyint(ldexp(m, 8));", "double r = trunc(ldexp(m, 8));"),
    ("bf16_round_wrong_width", "double r = nearbyint(ldexp(m, 8));\n    return ldexp(r, e - 8);",
     "double r = nearbyint(ldexp(m, 9));\n    return ldexp(r, e - 9);"),
]

# Fast pins that exercise the C oracle.
C_PINS = [
    (pins.test_unpack_golden_words, {}),
    (pins.test_unpack_roundtrip_bit_exact, {"shape": (3, 64)}),
    (pins.test_one_hot_input_selects_weight, {"group": 32}),
    (pins.test_one_hot_identity_probe_recovers_codes, {}),
    (pins.test_all_zero_codes_give_bias_rows, {"group": 32}),
    (pins.test_constant_codes_closed_form, {}),
    (pins.test_bruteforce_multi_group_128, {}),
    (pins.test_gemm_identity_recovers_codes, {}),
    (pins.test_gemm_bruteforce_small_exact, {}),
    (pins.test_round_bf16_matches_torch_cast, {}),
    (pins.test_gemm_rows_match_gemv_with_rounded_weights, {}),
]


def _failures(pin_list):
    failed = []
    for fn, kw in pin_list:
        try:
            fn(**kw)
        except AssertionError:
            failed.append(fn.__name__)
    return failed


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    mutated = src.replace(old, new)
    c_path = tmp_path / ("%s.c" % name)
    so_path = tmp_path / ("lib%s.so" % name)
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-shared", "-fPIC", "-std=c11", str(c_path), "-o",
                    str(so_path), "-lm"], check=True)
    return str(so_path)


def test_real_oracle_passes_the_pin_subset():
    assert _failures(C_PINS) == []


@pytest.mark.parametrize("name,old,new", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_c_mutant_is_caught(tmp_path, monkeypatch, name, old, new):
    so = _build_mutant(tmp_path, name, old, new)
    real = oracle._load()
    mutant = ctypes.CDLL(so)
    # reuse the real library's prototypes for the mutant's symbols
    for sym in ("orc_unpack", "orc_dequant", "orc_gemv", "orc_gemv_absw", "orc_round_bf16",
                "orc_round_bf16_array", "orc_gemm_entries", "orc_gemm"):
        f = getattr(mutant, sym)
        f.argtypes = getattr(real, sym).argtypes
        f.restype = getattr(real, sym).restype
    monkeypatch.setattr(oracle, "_lib", mutant)
    failed = _failures(C_PINS)
    assert failed, "mistake %r passed every pin" % name


def _router_desc_index_tiebreak(logits, k):
    z = np.asarray(logits, dtype=np.float64)
    p = np.exp(z - z.max())
    p = p / p.sum()
    order = np.lexsort((-np.arange(z.size), -p))      # ties broken by index descending
    ids = order[:k]
    return ids, p[ids] / p[ids].sum()


def _router_no_renorm(logits, k):
    z = np.asarray(logits, dtype=np.float64)
    p = np.exp(z - z.max())
    p = p / p.sum()
    ids = np.lexsort((np.arange(z.size), -p))[:k]
    return ids, p[ids]


def _silu_sigmoid_only(g):
    return 1.0 / (1.0 + np.exp(-np.asarray(g, dtype=np.float64)))


def _combine_no_residual(residual64, scalars, values):
    out = np.zeros_like(np.asarray(values[0], dtype=np.float64))
    for a, v in zip(scalars, values):
        out = out + float(a) * np.asarray(v, dtype=np.float64)
    return out


def _combine_unweighted(residual64, scalars, values):
    out = np.zeros_like(np.asarray(values[0], dtype=np.float64))
    if residual64 is not None:
        out = out + residual64
    for v in values:
        out = out + np.asarray(v, dtype=np.float64)
    return out


def _rms_sum_not_mean(x, x_dtype, gamma, eps):
    x64, g64 = oracle.widen(x, x_dtype), oracle.widen(gamma, x_dtype)
    return x64 * g64 / np.sqrt(np.sum(x64 * x64) + eps)


def _rms_eps_outside_sqrt(x, x_dtype, gamma, eps):
    x64, g64 = oracle.widen(x, x_dtype), oracle.widen(gamma, x_dtype)
    return x64 * g64 / (np.sqrt(np.mean(x64 * x64)) + eps)


def _rms_no_gamma(x, x_dtype, gamma, eps):
    x64 = oracle.widen(x, x_dtype)
    return x64 / np.sqrt(np.mean(x64 * x64) + eps)


def _rms_no_sqrt(x, x_dtype, gamma, eps):
    x64, g64 = oracle.widen(x, x_dtype), oracle.widen(gamma, x_dtype)
    return x64 * g64 / (np.mean(x64 * x64) + eps)


def _quant_variant(denom=15.0, use_raw=False, rounder=np.rint):
    real = oracle.quantize

    def fn(w, w_dtype, group_size, sb_dtype):
        w32 = oracle.widen(w, w_dtype).astype(np.float32)
        G = w32.reshape(w32.shape[:-1] + (w32.shape[-1] // group_size, group_size))
        lo, hi = G.min(-1), G.max(-1)
        s = (hi - lo) / np.float32(denom)
        codes, s_st, b_st = real(w, w_dtype, group_size, sb_dtype)
        sd = oracle.widen(s_st, sb_dtype).astype(np.float32) if not use_raw else s
        bd = oracle.widen(b_st, sb_dtype).astype(np.float32) if not use_raw else lo
        if denom != 15.0:
            sd = s if sb_dtype == "f32" else oracle.round_bf16(s.astype(np.float64)).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            t = rounder((G - bd[..., None]) / np.where(sd > 0, sd, 1)[..., None])
        q = np.where(sd[..., None] > 0, np.clip(t, 0, 15), 0).astype(np.uint32).reshape(w32.shape)
        qw = q.reshape(q.shape[:-1] + (q.shape[-1] // 8, 8))
        c = np.zeros(qw.shape[:-1], np.uint32)
        for k in range(8):
            c |= qw[..., k] << np.uint32(4 * k)
        if denom != 15.0:
            s_st = sd if sb_dtype == "f32" else (sd.view(np.uint32) >> 16).astype(np.uint16)
        return c, s_st, b_st
    return fn


PY_MUTANTS = [
    ("quant_codes_from_raw_scale", "quantize", _quant_variant(use_raw=True)),
    ("quant_denominator_16", "quantize", _quant_variant(denom=16.0)),
    ("quant_floor_not_round", "quantize", _quant_variant(rounder=np.floor)),
    ("rms_sum_not_mean", "rms_norm", _rms_sum_not_mean),
    ("rms_eps_outside_sqrt", "rms_norm", _rms_eps_outside_sqrt),
    ("rms_no_gamma", "rms_norm", _rms_no_gamma),
    ("rms_no_sqrt", "rms_norm", _rms_no_sqrt),
    ("router_tiebreak_index_desc", "router_topk", _router_desc_index_tiebreak),
    ("router_not_renormalised", "router_topk", _router_no_renorm),
    ("silu_is_sigmoid", "silu", _silu_sigmoid_only),
    ("combine_drops_residual", "combine", _combine_no_residual),
    ("combine_ignores_scalars", "combine", _combine_unweighted),
]

PY_PINS = [
    (pins.test_quantize_recovers_exact_grid, {"group": 64, "sbt": "bf16"}),
    (pins.test_quantize_picks_nearest_stored_grid_point, {"sbt": "bf16"}),
    (pins.test_quantize_scale_spans_the_group_range, {}),
    (pins.test_rms_norm_bruteforce_exact_rational, {}),
    (pins.test_rms_norm_unit_rms_and_scale_invariance, {}),
    (pins.test_rms_norm_one_hot_selects_scaled_column, {}),
    (pins.test_rms_norm_eps_inside_square_root, {}),
    (pins.test_router_worked_example_from_pages, {}),
    (pins.test_router_tie_break_index_ascending, {}),
    (pins.test_silu_against_scipy_expit, {}),
    (pins.test_combine_constant_vectors_closed_form, {}),
    (pins.test_combine_one_hot_positions, {}),
]


@pytest.mark.parametrize("name,attr,fn", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_python_mutant_is_caught(monkeypatch, name, attr, fn):
    monkeypatch.setattr(oracle, attr, fn)
    assert _failures(PY_PINS), "mistake %r passed every pin" % name
