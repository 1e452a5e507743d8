"""Pins for the fp64 CPU oracle (CPU only).

The oracle is the checker for the HIP path, so it is itself checked here
against things other than itself: the worked router example printed on the
pages (tests/golden), closed forms of special inputs, exact rational brute
force on 8x64 matrices, library routines for the special functions, and exact
invariants.  Each pin is chosen so that a plausible slip in the oracle (a
wrong nibble order, a wrong group index, a dropped bias, a transposed operand,
a wrong tie-break) fails at least one test.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mat(codes_u8, scales, biases, group, sb_dtype=synth.F32):
    n_out, k_in = codes_u8.shape
    return synth.QMatrix(codes=synth.pack_codes(codes_u8), scales=scales, biases=biases,
                         sb_dtype=sb_dtype, group_size=group, n_out=n_out, k_in=k_in)


def _rand_mat(rng, n_out, k_in, group, sb_dtype=synth.F32):
    return synth.draw_matrix(rng, n_out, k_in, group, sb_dtype, keep_raw=True)


# --------------------------------------------------------------------------
# unpack
# --------------------------------------------------------------------------

def _read_unpack_golden():
    rows = []
    with open(os.path.join(GOLDEN, "unpack_words.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((int(parts[0], 16), [int(v) for v in parts[1:]]))
    return rows


def test_unpack_golden_words():
    rows = _read_unpack_golden()
    words = np.array([[w for w, _ in rows]], dtype=np.uint32)      # one row of len(rows) words
    q = oracle.unpack(words, 8 * len(rows))
    expect = np.concatenate([np.array(c, dtype=np.uint8) for _, c in rows])
    assert np.array_equal(q[0], expect)


def _hex_unpack(codes_row: np.ndarray) -> list:
    """Independent unpack: hex digits of each word, least significant first."""
    out = []
    for w in codes_row.tolist():
        out.extend(int(ch, 16) for ch in reversed("%08x" % w))
    return out


@pytest.mark.parametrize("shape", [(1, 8), (3, 64), (17, 1024), (5, 4104)])
def test_unpack_roundtrip_bit_exact(shape):
    rng = np.random.default_rng(shape[0] * 7919 + shape[1])
    raw = rng.integers(0, 16, size=shape, dtype=np.uint8)
    q = oracle.unpack(synth.pack_codes(raw), shape[1])
    assert q.dtype == np.uint8
    assert np.array_equal(q, raw)


def test_unpack_matches_hex_digits():
    rng = np.random.default_rng(11)
    words = rng.integers(0, 2 ** 32, size=(4, 16), dtype=np.uint64).astype(np.uint32)
    q = oracle.unpack(words, 128)
    for r in range(4):
        assert q[r].tolist() == _hex_unpack(words[r])


def test_unpack_full_single_gemv_workload():
    d = synth.single_gemv(keep_raw=True)
    w = d["w"]
    assert np.array_equal(oracle.unpack(w.codes, w.k_in), w.raw_codes)


# --------------------------------------------------------------------------
# dequant and GEMV: closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("group", [32, 64, 128])
def test_one_hot_input_selects_weight(group):
    """x = e_k gives y[o] = s[o][k/g] * q[o][k] + b[o][k/g] exactly."""
    rng = np.random.default_rng(group)
    w = _rand_mat(rng, 16, 256, group)
    s64 = w.scales.astype(np.float64)
    b64 = w.biases.astype(np.float64)
    for k in [0, 1, 7, 8, 31, 32, 63, 64, 100, 255]:
        x = np.zeros(w.k_in, dtype=np.float32)
        x[k] = 1.0
        y, _ = oracle.gemv(w, x, synth.F32)
        expect = s64[:, k // group] * w.raw_codes[:, k].astype(np.float64) + b64[:, k // group]
        assert np.array_equal(y, expect), k


def test_one_hot_identity_probe_recovers_codes():
    """With s = 1, b = 0 the GEMV against e_k returns code k of every row."""
    rng = np.random.default_rng(5)
    raw = rng.integers(0, 16, size=(8, 128), dtype=np.uint8)
    w = _mat(raw, np.ones((8, 2), np.float32), np.zeros((8, 2), np.float32), 64)
    for k in range(128):
        x = np.zeros(128, np.float32)
        x[k] = 1.0
        y, _ = oracle.gemv(w, x, synth.F32)
        assert np.array_equal(y, raw[:, k].astype(np.float64))


@pytest.mark.parametrize("group", [32, 64])
def test_all_zero_codes_give_bias_rows(group):
    """q = 0 gives y[o] = sum_g b[o][g] * (sum of x over group g)."""
    rng = np.random.default_rng(100 + group)
    n_out, k_in = 8, 256
    raw = np.zeros((n_out, k_in), np.uint8)
    s = rng.uniform(0.005, 0.02, size=(n_out, k_in // group)).astype(np.float32)
    b = rng.normal(0, 0.1, size=(n_out, k_in // group)).astype(np.float32)
    w = _mat(raw, s, b, group)
    x = rng.standard_normal(k_in).astype(np.float32)
    y, _ = oracle.gemv(w, x, synth.F32)
    gsum = [math.fsum(float(v) for v in x[g * group:(g + 1) * group]) for g in range(k_in // group)]
    expect = np.array([math.fsum(float(b[o, g]) * gsum[g] for g in range(k_in // group))
                       for o in range(n_out)])
    assert np.allclose(y, expect, rtol=1e-13, atol=1e-13)


def test_constant_codes_closed_form():
    """q = c, s = sigma, b = beta everywhere gives y = (sigma c + beta) sum(x)."""
    rng = np.random.default_rng(7)
    k_in = 512
    for c, sigma, beta in [(0, 0.25, -1.0), (15, 0.0078125, -0.0625), (7, 0.5, 0.125)]:
        raw = np.full((4, k_in), c, np.uint8)
        w = _mat(raw, np.full((4, k_in // 64), sigma, np.float32),
                 np.full((4, k_in // 64), beta, np.float32), 64)
        x = rng.standard_normal(k_in).astype(np.float32)
        y, _ = oracle.gemv(w, x, synth.F32)
        expect = (sigma * c + beta) * math.fsum(float(v) for v in x)
        assert np.allclose(y, expect, rtol=1e-13, atol=1e-12)


def _exact_gemv(codes_words, scales, biases, group, x):
    """Exact rational y = W x, unpacking through hex digits (a different method)."""
    n_out = codes_words.shape[0]
    k_in = codes_words.shape[1] * 8
    xs = [Fraction(float(v)) for v in x]
    ys, mags = [], []
    for o in range(n_out):
        q = _hex_unpack(codes_words[o])
        acc = Fraction(0)
        mag = Fraction(0)
        for k in range(k_in):
            wk = Fraction(float(scales[o][k // group])) * q[k] + Fraction(float(biases[o][k // group]))
            acc += wk * xs[k]
            mag += abs(wk * xs[k])
        ys.append(acc)
        mags.append(mag)
    return ys, mags


def _check_against_exact(w, x, x_dtype):
    y, a = oracle.gemv(w, x, x_dtype)
    s = oracle.widen(w.scales, w.sb_dtype)
    b = oracle.widen(w.biases, w.sb_dtype)
    xv = oracle.widen(x, x_dtype)
    ys, mags = _exact_gemv(w.codes, s, b, w.group_size, xv)
    for o in range(w.n_out):
        # index-order float64 accumulation: |err| <= (K-1) * 2^-53 * sum|terms|
        bound = (w.k_in) * 2.0 ** -53 * float(mags[o])
        assert abs(Fraction(float(y[o])) - ys[o]) <= Fraction(bound), (o, float(y[o]), float(ys[o]))
        assert abs(float(a[o]) - float(mags[o])) <= bound


def test_bruteforce_8x64_random():
    """Exact rational brute force on 8x64, one group of 64: 1000 seeded cases."""
    for seed in range(1000):
        rng = np.random.default_rng(10_000 + seed)
        sbt = synth.F32 if seed % 2 == 0 else synth.BF16
        w = _rand_mat(rng, 8, 64, 64, sbt)
        xt = synth.F32 if seed % 3 else synth.BF16
        x = synth.draw_activation(rng, (64,), xt)
        _check_against_exact(w, x, xt)


@pytest.mark.parametrize("group", [32, 64])
def test_bruteforce_8x64_extreme_codes(group):
    rng = np.random.default_rng(77 + group)
    for c in (0, 15):
        raw = np.full((8, 64), c, np.uint8)
        s = rng.uniform(0.005, 0.02, size=(8, 64 // group)).astype(np.float32)
        b = (-8 * s + rng.normal(0, 0.001, size=s.shape)).astype(np.float32)
        w = _mat(raw, s, b, group)
        x = rng.standard_normal(64).astype(np.float32)
        _check_against_exact(w, x, synth.F32)


def test_bruteforce_multi_group_128():
    """8x128 with group 32 (four groups) catches a wrong group index."""
    rng = np.random.default_rng(4242)
    w = _rand_mat(rng, 8, 128, 32, synth.BF16)
    x = synth.draw_activation(rng, (128,), synth.BF16)
    _check_against_exact(w, x, synth.BF16)


def test_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(9)
    w = _rand_mat(rng, 32, 1024, 64)
    x = rng.standard_normal(1024).astype(np.float32)
    y, _ = oracle.gemv(w, x, synth.F32)
    y2, _ = oracle.gemv(w, (2 * x).astype(np.float32), synth.F32)
    assert np.array_equal(y2, 2 * y)
    w2 = synth.QMatrix(codes=w.codes, scales=(2 * w.scales).astype(np.float32),
                       biases=(2 * w.biases).astype(np.float32), sb_dtype=w.sb_dtype,
                       group_size=64, n_out=32, k_in=1024)
    y3, _ = oracle.gemv(w2, x, synth.F32)
    assert np.array_equal(y3, 2 * y)


def test_gemv_matches_dense_dequant_product():
    """GEMV equals the product of the dequantised matrix with x (numpy matmul)."""
    rng = np.random.default_rng(21)
    w = _rand_mat(rng, 48, 640, 64, synth.BF16)
    x = synth.draw_activation(rng, (640,), synth.BF16)
    y, a = oracle.gemv(w, x, synth.BF16)
    W = oracle.dequant(w)
    xv = oracle.widen(x, synth.BF16)
    assert np.allclose(y, W @ xv, rtol=1e-12, atol=1e-12)
    assert np.allclose(a, np.abs(W) @ np.abs(xv), rtol=1e-12)


# --------------------------------------------------------------------------
# SwiGLU, combine (8-way scalar FMA), router, MoE
# --------------------------------------------------------------------------

def test_silu_against_scipy_expit():
    from scipy.special import expit

    g = np.linspace(-30, 30, 1001)
    assert np.allclose(oracle.silu(g), g * expit(g), rtol=1e-14, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    big = oracle.silu(np.array([-1000.0]))[0]
    assert big == 0.0 and math.copysign(1.0, big) == -1.0
    assert oracle.silu(np.array([1000.0]))[0] == 1000.0
    u = np.linspace(-2, 2, 1001)
    assert np.allclose(oracle.swiglu(g, u), g * expit(g) * u, rtol=1e-14, atol=1e-300)


def test_combine_constant_vectors_closed_form():
    """Eight scalar FMAs on constant vectors: out = base + (sum a_k c_k) * 1."""
    rng = np.random.default_rng(3)
    n = 2048
    base = rng.standard_normal(n)
    a = rng.uniform(0, 1, 8)
    c = rng.standard_normal(8)
    vals = [np.full(n, ck) for ck in c]
    out = oracle.combine(base, a, vals)
    assert np.allclose(out, base + math.fsum(a * c), rtol=1e-14, atol=1e-14)


def test_combine_one_hot_positions():
    n = 64
    base = np.arange(n, dtype=np.float64)
    pos = [3, 9, 17, 20, 33, 40, 51, 63]
    a = [0.5, 0.25, 0.125, 1.0, 2.0, -1.0, 3.0, 0.75]
    vals = []
    for p in pos:
        v = np.zeros(n)
        v[p] = 1.0
        vals.append(v)
    out = oracle.combine(base, a, vals)
    expect = base.copy()
    for p, ak in zip(pos, a):
        expect[p] += ak
    assert np.array_equal(out, expect)
    assert np.array_equal(oracle.combine(None, a, vals), expect - base)


def _read_router_golden():
    vals = {}
    with open(os.path.join(GOLDEN, "router_topk_k2.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, *rest = line.split()
                vals[key] = rest
    return vals


def test_router_worked_example_from_pages():
    g = _read_router_golden()
    logits = np.array([float(v) for v in g["logits"]])
    ids, wts = oracle.router_topk(logits, int(g["k"][0]))
    assert ids.tolist() == [int(v) for v in g["ids"]]
    expect = np.array([float(v) for v in g["weights"]])
    assert np.allclose(wts, expect, rtol=0, atol=1e-15)
    assert abs(wts.sum() - 1.0) < 1e-15 and wts[0] > wts[1]
    # closed form: sigmoid of the logit gap
    assert abs(wts[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


def test_router_equals_softmax_over_kept_logits():
    rng = np.random.default_rng(12)
    for _ in range(50):
        z = rng.standard_normal(128)
        ids, wts = oracle.router_topk(z, 8)
        assert len(set(ids.tolist())) == 8
        assert np.all(z[ids][:-1] >= z[ids][1:])             # sorted by logit, descending
        assert z[ids].min() >= np.sort(z)[-8]                 # they are the largest eight
        zk = z[ids]
        ref = np.exp(zk - zk.max()) / np.exp(zk - zk.max()).sum()
        assert np.allclose(wts, ref, rtol=1e-13)


def test_router_tie_break_index_ascending():
    z = np.array([0.0, 2.0, 1.0, 2.0, 2.0, -1.0])
    ids, wts = oracle.router_topk(z, 3)
    assert ids.tolist() == [1, 3, 4]
    assert np.allclose(wts, 1.0 / 3.0)
    ids, _ = oracle.router_topk(z, 4)
    assert ids.tolist() == [1, 3, 4, 2]


def _small_moe(seed, E=6, hidden=128, inter=64):
    return synth.moe_layer(seed=seed, n_experts=E, hidden=hidden, inter=inter, group_size=32)


def test_moe_expert_slab_selection():
    """Stacked experts: picking expert 2 equals the GEMV of that slab alone."""
    d = _small_moe(1, E=4)
    gate = d["gate"]
    x = d["x"][0]
    for e in (0, 2, 3):
        slab = synth.QMatrix(codes=gate.codes[e].copy(), scales=gate.scales[e].copy(),
                             biases=gate.biases[e].copy(), sb_dtype=gate.sb_dtype,
                             group_size=gate.group_size, n_out=gate.n_out, k_in=gate.k_in)
        y_stack, _ = oracle.gemv(gate, x, synth.BF16, expert=e)
        y_slab, _ = oracle.gemv(slab, x, synth.BF16)
        assert np.array_equal(y_stack, y_slab)
    # different experts really differ
    y0, _ = oracle.gemv(gate, x, synth.BF16, expert=0)
    y1, _ = oracle.gemv(gate, x, synth.BF16, expert=1)
    assert not np.allclose(y0, y1)


def _plain(m, e):
    return synth.QMatrix(codes=m.codes[e].copy(), scales=m.scales[e].copy(), biases=m.biases[e].copy(),
                         sb_dtype=m.sb_dtype, group_size=m.group_size, n_out=m.n_out, k_in=m.k_in)


def test_moe_same_expert_reduces_to_dense_ffn():
    """All slots on expert e with weights summing to 1: residual + FFN_e(x)."""
    d = _small_moe(2)
    x, r = d["x"][0], d["residual"][0]
    e = 4
    wts = np.array([0.5, 0.25, 0.125, 0.0625, 0.03125, 0.015625, 0.0078125, 0.0078125])
    out, _ = oracle.moe(d["gate"], d["up"], d["down"], x, [e] * 8, wts, r, synth.BF16)
    y, _, _, _ = oracle.dense_ffn(_plain(d["gate"], e), _plain(d["up"], e), _plain(d["down"], e),
                                  x, synth.BF16)
    assert np.allclose(out, oracle.widen(r, synth.BF16) + y, rtol=1e-12, atol=1e-12)


def test_moe_one_hot_weights_and_zero_residual():
    d = _small_moe(3)
    x = d["x"][0]
    ids = [5, 1, 0, 3, 2, 4, 1, 0]
    wts = np.zeros(8)
    wts[3] = 1.0
    out, _ = oracle.moe(d["gate"], d["up"], d["down"], x, ids, wts, None, synth.BF16)
    y, _, _, _ = oracle.dense_ffn(_plain(d["gate"], 3), _plain(d["up"], 3), _plain(d["down"], 3),
                                  x, synth.BF16)
    assert np.allclose(out, y, rtol=1e-12, atol=1e-12)


def test_moe_is_weighted_sum_of_experts():
    d = _small_moe(4)
    x, r = d["x"][0], d["residual"][0]
    ids, wts = oracle.router_topk(d["logits"][0], 4)
    out, _ = oracle.moe(d["gate"], d["up"], d["down"], x, ids, wts, r, synth.BF16)
    acc = oracle.widen(r, synth.BF16).copy()
    for e, a in zip(ids, wts):
        y, _, _, _ = oracle.dense_ffn(_plain(d["gate"], e), _plain(d["up"], e), _plain(d["down"], e),
                                      x, synth.BF16)
        acc += a * y
    assert np.allclose(out, acc, rtol=1e-12, atol=1e-12)


def test_moe_out_of_range_ids_contribute_nothing():
    d = _small_moe(5)
    x, r = d["x"][0], d["residual"][0]
    ids_ok, wts = [1, 2], [0.6, 0.4]
    out_ok, _ = oracle.moe(d["gate"], d["up"], d["down"], x, ids_ok, wts, r, synth.BF16)
    out_bad, _ = oracle.moe(d["gate"], d["up"], d["down"], x, [1, 2, 6, 1000], wts + [0.3, 0.3],
                            r, synth.BF16)
    assert np.array_equal(out_ok, out_bad)


# --------------------------------------------------------------------------
# prefill GEMM
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch_cast():
    import torch

    rng = np.random.default_rng(8)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -9,
                                  255.5, 256.5, 0.0])]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref)
    # ties to even, explicitly
    assert oracle.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert oracle.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6


def test_gemm_identity_recovers_codes():
    """X = I (T = K) with s = 1, b = 0: Y^T is the code matrix, exactly."""
    rng = np.random.default_rng(31)
    raw = rng.integers(0, 16, size=(32, 64), dtype=np.uint8)
    w = _mat(raw, np.ones((32, 1), np.float32), np.zeros((32, 1), np.float32), 64)
    X = synth.f32_to_bf16_bits(np.eye(64, dtype=np.float32))
    Y, _ = oracle.gemm(w, X, synth.BF16)
    assert np.array_equal(Y.T, raw.astype(np.float64))


def test_gemm_rows_match_gemv_with_rounded_weights():
    rng = np.random.default_rng(32)
    w = _rand_mat(rng, 64, 256, 64, synth.BF16)
    X = synth.draw_activation(rng, (5, 256), synth.BF16)
    Y, _ = oracle.gemm(w, X, synth.BF16, round_w=False)
    for t in range(5):
        y, _ = oracle.gemv(w, X[t], synth.BF16)
        assert np.array_equal(Y[t], y)
    # the bf16-weight variant multiplies round_bf16(W) with X (numpy matmul)
    Yr, _ = oracle.gemm(w, X, synth.BF16, round_w=True)
    Wr = oracle.round_bf16(oracle.dequant(w))
    assert np.allclose(Yr, oracle.widen(X, synth.BF16) @ Wr.T, rtol=1e-12, atol=1e-12)
    # and the rounding is real: a sizeable share of weights is not bf16-exact
    assert np.mean(Wr != oracle.dequant(w)) > 0.2


def test_gemm_weight_is_rounded_once_to_bf16():
    """The prefill weight is the exact s q + b rounded once to the nearest bfloat16.

    Hand-derived cases, read out through one-hot X rows (bf16 ulp at 1 is 2^-7, so the
    bf16 neighbours of values just above 1 are 1 and 1 + 2^-7, with midpoint 1 + 2^-8):
      row 0: s = 1/2 + 2^-24, b = 1/2 + 2^-8, q = 1 -> exact 1 + 2^-8 + 2^-24, just above
             the midpoint -> 1 + 2^-7.  (Rounding to float32 first would land on the
             midpoint 1 + 2^-8 and then tie to even at 1.0: a double rounding.)
      row 1: s = 1/2, b = 1/2 + 2^-8, q = 1 -> exactly the midpoint -> ties to even 1.0.
      row 2: s = 3/8, b = -1, q = 5 -> 7/8, bf16-exact."""
    raw = np.zeros((3, 64), np.uint8)
    raw[0, 0] = 1
    raw[1, 0] = 1
    raw[2, 0] = 5
    w = _mat(raw, np.array([[0.5 + 2.0 ** -24], [0.5], [0.375]], np.float32),
             np.array([[0.5 + 2.0 ** -8], [0.5 + 2.0 ** -8], [-1.0]], np.float32), 64)
    X = np.zeros((1, 64), np.uint16)
    X[0, 0] = 0x3F80                                                 # bf16 1.0
    Y, _ = oracle.gemm(w, X, synth.BF16, round_w=True)
    assert Y[0, 0] == 1.0 + 2.0 ** -7
    assert Y[0, 1] == 1.0
    assert Y[0, 2] == 0.875
    Yx, _ = oracle.gemm(w, X, synth.BF16, round_w=False)
    assert Yx[0, 0] == 1 + 2.0 ** -8 + 2.0 ** -24                     # exact weight
    assert Yx[0, 1] == 1 + 2.0 ** -8


def test_gemm_entries_match_full():
    rng = np.random.default_rng(33)
    w = _rand_mat(rng, 96, 192, 32, synth.BF16)
    X = synth.draw_activation(rng, (7, 192), synth.BF16)
    Y, A = oracle.gemm(w, X, synth.BF16)
    t = rng.integers(0, 7, 50)
    o = rng.integers(0, 96, 50)
    y, a = oracle.gemm_entries(w, X, t, o, synth.BF16)
    assert np.array_equal(y, Y[t, o]) and np.array_equal(a, A[t, o])


def test_gemm_zero_padding_rows_do_not_change_real_rows():
    rng = np.random.default_rng(34)
    w = _rand_mat(rng, 32, 128, 64, synth.BF16)
    X = synth.draw_activation(rng, (30, 128), synth.BF16)
    Xp = np.concatenate([X, np.zeros((2, 128), np.uint16)])       # pad T=30 -> 32
    Y, _ = oracle.gemm(w, X, synth.BF16)
    Yp, _ = oracle.gemm(w, Xp, synth.BF16)
    assert np.array_equal(Yp[:30], Y)
    assert np.all(Yp[30:] == 0.0)


def test_gemm_bruteforce_small_exact():
    """8 output columns, T=3, K=64 against exact rationals with bf16-rounded weights."""
    rng = np.random.default_rng(35)
    w = _rand_mat(rng, 8, 64, 64, synth.BF16)
    X = synth.draw_activation(rng, (3, 64), synth.BF16)
    Y, A = oracle.gemm(w, X, synth.BF16)
    Wr = oracle.round_bf16(oracle.dequant(w))
    Xv = oracle.widen(X, synth.BF16)
    for t in range(3):
        for o in range(8):
            exact = sum(Fraction(float(Wr[o, k])) * Fraction(float(Xv[t, k])) for k in range(64))
            bound = 64 * 2.0 ** -53 * float(A[t, o])
            assert abs(Fraction(float(Y[t, o])) - exact) <= Fraction(bound)


# --------------------------------------------------------------------------
# RMSNorm prologue
# --------------------------------------------------------------------------

def test_rms_norm_bruteforce_exact_rational():
    """x in {+3, -3}, eps = 7: mean(x^2) + eps = 16 is a perfect square, so
    xn = x * gamma / 4 exactly and the normalised GEMV has an exact rational
    value (hex-digit unpack, Fractions).  A sum in place of the mean, eps
    outside the square root or a dropped gamma changes the result."""
    for seed in range(20):
        rng = np.random.default_rng(5000 + seed)
        k_in = 64 if seed % 2 else 128
        w = _rand_mat(rng, 8, k_in, 32 if seed % 3 == 0 else 64, synth.BF16)
        x = (3.0 * rng.choice([-1.0, 1.0], size=k_in)).astype(np.float32)
        gamma = rng.uniform(0.5, 1.5, size=k_in).astype(np.float32)
        xn = oracle.rms_norm(x, synth.F32, gamma, 7.0)
        expect = [Fraction(float(a)) * Fraction(float(g)) / 4 for a, g in zip(x, gamma)]
        assert [Fraction(float(v)) for v in xn] == expect
        (y, a), = oracle.rms_norm_multi([w], x, synth.F32, gamma, 7.0)
        s = oracle.widen(w.scales, w.sb_dtype)
        b = oracle.widen(w.biases, w.sb_dtype)
        ys, mags = _exact_gemv(w.codes, s, b, w.group_size, [float(e) for e in expect])
        for o in range(w.n_out):
            bound = k_in * 2.0 ** -53 * float(mags[o])
            assert abs(Fraction(float(y[o])) - ys[o]) <= Fraction(bound), o


def test_rms_norm_unit_rms_and_scale_invariance():
    """gamma = 1, eps = 0: the output has mean square 1, and scaling x by a
    power of two leaves it unchanged (bit for bit)."""
    rng = np.random.default_rng(31)
    x = synth.draw_activation(rng, (4096,), synth.BF16)
    ones = synth.f32_to_bf16_bits(np.ones(4096, np.float32))
    xn = oracle.rms_norm(x, synth.BF16, ones, 0.0)
    assert abs(np.mean(xn * xn) - 1.0) < 1e-14
    x4 = synth.f32_to_bf16_bits(4.0 * synth.bf16_bits_to_f32(x))
    assert np.array_equal(oracle.rms_norm(x4, synth.BF16, ones, 0.0), xn)


def test_rms_norm_one_hot_selects_scaled_column():
    """x = a e_k, eps = 0: xn = sqrt(K) sign(a) gamma_k e_k, so W xn is column k
    of the dequantised matrix times sqrt(K) sign(a) gamma_k."""
    rng = np.random.default_rng(32)
    K = 256
    w = _rand_mat(rng, 16, K, 64, synth.BF16)
    gamma = rng.uniform(0.5, 2.0, size=K).astype(np.float32)
    W = oracle.dequant(w)
    for k, a in ((0, 1.5), (77, -0.25), (255, 3.0)):
        x = np.zeros(K, np.float32)
        x[k] = a
        (y, _), = oracle.rms_norm_multi([w], x, synth.F32, gamma, 0.0)
        np.testing.assert_allclose(y, 16.0 * np.sign(a) * float(gamma[k]) * W[:, k], rtol=1e-14)


def test_rms_norm_eps_inside_square_root():
    """When eps dominates mean(x^2) the normaliser tends to 1 / sqrt(eps)."""
    rng = np.random.default_rng(33)
    x = (1e-9 * rng.standard_normal(512)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, size=512).astype(np.float32)
    xn = oracle.rms_norm(x, synth.F32, gamma, 4.0)
    np.testing.assert_allclose(xn, x.astype(np.float64) * gamma / 2.0, rtol=1e-12)


def test_rms_norm_swiglu_pair_composes():
    """The SwiGLU variant equals silu(gate xn) * (up xn) built from the pinned parts."""
    rng = np.random.default_rng(34)
    gate = _rand_mat(rng, 32, 128, 64, synth.BF16)
    up = _rand_mat(rng, 32, 128, 64, synth.BF16)
    x = synth.draw_activation(rng, (128,), synth.BF16)
    gamma = synth.draw_activation(rng, (128,), synth.BF16)
    h, _ = oracle.rms_norm_swiglu_pair(gate, up, x, synth.BF16, gamma, 1e-6)
    xn = oracle.rms_norm(x, synth.BF16, gamma, 1e-6)
    g = oracle.dequant(gate) @ xn
    u = oracle.dequant(up) @ xn
    np.testing.assert_allclose(h, g / (1.0 + np.exp(-g)) * u, rtol=1e-12, atol=1e-300)


# --------------------------------------------------------------------------
# quantiser
# --------------------------------------------------------------------------

def _qmat(codes, s, b, n_out, k_in, group, sbt):
    return synth.QMatrix(codes=codes, scales=s, biases=b, sb_dtype=sbt, group_size=group,
                         n_out=n_out, k_in=k_in)


@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("sbt", [synth.F32, synth.BF16])
def test_quantize_recovers_exact_grid(group, sbt):
    """Weights on a grid s q + b where every group holds codes 0 and 15 and
    s = 2^-e, b = m * s are exactly representable: the quantiser returns the
    same codes, scales and biases."""
    rng = np.random.default_rng(group)
    n_out, k_in = 12, 4 * group
    raw = rng.integers(0, 16, size=(n_out, k_in), dtype=np.uint8)
    raw[:, ::group] = 0
    raw[:, 1::group] = 15
    e = rng.integers(4, 9, size=(n_out, k_in // group))
    s = np.ldexp(1.0, -e).astype(np.float32)
    b = (rng.integers(-12, -4, size=s.shape) * s).astype(np.float32)
    sb = (lambda a: synth.f32_to_bf16_bits(a)) if sbt == synth.BF16 else (lambda a: a)
    w = _qmat(synth.pack_codes(raw), sb(s), sb(b), n_out, k_in, group, sbt)
    W = oracle.dequant(w).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), oracle.dequant(w))  # exact in float32
    codes, s2, b2 = oracle.quantize(W, synth.F32, group, sbt)
    assert np.array_equal(codes, w.codes)
    assert np.array_equal(s2, w.scales) and np.array_equal(b2, w.biases)


@pytest.mark.parametrize("sbt", [synth.F32, synth.BF16])
def test_quantize_picks_nearest_stored_grid_point(sbt):
    """Every code is the one whose s' q + b' (stored s', b') is nearest to w --
    checked by brute force over the 16 codes in float64 (a float32 rounding
    of (w - b') / s' may only matter within 1e-5 s' of a midpoint)."""
    rng = np.random.default_rng(7 if sbt == synth.F32 else 8)
    W = rng.standard_normal((40, 256)).astype(np.float32)
    codes, s, b = oracle.quantize(W, synth.F32, 64, sbt)
    w = _qmat(codes, s, b, 40, 256, 64, sbt)
    q = oracle.unpack(codes, 256).astype(np.float64)
    s64 = np.repeat(oracle.widen(s, sbt), 64, axis=1)
    b64 = np.repeat(oracle.widen(b, sbt), 64, axis=1)
    cand = s64[..., None] * np.arange(16.0) + b64[..., None]
    err_all = np.abs(cand - W[..., None].astype(np.float64))
    chosen = np.take_along_axis(err_all, q.astype(np.int64)[..., None], axis=-1)[..., 0]
    assert np.all(chosen <= err_all.min(axis=-1) + 1e-5 * s64)
    assert np.array_equal(oracle.dequant(w), s64 * q + b64)


def test_quantize_scale_spans_the_group_range():
    """float32 storage: b is the group minimum and b + 15 s its maximum (to rounding),
    so the extreme weights get codes 0 and 15."""
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((16, 512)) * 0.05).astype(np.float32)
    codes, s, b = oracle.quantize(W, synth.F32, 64, synth.F32)
    G = W.reshape(16, 8, 64)
    assert np.array_equal(b, G.min(axis=-1))
    np.testing.assert_allclose(b.astype(np.float64) + 15.0 * s, G.max(axis=-1), rtol=1e-6)
    q = oracle.unpack(codes, 512).reshape(16, 8, 64)
    assert np.all(q[np.arange(16)[:, None], np.arange(8)[None, :], G.argmin(-1)] == 0)
    assert np.all(q[np.arange(16)[:, None], np.arange(8)[None, :], G.argmax(-1)] == 15)


def test_quantize_constant_group_and_bf16_input():
    """A constant group gives s = 0, b = the constant and codes 0; bf16 input widens exactly."""
    W = np.full((2, 128), 0.375, np.float32)
    W[1, 64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    for wt in (synth.F32, synth.BF16):
        Win = W if wt == synth.F32 else synth.f32_to_bf16_bits(W)
        codes, s, b = oracle.quantize(Win, wt, 64, synth.F32)
        assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and b[0, 0] == np.float32(0.375)
        assert np.all(oracle.unpack(codes, 128)[0] == 0)
        assert s[1, 1] > 0


def test_quantize_codes_follow_rounded_not_raw_scale():
    """bf16 storage: codes are taken against the rounded s', b'.  Codes computed
    against the raw float32 s, b differ for some weights (the page's fixtures
    tell the two rules apart in the same way), and those are never nearer to w
    on the stored grid."""
    rng = np.random.default_rng(10)
    W = rng.standard_normal((64, 512)).astype(np.float32)
    codes, s, b = oracle.quantize(W, synth.F32, 64, synth.BF16)
    _, s32, b32 = oracle.quantize(W, synth.F32, 64, synth.F32)
    G = W.reshape(64, 8, 64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q_raw = np.clip(np.rint((G - b32[..., None]) / s32[..., None]), 0, 15).reshape(64, 512)
    q = oracle.unpack(codes, 512)
    assert np.count_nonzero(q != q_raw) > 0


# --------------------------------------------------------------------------
# MoE prefill
# --------------------------------------------------------------------------

def _exact_bf16_moe(seed, E=5, hidden=128, inter=64):
    """A MoE layer whose dequantised weights are bf16 values already (power-of-two
    scales, biases multiples of the scale), so rounding to bf16 is the identity."""
    rng = np.random.default_rng(seed)

    def stack(n_out, k_in):
        raw = rng.integers(0, 16, size=(E, n_out, k_in), dtype=np.uint8)
        s = np.ldexp(1.0, -rng.integers(5, 9, size=(E, n_out, k_in // 64))).astype(np.float32)
        b = (rng.integers(-10, -5, size=s.shape) * s).astype(np.float32)
        return synth.QMatrix(codes=synth.pack_codes(raw), scales=synth.f32_to_bf16_bits(s),
                             biases=synth.f32_to_bf16_bits(b), sb_dtype=synth.BF16, group_size=64,
                             n_out=n_out, k_in=k_in, n_experts=E)
    return stack(inter, hidden), stack(inter, hidden), stack(hidden, inter), rng


def test_moe_prefill_equals_decode_moe_when_weights_are_bf16():
    """With bf16-exact weights the prefill form is the pinned decode moe() token by token."""
    gate, up, down, rng = _exact_bf16_moe(1)
    T, K = 6, 3
    X = synth.draw_activation(rng, (T, 128), synth.BF16)
    ids = rng.integers(0, 5, size=(T, K))
    ids[2, 1] = 9  # out of range: contributes nothing
    wts = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    res = synth.draw_activation(rng, (T, 128), synth.BF16)
    out, a = oracle.moe_prefill(gate, up, down, X, ids, wts, res)
    for t in range(T):
        ref, a_ref = oracle.moe(gate, up, down, X[t], ids[t], wts[t], res[t], synth.BF16)
        np.testing.assert_allclose(out[t], ref, rtol=1e-12, atol=1e-12 * float(np.max(a_ref)))


def test_moe_prefill_rounds_weights_to_bf16():
    """Generic weights: each expert's contribution is the prefill GEMM (pinned gemm())
    of its rounded weights; one kept slot with weight 1 and no residual isolates it."""
    d = synth.moe_layer(seed=4, n_experts=4, hidden=128, inter=64, n_tokens=2)
    gate, up, down = d["gate"], d["up"], d["down"]
    X = np.stack([d["x"][0], d["x"][1]])
    ids = np.array([[2], [0]])
    wts = np.ones((2, 1), np.float32)
    out, _ = oracle.moe_prefill(gate, up, down, X, ids, wts, None)
    for t in range(2):
        e = int(ids[t][0])
        xt = oracle.widen(X[t], synth.BF16)
        W = lambda m: oracle.round_bf16(oracle.dequant(m, expert=e))
        g, u = W(gate) @ xt, W(up) @ xt
        h = g / (1.0 + np.exp(-g)) * u
        np.testing.assert_allclose(out[t], W(down) @ h, rtol=1e-10, atol=1e-12)


def test_moe_prefill_tokens_are_independent():
    """Permuting the tokens permutes the outputs (no cross-token term)."""
    gate, up, down, rng = _exact_bf16_moe(2)
    T, K = 5, 2
    X = synth.draw_activation(rng, (T, 128), synth.BF16)
    ids = rng.integers(0, 5, size=(T, K))
    wts = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    out, _ = oracle.moe_prefill(gate, up, down, X, ids, wts, None)
    perm = np.array([3, 0, 4, 1, 2])
    out_p, _ = oracle.moe_prefill(gate, up, down, X[perm], ids[perm], wts[perm], None)
    np.testing.assert_array_equal(out_p, out[perm])
