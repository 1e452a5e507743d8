"""GPU parity of qgemv_int4_smallm (T = 1..16 activation rows) against the fp64 oracle.

Each token's outputs follow the qgemv_int4 rules (per-element bf16 bound,
relative L2 for float32); the oracle runs one GEMV per token.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import check, check_f32, dev_matrix, lib, nan_like, oracle_threads, require_gpu, to_np64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _x(rng, T, k_in, ldx=None):
    """bf16 bits [T][k_in] and the device tensor [T][ldx] holding them (pad = NaN)."""
    x = synth.draw_activation(rng, (T, k_in), "bf16")
    ldx = ldx or k_in
    dev = torch.full((T, ldx), float("nan"), dtype=torch.bfloat16, device="cuda")
    dev[:, :k_in] = synth.to_torch(x, "bf16")
    return x, dev


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8, 9, 13, 16])
@pytest.mark.parametrize("n_out,k_in,g", [(256, 1024, 64), (1000, 2048, 32), (96, 4096, 128),
                                          (130, 5120, 64), (64, 640, 64)])
def test_smallm_single_matrix(T, n_out, k_in, g):
    q = lib()
    rng = np.random.default_rng(T * 1000 + n_out + k_in)
    w = synth.draw_matrix(rng, n_out, k_in, g, "bf16")
    x, xd = _x(rng, T, k_in)
    y = nan_like((T, n_out), torch.bfloat16)
    q.qgemv_int4_smallm([dev_matrix(w)], xd, [y])
    torch.cuda.synchronize()
    for t in range(T):
        ref, a = oracle.gemv(w, x[t], "bf16", threads=oracle_threads())
        check(y[t], ref, a, "smallm T=%d t=%d" % (T, t))


@pytest.mark.parametrize("T", [2, 4, 7, 11, 16])
def test_smallm_qkv_strided_rows_f32_out(T):
    """Three projections of T shared rows; x rows strided (ldx > k_in); float32 outputs."""
    q = lib()
    rng = np.random.default_rng(T)
    k_in = 2048
    ws = [synth.draw_matrix(rng, n, k_in, 64, "bf16") for n in (512, 128, 128)]
    x, xd = _x(rng, T, k_in, ldx=k_in + 64)
    ys = [nan_like((T, w.n_out), torch.float32) for w in ws]
    q.qgemv_int4_smallm([dev_matrix(w) for w in ws], xd, ys)
    torch.cuda.synchronize()
    for t in range(T):
        for w, y, (ref, a) in zip(ws, ys, oracle.multi(ws, x[t], "bf16")):
            check(y[t], ref, a, "smallm qkv t=%d" % t)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_smallm_swiglu_pair(T):
    """Fused gate/up SwiGLU for T rows; h is float32 [T][inter]."""
    q = lib()
    rng = np.random.default_rng(40 + T)
    hidden, inter = 1024, 768
    gate = synth.draw_matrix(rng, inter, hidden, 64, "bf16")
    up = synth.draw_matrix(rng, inter, hidden, 64, "bf16")
    x, xd = _x(rng, T, hidden)
    h = nan_like((T, inter), torch.float32)
    q.qgemv_int4_smallm([dev_matrix(gate), dev_matrix(up)], xd, [h], epilogue=q.EPI_SWIGLU_PAIR)
    torch.cuda.synchronize()
    for t in range(T):
        ref, a = oracle.swiglu_pair(gate, up, x[t], "bf16")
        got = to_np64(h[t])
        assert np.all(np.isfinite(got))
        # float32 SwiGLU of float32 sums: the bound of the T = 1 SwiGLU test
        check_f32(got, ref, "smallm swiglu h T=%d t=%d" % (T, t), a_ref=a)


def test_smallm_tokens_are_independent_and_exact_repeat():
    """Row t of a T=8 call equals a T=1 call on row t, bit for bit."""
    q = lib()
    rng = np.random.default_rng(77)
    w = synth.draw_matrix(rng, 384, 3072, 64, "bf16")
    x, xd = _x(rng, 8, 3072)
    y8 = nan_like((8, 384), torch.float32)
    q.qgemv_int4_smallm([dev_matrix(w)], xd, [y8])
    for t in (0, 5, 7):
        y1 = nan_like((1, 384), torch.float32)
        q.qgemv_int4_smallm([dev_matrix(w)], xd[t:t + 1].contiguous(), [y1])
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y8[t]), t


def test_smallm_rejects_float32_multi_row():
    q = lib()
    rng = np.random.default_rng(3)
    w = synth.draw_matrix(rng, 64, 256, 64, "bf16")
    x = torch.zeros((2, 256), dtype=torch.float32, device="cuda")
    y = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(q.Int4Error) as e:
        q.qgemv_int4_smallm([dev_matrix(w)], x, [y])
    assert e.value.status == "ERR_DTYPE"


# The MFMA form of small-M calls (bf16 activations, stored outputs, group 32/64/128,
# k_in a multiple of 512 up to 8192): one wave per 512-k slice of a 16-row tile.
@pytest.mark.parametrize("n_out,k_in,g,sb", [(40, 512, 64, "bf16"), (37, 8192, 64, "bf16"),
                                             (300, 1536, 32, "f32"), (129, 2560, 128, "f32"),
                                             (16, 4096, 128, "bf16"), (1, 512, 128, "bf16"),
                                             (17, 1024, 32, "f32")])
@pytest.mark.parametrize("T", [1, 3, 8])
def test_smallm_mfma_form_shapes(T, n_out, k_in, g, sb):
    """One wave per tile (k_in 512: 128 outputs over 64 threads), sixteen (8192), float32
    scales, ragged 16-row tiles, padded activation rows (ldx > k_in)."""
    q = lib()
    rng = np.random.default_rng(T * 7 + n_out + k_in)
    w = synth.draw_matrix(rng, n_out, k_in, g, sb)
    x, xd = _x(rng, T, k_in, ldx=k_in + 24)
    y = torch.full((T, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    q.qgemv_int4_smallm([dev_matrix(w)], xd, [y])
    torch.cuda.synchronize()
    for t in range(T):
        ref, a = oracle.gemv(w, x[t], "bf16", threads=oracle_threads())
        check(y[t], ref, a, "smallm mfma T=%d t=%d %dx%d g%d %s" % (T, t, n_out, k_in, g, sb))


def test_smallm_mfma_rows_independent_of_T_and_close_to_the_gemv():
    """Rows of a T = 5 call equal T = 1 calls bit for bit; a T = 1 small-M call (MFMA sums)
    agrees with qgemv_int4 (v_dot2 sums) within float32 rounding of the sums."""
    q = lib()
    rng = np.random.default_rng(91)
    w = synth.draw_matrix(rng, 200, 2048, 64, "bf16")
    x, xd = _x(rng, 5, 2048)
    y5 = nan_like((5, 200), torch.float32)
    q.qgemv_int4_smallm([dev_matrix(w)], xd, [y5])
    for t in range(5):
        y1 = nan_like((1, 200), torch.float32)
        q.qgemv_int4_smallm([dev_matrix(w)], xd[t:t + 1].contiguous(), [y1])
        yg = nan_like(200, torch.float32)
        q.qgemv_int4(dev_matrix(w), xd[t].contiguous(), yg)
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y5[t]), t
        ref, a = oracle.gemv(w, x[t], "bf16")
        check(y5[t], ref, a, "smallm mfma t=%d" % t)
        diff = (y1[0].double() - yg.double()).abs().cpu().numpy()
        assert np.all(diff <= 2.0 ** -16 * a), t


@pytest.mark.parametrize("inter,hidden,g,sb,h_dt", [(1000, 2560, 32, "f32", "bf16"),
                                                    (37, 8192, 128, "bf16", "f32"),
                                                    (48, 512, 64, "bf16", "bf16")])
@pytest.mark.parametrize("T", [1, 5, 8])
def test_smallm_swiglu_pair_mfma_form(T, inter, hidden, g, sb, h_dt):
    """The gate/up pair on the MFMA form: two code streams per 16-row tile, SwiGLU after
    the sum of the K slices; group 32 with float32 scales, 16 waves per tile, one wave."""
    q = lib()
    rng = np.random.default_rng(T + inter + hidden)
    gate = synth.draw_matrix(rng, inter, hidden, g, sb)
    up = synth.draw_matrix(rng, inter, hidden, g, sb)
    x, xd = _x(rng, T, hidden)
    h = torch.full((T, inter), float("nan"), dtype=torch.bfloat16 if h_dt == "bf16" else torch.float32,
                   device="cuda")
    q.qgemv_int4_smallm([dev_matrix(gate), dev_matrix(up)], xd, [h], epilogue=q.EPI_SWIGLU_PAIR)
    torch.cuda.synchronize()
    for t in range(T):
        ref, a = oracle.swiglu_pair(gate, up, x[t], "bf16")
        got = to_np64(h[t])
        assert np.all(np.isfinite(got))
        if h_dt == "bf16":
            check(h[t], ref, a, "swiglu mfma T=%d t=%d" % (T, t))
        else:
            check_f32(got, ref, "smallm swiglu h T=%d t=%d" % (T, t), a_ref=a)


def test_smallm_swiglu_pair_rows_independent_of_T():
    q = lib()
    rng = np.random.default_rng(12)
    gate = synth.draw_matrix(rng, 320, 3072, 64, "bf16")
    up = synth.draw_matrix(rng, 320, 3072, 64, "bf16")
    x, xd = _x(rng, 6, 3072)
    h6 = nan_like((6, 320), torch.float32)
    q.qgemv_int4_smallm([dev_matrix(gate), dev_matrix(up)], xd, [h6], epilogue=q.EPI_SWIGLU_PAIR)
    for t in (0, 3, 5):
        h1 = nan_like((1, 320), torch.float32)
        q.qgemv_int4_smallm([dev_matrix(gate), dev_matrix(up)], xd[t:t + 1].contiguous(), [h1],
                            epilogue=q.EPI_SWIGLU_PAIR)
        torch.cuda.synchronize()
        assert torch.equal(h1[0], h6[t]), t


def test_smallm_workload_sizes_mfma_form():
    """The benchmark shapes on the MFMA form: q/k/v (4096 -> 4096/1024/1024) and the
    5120 -> 17408 gate/up pair at T = 8, every output against the oracle."""
    q = lib()
    d = synth.qkv_multi()
    rng = np.random.default_rng(808)
    x, xd = _x(rng, 8, 4096)
    ys = [torch.full((8, w.n_out), float("nan"), dtype=torch.bfloat16, device="cuda") for w in d["ws"]]
    q.qgemv_int4_smallm([dev_matrix(w) for w in d["ws"]], xd, ys)
    torch.cuda.synchronize()
    for t in range(8):
        for i, (w, y, (ref, a)) in enumerate(zip(d["ws"], ys, oracle.multi(d["ws"], x[t], "bf16",
                                                                             threads=oracle_threads()))):
            check(y[t], ref, a, "qkv T=8 t=%d m=%d" % (t, i))

    dl = synth.dense_layer()
    x, xd = _x(rng, 8, 5120)
    h = nan_like((8, 17408), torch.float32)
    q.qgemv_int4_smallm([dev_matrix(dl["gate"]), dev_matrix(dl["up"])], xd, [h],
                        epilogue=q.EPI_SWIGLU_PAIR)
    torch.cuda.synchronize()
    hs = to_np64(h)
    for t in range(8):
        ref, a = oracle.swiglu_pair(dl["gate"], dl["up"], x[t], "bf16", threads=oracle_threads())
        check_f32(hs[t], ref, "smallm dense gate/up T=8 t=%d" % t, a_ref=a)


@pytest.mark.parametrize("k_in", [2048, 6144, 17408])
def test_smallm_sixteen_rows_equal_single_rows(k_in):
    """Row t of a T = 16 call equals a T = 1 call on row t bit for bit: all 16 rows in one
    MFMA launch (k_in 2048), two 8-row MFMA launches (6144: 16 staged rows exceed LDS), and
    the GEMV form (17408, not a multiple of 512 ... 8192)."""
    q = lib()
    rng = np.random.default_rng(k_in)
    w = synth.draw_matrix(rng, 96, k_in, 64, "bf16")
    x, xd = _x(rng, 16, k_in)
    y16 = nan_like((16, 96), torch.float32)
    q.qgemv_int4_smallm([dev_matrix(w)], xd, [y16])
    for t in (0, 7, 8, 15):
        y1 = nan_like((1, 96), torch.float32)
        q.qgemv_int4_smallm([dev_matrix(w)], xd[t:t + 1].contiguous(), [y1])
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y16[t]), t
    for t in range(16):
        ref, a = oracle.gemv(w, x[t], "bf16")
        check(y16[t], ref, a, "smallm T=16 k=%d t=%d" % (k_in, t))


@pytest.mark.parametrize("T", [9, 16])
def test_smallm_swiglu_pair_verify_rounds(T):
    """The gate/up pair for 9- and 16-token verify rounds (hidden 2048: one launch; 5120:
    blocks of 8 rows)."""
    q = lib()
    for hidden in (2048, 5120):
        rng = np.random.default_rng(T * 31 + hidden)
        gate = synth.draw_matrix(rng, 384, hidden, 64, "bf16")
        up = synth.draw_matrix(rng, 384, hidden, 64, "bf16")
        x, xd = _x(rng, T, hidden)
        h = nan_like((T, 384), torch.float32)
        q.qgemv_int4_smallm([dev_matrix(gate), dev_matrix(up)], xd, [h], epilogue=q.EPI_SWIGLU_PAIR)
        torch.cuda.synchronize()
        for t in range(T):
            ref, a = oracle.swiglu_pair(gate, up, x[t], "bf16")
            check_f32(to_np64(h[t]), ref, "swiglu T=%d hidden %d t=%d" % (T, hidden, t), a_ref=a)


@pytest.mark.parametrize("T", [9, 16])
def test_smallm_more_tiles_than_workgroups(T):
    """From 8 tokens on a workgroup takes several 16-row tiles (its staged activation serves
    them all): the q/k/v set (384 tiles on at most 256 workgroups at T = 16) and a 4160-row
    gate/up pair at hidden 5120 (260 tiles; blocks of 8 rows, then the rest), every output."""
    q = lib()
    rng = np.random.default_rng(900 + T)
    ws = [synth.draw_matrix(rng, n, 4096, 64, "bf16") for n in (4096, 1024, 1024)]
    x, xd = _x(rng, T, 4096)
    ys = [nan_like((T, w.n_out), torch.bfloat16) for w in ws]
    q.qgemv_int4_smallm([dev_matrix(w) for w in ws], xd, ys)
    torch.cuda.synchronize()
    for w, y in zip(ws, ys):
        for t in range(T):
            ref, a = oracle.gemv(w, x[t], "bf16", threads=oracle_threads())
            check(y[t], ref, a, "smallm qkv T=%d n=%d t=%d" % (T, w.n_out, t))
    gate = synth.draw_matrix(rng, 4160, 5120, 64, "bf16")
    up = synth.draw_matrix(rng, 4160, 5120, 64, "bf16")
    x, xd = _x(rng, T, 5120)
    h = nan_like((T, 4160), torch.float32)
    q.qgemv_int4_smallm([dev_matrix(gate), dev_matrix(up)], xd, [h], epilogue=q.EPI_SWIGLU_PAIR)
    torch.cuda.synchronize()
    for t in range(T):
        ref, a = oracle.swiglu_pair(gate, up, x[t], "bf16")
        check_f32(to_np64(h[t]), ref, "swiglu pair 4160 T=%d t=%d" % (T, t), a_ref=a)
