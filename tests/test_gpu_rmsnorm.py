"""GPU parity of rms_norm_qgemv_int4 (RMSNorm prologue fused into the GEMV) against the
fp64 oracle, through the C ABI.  Tolerances are those of qgemv_int4 (float32: relative
L2 <= 1e-5; bf16: per element 2^-7 |y| + 2^-16 a)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import check, check_f32, dev_matrix, lib, nan_like, oracle_threads, require_gpu, to_np64

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}
EPS = float(np.float32(1e-6))


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _run(ws, x, gamma, x_dt, y_dt, eps=EPS, epilogue=0, n_outs=None):
    q = lib()
    dws = [dev_matrix(w) for w in ws]
    n_outs = n_outs if n_outs is not None else [w.n_out for w in ws]
    ys = [nan_like(n, TD[y_dt]) for n in n_outs]
    q.rms_norm_qgemv_int4(dws, synth.to_torch(x, x_dt), synth.to_torch(gamma, x_dt), eps, ys,
                          epilogue=epilogue)
    torch.cuda.synchronize()
    return ys


def test_rms_qkv_workload_full_size():
    """The measured workload: RMSNorm + q/k/v 4096 -> 4096/1024/1024, bf16 in and out."""
    d = synth.rms_qkv()
    ys = _run(d["ws"], d["x"], d["gamma"], "bf16", "bf16", eps=d["eps"])
    refs = oracle.rms_norm_multi(d["ws"], d["x"], "bf16", d["gamma"], d["eps"],
                                 threads=oracle_threads())
    for i, (y, (ref, a)) in enumerate(zip(ys, refs)):
        check(y, ref, a, "rms qkv %d" % i)


@pytest.mark.parametrize("n_out,k_in,g", [(1, 64, 64), (7, 96, 32), (100, 1024, 128), (257, 5120, 64),
                                          (130, 2048, 32), (50, 17408, 64), (1000, 4096, 64)])
@pytest.mark.parametrize("x_dt,sb_dt,y_dt", [("bf16", "bf16", "bf16"), ("f32", "f32", "f32"),
                                             ("bf16", "bf16", "f32"), ("f32", "bf16", "bf16")])
def test_rms_single_shapes_and_dtypes(n_out, k_in, g, x_dt, sb_dt, y_dt):
    rng = np.random.default_rng(3 * n_out + k_in + g)
    w = synth.draw_matrix(rng, n_out, k_in, g, sb_dt)
    x = synth.draw_activation(rng, (k_in,), x_dt)
    gamma = synth.draw_norm_weight(rng, k_in, x_dt)
    (y,) = _run([w], x, gamma, x_dt, y_dt)
    (ref, a), = oracle.rms_norm_multi([w], x, x_dt, gamma, EPS)
    check(y, ref, a, "rms %dx%d g%d %s/%s/%s" % (n_out, k_in, g, x_dt, sb_dt, y_dt))


@pytest.mark.parametrize("scale,eps", [(1e-3, EPS), (300.0, EPS), (1.0, 1.0), (1e-4, 1e-2)])
def test_rms_input_scale_and_eps(scale, eps):
    """Tiny, huge and eps-dominated inputs: the normaliser is taken inside the kernel."""
    rng = np.random.default_rng(int(scale * 1000) + 7)
    w = synth.draw_matrix(rng, 384, 2048, 64, "bf16")
    x = (scale * rng.standard_normal(2048)).astype(np.float32)
    gamma = synth.draw_norm_weight(rng, 2048, "f32")
    eps = float(np.float32(eps))
    (y,) = _run([w], x, gamma, "f32", "f32", eps=eps)
    (ref, a), = oracle.rms_norm_multi([w], x, "f32", gamma, eps)
    check(y, ref, a, "rms scale %g eps %g" % (scale, eps))


def test_rms_swiglu_pair():
    """Pre-FFN norm fused with the gate/up pair: h = silu(gate xn) * (up xn), float32."""
    rng = np.random.default_rng(61)
    hidden, inter = 1024, 768
    gate = synth.draw_matrix(rng, inter, hidden, 64, "bf16")
    up = synth.draw_matrix(rng, inter, hidden, 64, "bf16")
    x = synth.draw_activation(rng, (hidden,), "bf16")
    gamma = synth.draw_norm_weight(rng, hidden, "bf16")
    (h,) = _run([gate, up], x, gamma, "bf16", "f32", epilogue=lib().EPI_SWIGLU_PAIR, n_outs=[inter])
    ref, a = oracle.rms_norm_swiglu_pair(gate, up, x, "bf16", gamma, EPS)
    got = to_np64(h)
    assert np.all(np.isfinite(got))
    # float32 SwiGLU of float32 sums: the bound of the plain SwiGLU test
    check_f32(got, ref, "rms swiglu h", a_ref=a)


def test_rms_one_hot_column():
    """x = a e_k: xn = sqrt(K / (a^2 + K eps)) * a * gamma_k e_k selects column k."""
    rng = np.random.default_rng(62)
    K = 1024
    w = synth.draw_matrix(rng, 200, K, 64, "f32")
    gamma = synth.draw_norm_weight(rng, K, "f32")
    for k in (0, 517, K - 1):
        x = np.zeros(K, np.float32)
        x[k] = -2.5
        (y,) = _run([w], x, gamma, "f32", "f32")
        (ref, a), = oracle.rms_norm_multi([w], x, "f32", gamma, EPS)
        check(y, ref, a, "one-hot %d" % k)


def test_rms_matches_plain_multi_on_normalised_input():
    """Against the already-parity-tested qgemv_int4_multi on the host-normalised float32 input:
    the two launches see the same float32 activation up to its rounding, so they agree to 1e-5."""
    q = lib()
    d = synth.rms_qkv(seed=9, hidden=2048, outs=(512, 256))
    y_rms = _run(d["ws"], d["x"], d["gamma"], "bf16", "f32", eps=d["eps"])
    xn = oracle.rms_norm(d["x"], "bf16", d["gamma"], d["eps"]).astype(np.float32)
    ys = [nan_like(w.n_out, torch.float32) for w in d["ws"]]
    q.qgemv_int4_multi([dev_matrix(w) for w in d["ws"]], torch.tensor(xn, device="cuda"), ys)
    torch.cuda.synchronize()
    for a_, b_ in zip(y_rms, ys):
        a64, b64 = to_np64(a_), to_np64(b_)
        assert np.linalg.norm(a64 - b64) / np.linalg.norm(b64) <= 1e-5


# the activation-stationary form behind the RMSNorm prologue (x * gamma and sum(x^2) taken in
# registers, the row sums scaled at the end): one matrix over 2048, 5120 and 17408 columns,
# q/k/v of a 5120 activation, and gate/up pairs over 2048 and 6144 columns
XS_RMS = [([12801], 2048, "bf16", 0), ([5120], 5120, "bf16", 0), ([2000], 17408, "f32", 0),
          ([5120, 1024, 1024], 5120, "bf16", 0), ([8192, 8192], 2048, "bf16", 1),
          ([3000, 3000], 6144, "f32", 1)]


@pytest.mark.parametrize("n_outs,k_in,x_dt,pair", XS_RMS)
@pytest.mark.parametrize("sb_dt,y_dt", [("bf16", "bf16"), ("f32", "f32")])
def test_rms_xs_forms(n_outs, k_in, x_dt, pair, sb_dt, y_dt):
    q = lib()
    epi = q.EPI_SWIGLU_PAIR if pair else q.EPI_NONE
    f = q.plan_qgemv(n_outs, k_in, x_dtype=x_dt, epilogue=epi, call=q.CALL_RMS_NORM)
    assert f["kernel"] == "xs", f
    rng = np.random.default_rng(sum(n_outs) + k_in + pair)
    ws = [synth.draw_matrix(rng, n, k_in, 64, sb_dt) for n in n_outs]
    x = synth.draw_activation(rng, (k_in,), x_dt)
    gamma = synth.draw_norm_weight(rng, k_in, x_dt)
    if pair:
        (h,) = _run(ws, x, gamma, x_dt, y_dt, epilogue=epi, n_outs=[n_outs[0]])
        ref, a = oracle.rms_norm_swiglu_pair(ws[0], ws[1], x, x_dt, gamma, EPS, threads=oracle_threads())
        check(h, ref, a, "xs rms pair %dx%d %s %s/%s" % (n_outs[0], k_in, x_dt, sb_dt, y_dt))
        return
    ys = _run(ws, x, gamma, x_dt, y_dt)
    refs = oracle.rms_norm_multi(ws, x, x_dt, gamma, EPS, threads=oracle_threads())
    for i, (y, (ref, a)) in enumerate(zip(ys, refs)):
        check(y, ref, a, "xs rms %s x %d matrix %d %s %s/%s" % (n_outs, k_in, i, x_dt, sb_dt, y_dt))


def test_rms_xs_matches_plain_xs_on_normalised_input():
    """The RMSNorm form of the activation-stationary kernel against its plain form on the
    host-normalised float32 input (both parity-tested): they agree to 1e-5."""
    q = lib()
    rng = np.random.default_rng(404)
    ws = [synth.draw_matrix(rng, n, 5120, 64, "bf16") for n in (5120, 1024, 1024)]
    x = synth.draw_activation(rng, (5120,), "bf16")
    gamma = synth.draw_norm_weight(rng, 5120, "bf16")
    assert q.plan_qgemv([5120, 1024, 1024], 5120, x_dtype="f32")["kernel"] == "xs"
    y_rms = _run(ws, x, gamma, "bf16", "f32")
    xn = oracle.rms_norm(x, "bf16", gamma, EPS).astype(np.float32)
    ys = [nan_like(w.n_out, torch.float32) for w in ws]
    q.qgemv_int4_multi([dev_matrix(w) for w in ws], torch.tensor(xn, device="cuda"), ys)
    torch.cuda.synchronize()
    for a_, b_ in zip(y_rms, ys):
        a64, b64 = to_np64(a_), to_np64(b_)
        assert np.linalg.norm(a64 - b64) / np.linalg.norm(b64) <= 1e-5
