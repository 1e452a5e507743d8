"""GPU parity of qgemm_int4_padT (prefill, bf16 MFMA) against the fp64 oracle.

The oracle for this path rounds each dequantised weight once to bfloat16 before
the product, because the kernel multiplies bf16 weights held in LDS; the
kernel's float32 dequantisation step is covered by gemm_rounding_slack.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import (check, check_gemm, check_bf16, dev_matrix, gemm_rounding_slack, lib,
                              oracle_threads, prefill_reference, require_gpu, to_np64)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _gemm(w, X_np, y_dtype=torch.bfloat16, ldx=None, ldy=None, fill=float("nan")):
    q = lib()
    T, K = X_np.shape
    ldx = ldx or K
    ldy = ldy or w.n_out
    xs = torch.zeros((T, ldx), dtype=torch.bfloat16, device="cuda")
    xs[:, :K] = synth.to_torch(X_np, "bf16")
    y = torch.full((T, ldy), fill, dtype=y_dtype, device="cuda")
    q.qgemm_int4_padT(dev_matrix(w), xs, y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T,n_out,k_in,g", [(1, 32, 64, 64), (5, 96, 96, 32), (32, 64, 256, 64),
                                            (33, 128, 512, 128), (64, 256, 320, 64),
                                            (100, 160, 128, 32), (130, 288, 1024, 64),
                                            (257, 512, 640, 64)])
@pytest.mark.parametrize("y_dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("sbd", ["bf16", "f32"])
def test_gemm_small_full(T, n_out, k_in, g, y_dt, sbd):
    rng = np.random.default_rng(T * 7 + n_out + k_in)
    w = synth.draw_matrix(rng, n_out, k_in, g, sbd)
    X = synth.draw_activation(rng, (T, k_in), "bf16")
    y = _gemm(w, X, y_dt)
    Y_ref, A_ref = oracle.gemm(w, X, "bf16", round_w=True, threads=oracle_threads())
    slack, n_sites = gemm_rounding_slack(w, X)
    if sbd == "bf16":
        assert n_sites == 0
    check_gemm(y, Y_ref, A_ref, "gemm %d/%d/%d %s" % (T, n_out, k_in, sbd), slack=slack)


def test_gemm_identity_probe_recovers_codes():
    """X = I (T = K = 256), s = 1, b = 0: Y^T is the code matrix, bit-exact."""
    rng = np.random.default_rng(81)
    n_out, k_in = 64, 256
    raw = rng.integers(0, 16, size=(n_out, k_in), dtype=np.uint8)
    w = synth.QMatrix(codes=synth.pack_codes(raw),
                      scales=synth.f32_to_bf16_bits(np.ones((n_out, 4), np.float32)),
                      biases=synth.f32_to_bf16_bits(np.zeros((n_out, 4), np.float32)),
                      sb_dtype="bf16", group_size=64, n_out=n_out, k_in=k_in)
    X = synth.f32_to_bf16_bits(np.eye(k_in, dtype=np.float32))
    y = _gemm(w, X, torch.float32)
    assert np.array_equal(to_np64(y).T, raw.astype(np.float64))


def test_gemm_padding_invariant_and_canary():
    """T=1000 equals rows 0..999 of T=1024 with zero rows; rows >= T never written."""
    rng = np.random.default_rng(82)
    w = synth.draw_matrix(rng, 256, 512, 64, "bf16")
    X = synth.draw_activation(rng, (1000, 512), "bf16")
    Xp = np.concatenate([X, np.zeros((24, 512), np.uint16)])
    q = lib()
    dw = dev_matrix(w)
    xs = synth.to_torch(Xp, "bf16")
    y_big = torch.full((1024, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    q.qgemm_int4_padT(dw, xs, y_big)
    # T=1000 into a 1024-row buffer whose last 24 rows hold a canary
    y_small = torch.full((1024, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    q.qgemm_int4_padT(dw, xs[:1000], y_small[:1000])
    torch.cuda.synchronize()
    assert torch.equal(y_small[:1000], y_big[:1000])
    assert torch.all(y_small[1000:] == 7.0)
    assert torch.all(y_big[1000:] == 0.0)


def test_gemm_strided_rows():
    rng = np.random.default_rng(83)
    w = synth.draw_matrix(rng, 96, 192, 64, "bf16")
    X = synth.draw_activation(rng, (40, 192), "bf16")
    y = _gemm(w, X, torch.bfloat16, ldx=200, ldy=104, fill=3.0)
    Y_ref, A_ref = oracle.gemm(w, X, "bf16")
    got = to_np64(y)
    check_bf16(got[:, :96], Y_ref, A_ref, "strided")
    assert np.all(got[:, 96:] == 3.0)


@pytest.mark.parametrize("T", synth.PREFILL_T)
def test_prefill_workload_full(T):
    """K=5120, N=17408, bf16 activations: every output of the T rows against the oracle."""
    d, Y_ref, A_ref = prefill_reference(T)
    y = _gemm(d["w"], d["X"], torch.bfloat16)
    rel = check_gemm(y, Y_ref, A_ref, "prefill T=%d" % T)
    print("prefill T=%d max rel %.3e" % (T, rel))


@pytest.mark.parametrize("T,n_out,k_in,g,sbd,y_dt", [
    (2049, 32, 64, 64, "bf16", torch.bfloat16),
    (2100, 544, 96, 32, "f32", torch.float32),
    (2200, 1056, 320, 64, "bf16", torch.float32),
    (4100, 96, 1024, 128, "bf16", torch.bfloat16),
    (2049, 512, 640, 64, "f32", torch.bfloat16),
])
def test_gemm_long_prompt_full(T, n_out, k_in, g, sbd, y_dt):
    """Long prompts (the 128 x 512-tile form): ragged T, n_out not a multiple of the tile,
    k_in not a multiple of 64, both scale dtypes and output dtypes; every output."""
    rng = np.random.default_rng(T + 3 * n_out + k_in)
    w = synth.draw_matrix(rng, n_out, k_in, g, sbd)
    X = synth.draw_activation(rng, (T, k_in), "bf16")
    y = _gemm(w, X, y_dt)
    Y_ref, A_ref = oracle.gemm(w, X, "bf16", round_w=True, threads=oracle_threads())
    slack, n_sites = gemm_rounding_slack(w, X)
    if sbd == "bf16":
        assert n_sites == 0
    check_gemm(y, Y_ref, A_ref, "gemm long %d/%d/%d %s" % (T, n_out, k_in, sbd), slack=slack)
