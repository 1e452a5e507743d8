"""GPU parity at the size limits of each entry point.

* GEMV / small-M: the activation and its chunk sums are staged in LDS, so k_in is bounded by
  160 KB per workgroup; the largest accepted k_in (found by asking the library, a rejected call
  fails validation before any launch) must compute correctly, and 2^20 must be rejected.
* Prefill GEMM: a 64-step-long K range split into many slices (more partial planes than the
  reduce adds in one round), and the LDS-tiled kernel with a scale table too large for LDS
  (scales loaded per step).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import (check, check_gemm, check_bf16, dev_matrix, gemm_rounding_slack, lib, nan_like, oracle_threads,
                              require_gpu, to_np64)

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _accepts_gemv(q, k_in, x_dt, T=1):
    """True if the library accepts a T-row GEMV with this k_in (tiny dummy data, n_out = 64)."""
    w = synth.draw_matrix(np.random.default_rng(0), 64, k_in, 64, "bf16")
    dw = dev_matrix(w)
    if T == 1:
        x = torch.zeros(k_in, dtype=TD[x_dt], device="cuda")
        y = torch.empty(64, dtype=torch.float32, device="cuda")
        call = lambda: q.qgemv_int4(dw, x, y)  # noqa: E731
    else:
        x = torch.zeros((T, k_in), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((T, 64), dtype=torch.float32, device="cuda")
        call = lambda: q.qgemv_int4_smallm([dw], x, [y])  # noqa: E731
    try:
        call()
    except q.Int4Error as e:
        assert "LDS" in str(e), str(e)
        return False
    torch.cuda.synchronize()
    return True


def _largest_k(q, x_dt, T=1):
    for k in range(81920, 0, -2048):
        if _accepts_gemv(q, k, x_dt, T):
            return k
    raise AssertionError("no k_in accepted")


@pytest.mark.parametrize("x_dt", ["bf16", "f32"])
def test_gemv_largest_k_in(x_dt):
    q = lib()
    assert not _accepts_gemv(q, 1 << 20, x_dt)
    k = _largest_k(q, x_dt)
    assert k >= (32768 if x_dt == "f32" else 65536), k
    rng = np.random.default_rng(k)
    w = synth.draw_matrix(rng, 96, k, 64, "bf16")
    x = synth.draw_activation(rng, (k,), x_dt)
    y = nan_like(96, torch.float32)
    q.qgemv_int4(dev_matrix(w), synth.to_torch(x, x_dt), y)
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.gemv(w, x, x_dt, threads=oracle_threads())
    check(y, y_ref, a_ref, "gemv k_in=%d %s" % (k, x_dt))
    print("largest %s k_in %d" % (x_dt, k))


def test_smallm_largest_k_in_at_8_tokens():
    q = lib()
    k = _largest_k(q, "bf16", T=8)
    rng = np.random.default_rng(k + 1)
    w = synth.draw_matrix(rng, 64, k, 64, "bf16")
    X = synth.draw_activation(rng, (8, k), "bf16")
    y = torch.full((8, 64), float("nan"), dtype=torch.float32, device="cuda")
    q.qgemv_int4_smallm([dev_matrix(w)], synth.to_torch(X, "bf16"), [y])
    torch.cuda.synchronize()
    for t in range(8):
        y_ref, a_ref = oracle.gemv(w, X[t], "bf16", threads=oracle_threads())
        check(y[t], y_ref, a_ref, "smallm T=8 k_in=%d row %d" % (k, t))
    print("largest 8-token k_in %d" % k)


def test_gemm_ws_long_k_many_slices():
    """k_in = 65536 (512 steps), 64 rows: the planner cuts K into many slices, more than
    the reduce adds in one round of eight planes."""
    q = lib()
    T, n_out, k_in = 16, 64, 65536
    n = q.qgemm_int4_padT_workspace_bytes(T, n_out, k_in)
    assert n >= 9 * T * n_out * 4, n                      # at least nine partial planes
    rng = np.random.default_rng(95)
    w = synth.draw_matrix(rng, n_out, k_in, 64, "bf16")
    X = synth.draw_activation(rng, (T, k_in), "bf16")
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.full((T, n_out), float("nan"), dtype=torch.float32, device="cuda")
    q.qgemm_int4_padT_ws(dev_matrix(w), synth.to_torch(X, "bf16"), y, ws)
    torch.cuda.synchronize()
    Y_ref, A_ref = oracle.gemm(w, X, "bf16", round_w=True, threads=oracle_threads())
    check_gemm(y, Y_ref, A_ref, "ws k_in=65536")


@pytest.mark.parametrize("sbd", ["bf16", "f32"])
def test_tiled_gemm_scales_beyond_lds(sbd):
    """T = 100 (LDS-tiled kernel), k_in = 65536 with group 32: the 64-row scale and bias
    table (256 KB bf16, 512 KB f32) does not fit in LDS, so every step loads them."""
    q = lib()
    T, n_out, k_in = 100, 64, 65536
    rng = np.random.default_rng(96)
    w = synth.draw_matrix(rng, n_out, k_in, 32, sbd)
    X = synth.draw_activation(rng, (T, k_in), "bf16")
    y = torch.full((T, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    q.qgemm_int4_padT(dev_matrix(w), synth.to_torch(X, "bf16"), y)
    torch.cuda.synchronize()
    Y_ref, A_ref = oracle.gemm(w, X, "bf16", round_w=True, threads=oracle_threads())
    slack, n_sites = gemm_rounding_slack(w, X)
    if sbd == "bf16":
        assert n_sites == 0
    check_gemm(y, Y_ref, A_ref, "tiled k_in=65536 %s" % sbd, slack=slack)
