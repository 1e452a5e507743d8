"""GPU parity of qgemm_int4_padT_ws (prefill GEMM with a K-split workspace, T <= 64)
against the fp64 oracle with bf16-rounded weights, as for qgemm_int4_padT.

The split changes only the order in which float32 partial sums over k are added,
so the bounds are those of qgemm_int4_padT.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import (check, check_gemm, dev_matrix, gemm_rounding_slack, lib, oracle_threads,
                              prefill_reference, require_gpu, to_np64)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _ws_for(T, w, scale=1.0):
    q = lib()
    n = q.qgemm_int4_padT_workspace_bytes(T, w.n_out, w.k_in)
    n = int(n * scale)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda") if n > 0 else None, n


def _gemm_ws(w, X_np, y_dtype=torch.bfloat16, ws_scale=1.0, fill=float("nan")):
    q = lib()
    T, K = X_np.shape
    xs = synth.to_torch(X_np, "bf16")
    y = torch.full((T, w.n_out), fill, dtype=y_dtype, device="cuda")
    ws, _ = _ws_for(T, w, ws_scale)
    q.qgemm_int4_padT_ws(dev_matrix(w), xs, y, ws)
    torch.cuda.synchronize()
    return y


# (T, n_out, k_in, group, sb dtype): token blocks of 16 / 32 / 64, ragged row blocks
# (n_out not a multiple of 64), ragged K (k_in not a multiple of 128, a last slice
# of one partial step), slices of 4 / 5 steps, a bf16 table starting at an odd
# group (g = 128, 5-step slices), every group size and both scale dtypes
CASES = [(1, 64, 2048, 64, "bf16"), (7, 96, 1280, 32, "bf16"), (16, 160, 2624, 64, "f32"),
         (17, 64, 1280, 128, "bf16"), (32, 224, 2560, 64, "bf16"), (33, 96, 1088, 32, "f32"),
         (48, 128, 3200, 128, "f32"), (64, 288, 2112, 64, "bf16"),
         # 35 bf16 groups per row: rows not dword-aligned, scales loaded per step
         (20, 64, 2240, 64, "bf16")]


@pytest.mark.parametrize("T,n_out,k_in,g,sbd", CASES)
@pytest.mark.parametrize("y_dt", [torch.bfloat16, torch.float32])
def test_gemm_ws_full(T, n_out, k_in, g, sbd, y_dt):
    rng = np.random.default_rng(T * 11 + n_out + k_in)
    w = synth.draw_matrix(rng, n_out, k_in, g, sbd)
    X = synth.draw_activation(rng, (T, k_in), "bf16")
    assert lib().qgemm_int4_padT_workspace_bytes(T, n_out, k_in) > 0, "shape meant to split"
    y = _gemm_ws(w, X, y_dt)
    Y_ref, A_ref = oracle.gemm(w, X, "bf16", round_w=True, threads=oracle_threads())
    slack, n_sites = gemm_rounding_slack(w, X)
    if sbd == "bf16":
        assert n_sites == 0
    check_gemm(y, Y_ref, A_ref, "gemm_ws %d/%d/%d %s" % (T, n_out, k_in, sbd), slack=slack)


@pytest.mark.parametrize("scale", [0.0, 0.4, 0.7])
def test_gemm_ws_short_workspace(scale):
    """A workspace smaller than asked for (or none) means fewer slices, same results."""
    rng = np.random.default_rng(90)
    w = synth.draw_matrix(rng, 128, 4096, 64, "bf16")
    X = synth.draw_activation(rng, (24, 4096), "bf16")
    y = _gemm_ws(w, X, torch.float32, ws_scale=scale)
    Y_ref, A_ref = oracle.gemm(w, X, "bf16", round_w=True, threads=oracle_threads())
    check_gemm(y, Y_ref, A_ref, "gemm_ws short workspace %.1f" % scale)


def test_gemm_ws_identity_probe_recovers_codes():
    """X = I (T = 64 rows of I_2048 = the first 64 columns), s = 1, b = 0: Y^T is the
    first 64 code columns, bit-exact, through split partial sums."""
    rng = np.random.default_rng(91)
    n_out, k_in, T = 64, 2048, 64
    raw = rng.integers(0, 16, size=(n_out, k_in), dtype=np.uint8)
    gpr = k_in // 64
    w = synth.QMatrix(codes=synth.pack_codes(raw),
                      scales=synth.f32_to_bf16_bits(np.ones((n_out, gpr), np.float32)),
                      biases=synth.f32_to_bf16_bits(np.zeros((n_out, gpr), np.float32)),
                      sb_dtype="bf16", group_size=64, n_out=n_out, k_in=k_in)
    X = synth.f32_to_bf16_bits(np.eye(k_in, dtype=np.float32)[:T])
    y = _gemm_ws(w, X, torch.float32)
    assert np.array_equal(to_np64(y).T, raw[:, :T].astype(np.float64))


def test_gemm_ws_matches_plain_path_and_keeps_canary():
    """Split and unsplit kernels agree to the fp32 summation-order bound; rows of y
    past T and columns past n_out (ldy > n_out) are never written."""
    rng = np.random.default_rng(92)
    q = lib()
    w = synth.draw_matrix(rng, 192, 3072, 64, "bf16")
    X = synth.draw_activation(rng, (40, 3072), "bf16")
    dw = dev_matrix(w)
    xs = synth.to_torch(X, "bf16")
    y0 = torch.full((48, 200), 5.0, dtype=torch.float32, device="cuda")
    y1 = torch.full((48, 200), 5.0, dtype=torch.float32, device="cuda")
    q.qgemm_int4_padT(dw, xs, y0[:40, :192])
    ws, n = _ws_for(40, w)
    assert n > 0
    q.qgemm_int4_padT_ws(dw, xs, y1[:40, :192], ws)
    torch.cuda.synchronize()
    _, A_ref = oracle.gemm(w, X, "bf16", round_w=True, threads=oracle_threads())
    d = (y0[:40, :192] - y1[:40, :192]).abs().cpu().double().numpy()
    assert np.all(d <= 2.0 ** -15 * A_ref)
    for y in (y0, y1):
        assert torch.all(y[40:] == 5.0) and torch.all(y[:, 192:] == 5.0)


@pytest.mark.parametrize("T", [t for t in synth.PREFILL_T if t <= 64])
def test_gemm_ws_prefill_workload_full(T):
    """K=5120, N=17408 at the workspace-split launch bench.py times: every output."""
    d, Y_ref, A_ref = prefill_reference(T)
    w, X = d["w"], d["X"]
    assert lib().qgemm_int4_padT_workspace_bytes(T, w.n_out, w.k_in) > 0
    y = _gemm_ws(w, X, torch.bfloat16)
    check_gemm(y, Y_ref, A_ref, "prefill ws T=%d" % T)
