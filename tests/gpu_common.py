"""Shared helpers of the GPU parity tests: device upload and the tolerance rules.

Tolerances (stated once, used by every parity test):
  * unpacked codes: bit-exact;
  * float32 outputs: relative L2 error ||y_hat - y||_2 / ||y||_2 <= 1e-5;
  * bfloat16 outputs: per element |y_hat - y| <= 2^-7 |y| + 2^-16 a, where y is
    the unrounded fp64 oracle value and a = sum_k |w_k x_k| (plus what the
    float32 intermediates carry, for chained products).  The 2^-16 a floor
    covers outputs that cancel to ~0, where float32 accumulation order, not the
    method, decides the last bits; it is far below the error any real defect
    (a wrong code, group, scale or row) produces.
"""
import numpy as np
import pytest
import torch

import synth

REL_L2_F32 = 1e-5
BF16_REL = 2.0 ** -7
BF16_FLOOR = 2.0 ** -16


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def lib():
    import dequant_matmul_int4_amd as q

    q.load()
    return q


def dev_matrix(w: synth.QMatrix):
    q = lib()
    d = synth.matrix_to_torch(w)
    return q.QInt4Matrix(d["codes"], d["scales"], d["biases"], d["group_size"])


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def nan_like(n, dtype):
    return torch.full((n,) if isinstance(n, int) else n, float("nan"), dtype=dtype, device="cuda")


def check_f32(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(y_gpu)), "%s: non-finite output" % what
    err = np.linalg.norm(y_gpu - y_ref) / np.linalg.norm(y_ref)
    assert err <= REL_L2_F32, "%s: relative L2 %.3e > %.1e" % (what, err, REL_L2_F32)
    return err


def check_bf16(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(y_gpu)), "%s: non-finite output" % what
    diff = np.abs(y_gpu - y_ref)
    bound = BF16_REL * np.abs(y_ref) + BF16_FLOOR * a_ref
    bad = np.nonzero(diff > bound)[0]
    assert bad.size == 0, "%s: %d elements out of tolerance, first %s: got %r want %r (a=%r)" % (
        what, bad.size, bad[:5].tolist(), y_gpu[bad[:5]].tolist(), y_ref[bad[:5]].tolist(),
        a_ref[bad[:5]].tolist())
    rel = diff / np.maximum(np.abs(y_ref), 1e-300)
    return float(rel.max())


def check(y_gpu_t: torch.Tensor, y_ref, a_ref, what=""):
    y = to_np64(y_gpu_t).reshape(-1)
    y_ref = np.asarray(y_ref).reshape(-1)
    a_ref = np.asarray(a_ref).reshape(-1)
    if y_gpu_t.dtype == torch.float32:
        return check_f32(y, y_ref, what)
    return check_bf16(y, y_ref, a_ref, what)


def oracle_threads():
    import oracle

    return max(1, min(16, oracle.max_threads()))
