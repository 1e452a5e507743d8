"""Shared helpers of the GPU parity tests: device upload and the tolerance rules.

Tolerances (stated once, used by every parity test):
  * unpacked codes: bit-exact;
  * float32 outputs: relative L2 error ||y_hat - y||_2 / ||y||_2 <= 1e-5 over the
    whole output; where a test asks for it (products whose weights are materialised,
    and the SwiGLU intermediates), also per element |y_hat - y| <= 1e-5 |y| + 2^-16 a;
  * bfloat16 outputs: per element |y_hat - y| <= 2^-7 |y| + 2^-16 a, where y is
    the unrounded fp64 oracle value and a = sum_k |w_k x_k| (plus what the
    float32 intermediates carry, for chained products).  The 2^-16 a floor
    covers outputs that cancel to ~0, where float32 accumulation order, not the
    method, decides the last bits; it is far below the error any real defect
    (a wrong code, group, scale or row) produces.  Every bf16 check also
    reports the largest relative error without the floor and how many elements
    only the floor admitted (set QINT4_PARITY_REPORT=<file> to collect them).

Prefill GEMMs round each weight to bf16 before the product; the oracle rounds
the exact s q + b once.  The kernels form s q + b with one float32 fused
multiply-add and round that to bf16, which is the same value whenever the
float32 result is exact or does not land exactly on a bf16 rounding midpoint.
``gemm_rounding_slack`` finds the weights where the two differ (none for bf16
scales and biases in the workloads' value ranges; a few in 2^16 for float32
ones) and bounds what they move each output by.
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


REPORT = []  # one dict per bf16 / f32 check, written out by conftest when requested


def check_f32(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = "", a_ref=None, slack=None,
              elem_rel: float = REL_L2_F32):
    """Relative L2 <= 1e-5 over the output; with a_ref, also the per-element bound
    elem_rel |y| + 2^-16 a.  slack: a documented extra per-element bound, taken off each
    element's error before both tests."""
    y_gpu = np.asarray(y_gpu, np.float64).reshape(-1)
    y_ref = np.asarray(y_ref, np.float64).reshape(-1)
    assert np.all(np.isfinite(y_gpu)), "%s: non-finite output" % what
    diff = np.abs(y_gpu - y_ref)
    if slack is not None:
        diff = np.maximum(diff - np.asarray(slack, np.float64).reshape(-1), 0.0)
    nrm = np.linalg.norm(y_ref)
    err = np.linalg.norm(diff) / nrm if nrm > 0 else np.linalg.norm(diff)
    assert err <= REL_L2_F32, "%s: relative L2 %.3e > %.1e" % (what, err, REL_L2_F32)
    if a_ref is not None:
        a_ref = np.asarray(a_ref, np.float64).reshape(-1)
        bad = np.nonzero(diff > elem_rel * np.abs(y_ref) + BF16_FLOOR * a_ref)[0]
        assert bad.size == 0, "%s: %d elements outside %g |y| + 2^-16 a, first %s" % (
            what, bad.size, elem_rel, bad[:5].tolist())
    REPORT.append({"check": what, "dtype": "f32", "n": int(y_ref.size), "rel_l2": float(err)})
    return err


def check_bf16(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray, what: str = "",
               slack=None):
    """Per element |y_hat - y| <= 2^-7 |y| + 2^-16 a (+ slack, a documented extra bound).
    Returns the largest relative error; records it with the floor-rescued count."""
    y_gpu = np.asarray(y_gpu, np.float64).reshape(-1)
    y_ref = np.asarray(y_ref, np.float64).reshape(-1)
    a_ref = np.asarray(a_ref, np.float64).reshape(-1)
    assert np.all(np.isfinite(y_gpu)), "%s: non-finite output" % what
    diff = np.abs(y_gpu - y_ref)
    rel_part = BF16_REL * np.abs(y_ref)
    bound = rel_part + BF16_FLOOR * a_ref
    if slack is not None:
        bound = bound + np.asarray(slack, np.float64).reshape(-1)
    bad = np.nonzero(diff > bound)[0]
    assert bad.size == 0, "%s: %d elements out of tolerance, first %s: got %r want %r (a=%r)" % (
        what, bad.size, bad[:5].tolist(), y_gpu[bad[:5]].tolist(), y_ref[bad[:5]].tolist(),
        a_ref[bad[:5]].tolist())
    nz = np.abs(y_ref) > 0
    rel = diff[nz] / np.abs(y_ref[nz])
    max_rel = float(rel.max()) if rel.size else 0.0
    rescued = int(np.count_nonzero(diff > rel_part))
    REPORT.append({"check": what, "dtype": "bf16", "n": int(y_ref.size),
                   "max_rel_no_floor": max_rel, "floor_rescued": rescued})
    return max_rel


def gemm_rounding_slack(w, X, x_dtype="bf16", T_rows=None):
    """Extra per-output bound for the prefill GEMMs' float32 dequantisation step.

    Returns (slack [T][n_out], n_sites): n_sites weights where
    RNE_bf16(RNE_f32(w)) != RNE_bf16(w), and for each output the sum over those
    weights of |difference| * |x|.  Zero (and n_sites 0) when every float32
    dequantisation is exact or misses the bf16 midpoints."""
    import oracle

    W = oracle.dequant(w)                                  # exact, float64
    once = oracle.round_bf16(W)
    twice = oracle.round_bf16(W.astype(np.float32).astype(np.float64))
    delta = np.abs(twice - once)
    n_sites = int(np.count_nonzero(delta))
    Xa = np.abs(oracle.widen(X, x_dtype))
    if T_rows is not None:
        Xa = Xa[:T_rows]
    if n_sites == 0:
        return np.zeros((Xa.shape[0], w.n_out)), 0
    return Xa @ delta.T, n_sites


def check_gemm(y_gpu_t: torch.Tensor, y_ref, a_ref, what="", slack=None):
    """Prefill GEMM outputs (bf16 weights materialised before the product): float32 ->
    relative L2 and, per element, the float32 accumulation bound 2^-16 a; bfloat16 ->
    the per-element rule of check_bf16."""
    if y_gpu_t.dtype == torch.float32:
        return check_f32(to_np64(y_gpu_t), y_ref, what, a_ref=a_ref, slack=slack, elem_rel=0.0)
    return check(y_gpu_t, y_ref, a_ref, what, slack=slack)


def check(y_gpu_t: torch.Tensor, y_ref, a_ref, what="", slack=None):
    """Dispatch on the output dtype: float32 -> relative L2 over the output (the per-element
    float32 bound is asked for explicitly through check_f32's a_ref: a factorised GEMV,
    s (sum q x) + b (sum x), can miss it where s q + b cancels to ~0 while staying far
    inside the relative L2 bound); bfloat16 -> the per-element rule of check_bf16."""
    y = to_np64(y_gpu_t).reshape(-1)
    y_ref = np.asarray(y_ref).reshape(-1)
    a_ref = np.asarray(a_ref).reshape(-1)
    if y_gpu_t.dtype == torch.float32:
        return check_f32(y, y_ref, what, slack=slack)
    return check_bf16(y, y_ref, a_ref, what, slack=slack)


def oracle_threads():
    import oracle

    return max(1, min(16, oracle.max_threads()))


_PREFILL = {}


def prefill_reference(T: int):
    """The prefill workload with T rows (K = 5120, N = 17408) and the oracle's full
    output (Y, A) for it.  X of every T is the first T rows of the largest
    workload's X (one seeded stream, drawn row by row), and a row of Y depends
    only on its row of X, so the largest product is computed once and sliced."""
    import oracle

    t_max = max(synth.PREFILL_T)
    if T > t_max:
        raise ValueError("T above the largest prefill workload")
    if "full" not in _PREFILL:
        d = synth.prefill_gemm(T=t_max)
        Y, A = oracle.gemm(d["w"], d["X"], "bf16", round_w=True, threads=oracle_threads())
        slack, n_sites = gemm_rounding_slack(d["w"], d["X"][:1])
        assert n_sites == 0, "bf16 scales: the float32 dequantisation must be exact"
        _PREFILL["full"] = (d, Y, A)
    d, Y, A = _PREFILL["full"]
    return {"w": d["w"], "X": d["X"][:T], "T": T}, Y[:T], A[:T]
