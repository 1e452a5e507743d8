"""GPU results against closed forms computed here, independently of the oracle.

* All-zero codes: every weight is its group's bias, so y = sum_g b_g * (sum of x over group g)
  -- for the GEMV (bf16 and float32 activations), the K-split stream GEMM and the LDS-tiled GEMM.
* Constant codes q = c: y = sum_g (c s_g + b_g) * (sum of x over group g).
* The K-way scalar-FMA combine of the MoE: eight slots routed to one expert with weights w_k give
  the same output as one slot of that expert with weight sum_k w_k (the combine is linear in the
  slot weights; bf16 outputs, compared within their rounding), and a zero weight removes a slot.
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_common import check_bf16, check_f32, dev_matrix, lib, require_gpu, to_np64

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _const_matrix(rng, n_out, k_in, g, sbd, code):
    """codes all equal to `code`; scales and biases drawn as usual."""
    w = synth.draw_matrix(rng, n_out, k_in, g, sbd)
    raw = np.full((n_out, k_in), code, dtype=np.uint8)
    w.codes = synth.pack_codes(raw)
    return w


def _sb64(w, a):
    arr = getattr(w, a)
    if w.sb_dtype == "bf16":
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return arr.astype(np.float64)


def _closed(w, X, code):
    """Y[t][o] = sum_g (code * s[o][g] + b[o][g]) * sum_{k in g} X[t][k], in float64."""
    g = w.group_size
    s64, b64 = _sb64(w, "scales"), _sb64(w, "biases")
    Xg = X.reshape(X.shape[0], -1, g).sum(axis=2)            # [T][groups]
    W = code * s64 + b64                                      # [n_out][groups]
    A = np.abs(Xg) @ np.abs(W).T                              # bound on sum |w x|
    return Xg @ W.T, A


def _x64(x_np, dt):
    if dt == "bf16":
        return (x_np.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x_np.astype(np.float64)


@pytest.mark.parametrize("code", [0, 7, 15])
@pytest.mark.parametrize("x_dt,sbd", [("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16")])
def test_gemv_constant_codes(code, x_dt, sbd):
    rng = np.random.default_rng(300 + code)
    n_out, k_in = 160, 2048
    w = _const_matrix(rng, n_out, k_in, 64, sbd, code)
    x = synth.draw_activation(rng, (k_in,), x_dt)
    y = torch.full((n_out,), float("nan"), dtype=torch.float32, device="cuda")
    lib().qgemv_int4(dev_matrix(w), synth.to_torch(x, x_dt), y)
    torch.cuda.synchronize()
    ref, A = _closed(w, _x64(x, x_dt)[None, :], code)
    # relative L2 and the per-element float32 accumulation bound (the closed form is
    # exact in float64)
    check_f32(to_np64(y), ref[0], "constant codes %d %s/%s" % (code, x_dt, sbd), a_ref=A[0])


@pytest.mark.parametrize("code", [0, 15])
@pytest.mark.parametrize("T,ws", [(16, True), (48, True), (48, False), (100, False)])
def test_gemm_constant_codes(code, T, ws):
    """bf16 scales and biases: with code 0 the weight is the bias exactly (a bf16 value);
    with 15, 15 s + b in float32, rounded to bf16 as the kernels and the oracle do."""
    q = lib()
    rng = np.random.default_rng(400 + code + T)
    n_out, k_in = 128, 2048
    w = _const_matrix(rng, n_out, k_in, 64, "bf16", code)
    X = synth.draw_activation(rng, (T, k_in), "bf16")
    y = torch.full((T, n_out), float("nan"), dtype=torch.float32, device="cuda")
    if ws:
        n = q.qgemm_int4_padT_workspace_bytes(T, n_out, k_in)
        assert n > 0
        q.qgemm_int4_padT_ws(dev_matrix(w), synth.to_torch(X, "bf16"), y,
                             torch.empty(n, dtype=torch.uint8, device="cuda"))
    else:
        q.qgemm_int4_padT(dev_matrix(w), synth.to_torch(X, "bf16"), y)
    torch.cuda.synchronize()
    # the bf16 weight of each group: the exact code * s + b rounded once to nearest
    # even; for bf16 s, b and a small code the product is exact in float32, so
    # torch's float32 -> bf16 cast rounds the exact value
    w_exact = code * _sb64(w, "scales") + _sb64(w, "biases")
    wf = w_exact.astype(np.float32)
    assert np.array_equal(wf.astype(np.float64), w_exact)
    wb = torch.tensor(wf).to(torch.bfloat16).float().numpy().astype(np.float64)
    Xg = _x64(X, "bf16").reshape(T, -1, 64).sum(axis=2)
    ref = Xg @ wb.T
    A = np.abs(Xg) @ np.abs(wb).T
    check_f32(to_np64(y), ref, "gemm constant codes %d T=%d" % (code, T), a_ref=A)


def test_moe_scalar_fma_chain_is_linear_in_slot_weights():
    """8 slots on one expert with weights w_k == 1 slot with weight sum w_k; a zero
    weight drops its slot (bf16 output, float32 combine)."""
    q = lib()
    m = synth.moe_layer(seed=31, n_experts=16, hidden=512, inter=256)
    g, u, d = (dev_matrix(m[k]) for k in ("gate", "up", "down"))
    x = synth.to_torch(m["x"][0], "bf16")
    w8 = torch.tensor([0.3, 0.05, 0.2, 0.0, 0.15, 0.1, 0.12, 0.08], dtype=torch.float32, device="cuda")

    def run(ids, wts):
        out = torch.full((512,), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(q.moe_gather_qgemv_int4_workspace_bytes(d, len(ids)), dtype=torch.uint8,
                         device="cuda")
        q.moe_gather_qgemv_int4(g, u, d, x, torch.tensor(ids, dtype=torch.int32, device="cuda"),
                                wts, out, ws)
        torch.cuda.synchronize()
        return to_np64(out)

    e = 5
    chain = run([e] * 8, w8)
    one = run([e], w8.sum().reshape(1))
    # linear in the slot weights: equal up to the bf16 rounding of the two outputs
    assert np.all(np.abs(chain - one) <= 2.0 ** -7 * np.abs(one) + 2.0 ** -12 * np.abs(one).max())
    assert np.abs(one).max() > 0
    # zero weight: slot 3 (weight 0) contributes nothing, even with a different expert
    ids = [e] * 8
    ids[3] = 9
    assert np.array_equal(run(ids, w8), chain)
