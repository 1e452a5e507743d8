"""GPU parity of moe_router_topk against the fp64 oracle router (through the C ABI).

Expert ids are integer decisions and must match exactly; the kernel ranks the
logits (exact inputs) and the oracle the fp64 probabilities, which order the
same way.  Weights are float32 softmaxes over at most 8 kept logits: each is
within a few float32 ulps of the fp64 value (rtol 2e-6 here).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import check, dev_matrix, lib, nan_like, require_gpu

pytestmark = pytest.mark.gpu

W_RTOL = 2e-6


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _route(logits: np.ndarray, top_k: int, dtype: str = "f32"):
    """logits: [n_tokens][n_experts] float32 (or uint16 bf16 bits)."""
    q = lib()
    n_tokens = logits.shape[0]
    lg = synth.to_torch(logits, dtype)
    ids = torch.full((n_tokens, top_k), -1, dtype=torch.int32, device="cuda")
    wts = torch.full((n_tokens, top_k), float("nan"), dtype=torch.float32, device="cuda")
    q.moe_router_topk(lg, top_k, ids, wts)
    torch.cuda.synchronize()
    return ids.cpu().numpy().astype(np.int64), wts.cpu().numpy().astype(np.float64)


def _expect(logits64: np.ndarray, top_k: int):
    ids, wts = zip(*(oracle.router_topk(row, top_k) for row in logits64))
    return np.array(ids), np.array(wts)


@pytest.mark.parametrize("n_experts", [8, 64, 128, 256, 1000, 4096])
@pytest.mark.parametrize("top_k", [1, 2, 8])
def test_router_random_logits(n_experts, top_k):
    if top_k > n_experts:
        pytest.skip("top_k > n_experts")
    rng = np.random.default_rng(n_experts * 10 + top_k)
    logits = rng.standard_normal((37, n_experts)).astype(np.float32)
    ids, wts = _route(logits, top_k)
    ref_ids, ref_wts = _expect(logits.astype(np.float64), top_k)
    assert np.array_equal(ids, ref_ids)
    np.testing.assert_allclose(wts, ref_wts, rtol=W_RTOL, atol=0)
    np.testing.assert_allclose(wts.sum(axis=1), 1.0, rtol=1e-6)


def test_router_bf16_logits():
    rng = np.random.default_rng(5)
    logits = synth.f32_to_bf16_bits(rng.standard_normal((16, 128)).astype(np.float32))
    ids, wts = _route(logits, 8, "bf16")
    ref_ids, ref_wts = _expect(synth.bf16_bits_to_f32(logits).astype(np.float64), 8)
    assert np.array_equal(ids, ref_ids)
    np.testing.assert_allclose(wts, ref_wts, rtol=W_RTOL, atol=0)


def test_router_ties_go_to_smaller_index():
    """Integer logits from a tiny range: most of the top-8 are ties."""
    rng = np.random.default_rng(6)
    logits = rng.integers(0, 3, size=(20, 256)).astype(np.float32)
    ids, wts = _route(logits, 8)
    ref_ids, ref_wts = _expect(logits.astype(np.float64), 8)
    assert np.array_equal(ids, ref_ids)
    np.testing.assert_allclose(wts, ref_wts, rtol=W_RTOL, atol=0)
    # the page's worked example, as one more row
    ids1, wts1 = _route(np.array([[1, 5, 3, 4]], np.float32), 2)
    assert ids1.tolist() == [[1, 3]]
    np.testing.assert_allclose(wts1[0], [0.7310585786300049, 0.2689414213699951], rtol=W_RTOL)


@pytest.mark.parametrize("n_experts", [64, 128, 256])
def test_router_negative_logits_and_signed_zeros(n_experts):
    """Integer logits from -3 to 3 with zeros of both signs: -0 and +0 tie (the lower index goes
    first) and negative logits rank below positive ones in their float order."""
    rng = np.random.default_rng(n_experts + 8)
    logits = rng.integers(-3, 4, size=(24, n_experts)).astype(np.float32)
    zeros = logits == 0
    logits[zeros & (rng.random(logits.shape) < 0.5)] = -0.0
    logits[:4] = -np.abs(logits[:4])  # rows with no positive logit
    ids, wts = _route(logits, 8)
    ref_ids, ref_wts = _expect(logits.astype(np.float64), 8)
    assert np.array_equal(ids, ref_ids)
    np.testing.assert_allclose(wts, ref_wts, rtol=W_RTOL, atol=0)


def test_router_nan_and_inf_logits():
    """NaN ranks below every number; -inf logits get weight 0."""
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((8, 64)).astype(np.float32)
    logits[:, ::3] = np.nan
    logits[0, 1] = np.inf * -1
    logits[1, :] = -np.inf
    logits[1, 10] = 0.5
    ids, wts = _route(logits, 4)
    ranked = np.where(np.isnan(logits), -np.inf, logits).astype(np.float64)
    ref_ids, ref_wts = _expect(ranked, 4)
    assert np.array_equal(ids, ref_ids)
    np.testing.assert_allclose(wts, ref_wts, rtol=W_RTOL, atol=1e-30)
    assert wts[1, 0] == 1.0 and np.all(wts[1, 1:] == 0.0)


def test_router_feeds_moe_without_host_round_trip():
    """Router and expert gather on one stream; result equals the fp64 MoE of the oracle route."""
    q = lib()
    d = synth.moe_layer()
    gate, up, down = (dev_matrix(d[k]) for k in ("gate", "up", "down"))
    hidden, inter = d["gate"].k_in, d["gate"].n_out
    logits = torch.tensor(d["logits"][0][None, :].astype(np.float32), device="cuda")
    ids = torch.empty(8, dtype=torch.int32, device="cuda")
    wts = torch.empty(8, dtype=torch.float32, device="cuda")
    ws = torch.empty(q.moe_gather_qgemv_int4_workspace_bytes(down, 8), dtype=torch.uint8,
                     device="cuda")
    out = nan_like(hidden, torch.bfloat16)
    x = synth.to_torch(d["x"][0], "bf16")
    res = synth.to_torch(d["residual"][0], "bf16")
    q.moe_router_topk(logits, 8, ids, wts)
    q.moe_gather_qgemv_int4(gate, up, down, x, ids, wts, out, ws, residual=res)
    torch.cuda.synchronize()
    ref_ids, ref_wts = oracle.router_topk(d["logits"][0], 8)
    assert ids.cpu().numpy().tolist() == ref_ids.tolist()
    ref, a_ref = oracle.moe(d["gate"], d["up"], d["down"], d["x"][0], ref_ids,
                            wts.cpu().numpy(), d["residual"][0], "bf16")
    check(out, ref, a_ref, "router + moe")


def _moe_inputs(E, top_k, seed, logit_dtype="f32"):
    d = synth.moe_layer(seed=seed, n_experts=E, hidden=256, inter=128)
    logits = d["logits"][0]
    if logit_dtype == "bf16":
        logits = synth.f32_to_bf16_bits(logits)
    return d, logits


@pytest.mark.parametrize("E,top_k", [(8, 1), (8, 8), (64, 4), (128, 8), (256, 8), (200, 3)])
@pytest.mark.parametrize("logit_dtype", ["f32", "bf16"])
def test_fused_route_gather_equals_router_then_gather(E, top_k, logit_dtype):
    """moe_route_gather_qgemv_int4 == moe_router_topk + moe_gather_qgemv_int4, bit for bit
    (ids, weights and the output), and the oracle agrees."""
    q = lib()
    d, logits = _moe_inputs(E, top_k, seed=E * 10 + top_k, logit_dtype=logit_dtype)
    gate, up, down = (dev_matrix(d[k]) for k in ("gate", "up", "down"))
    lg = synth.to_torch(logits, logit_dtype)
    x = synth.to_torch(d["x"][0], "bf16")
    res = synth.to_torch(d["residual"][0], "bf16")
    ws = torch.empty(q.moe_gather_qgemv_int4_workspace_bytes(down, top_k), dtype=torch.uint8, device="cuda")
    ids1 = torch.full((top_k,), -1, dtype=torch.int32, device="cuda")
    wts1 = torch.full((top_k,), float("nan"), dtype=torch.float32, device="cuda")
    out1 = nan_like(256, torch.bfloat16)
    q.moe_router_topk(lg, top_k, ids1, wts1)
    q.moe_gather_qgemv_int4(gate, up, down, x, ids1, wts1, out1, ws, residual=res)
    ids2 = torch.full((top_k,), -1, dtype=torch.int32, device="cuda")
    wts2 = torch.full((top_k,), float("nan"), dtype=torch.float32, device="cuda")
    out2 = nan_like(256, torch.bfloat16)
    q.moe_route_gather_qgemv_int4(gate, up, down, x, lg, top_k, ids2, wts2, out2, ws, residual=res)
    torch.cuda.synchronize()
    assert torch.equal(ids1, ids2)
    assert torch.equal(wts1.view(torch.int32), wts2.view(torch.int32))
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    l64 = (synth.bf16_bits_to_f32(logits) if logit_dtype == "bf16" else logits).astype(np.float64)
    ref_ids, _ = oracle.router_topk(l64, top_k)
    assert ids2.cpu().numpy().tolist() == ref_ids.tolist()
    ref, a = oracle.moe(d["gate"], d["up"], d["down"], d["x"][0], ref_ids, wts2.cpu().numpy(),
                        d["residual"][0], "bf16")
    check(out2, ref, a, "fused route+gather")


def test_fused_route_gather_nan_and_all_neg_inf():
    """NaN logits rank last; an all -inf row keeps experts 0..k-1 with weights 1/k."""
    q = lib()
    for case in ("nan", "neginf"):
        d, logits = _moe_inputs(64, 4, seed=3)
        logits = logits.copy()
        if case == "nan":
            logits[::2] = np.nan
        else:
            logits[:] = -np.inf
        gate, up, down = (dev_matrix(d[k]) for k in ("gate", "up", "down"))
        lg = synth.to_torch(logits, "f32")
        x = synth.to_torch(d["x"][0], "bf16")
        ws = torch.empty(q.moe_gather_qgemv_int4_workspace_bytes(down, 4), dtype=torch.uint8, device="cuda")
        ids = torch.empty(4, dtype=torch.int32, device="cuda")
        wts = torch.empty(4, dtype=torch.float32, device="cuda")
        out = nan_like(256, torch.bfloat16)
        q.moe_route_gather_qgemv_int4(gate, up, down, x, lg, 4, ids, wts, out, ws)
        ids_r = torch.empty(4, dtype=torch.int32, device="cuda")
        wts_r = torch.empty(4, dtype=torch.float32, device="cuda")
        q.moe_router_topk(lg, 4, ids_r, wts_r)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_r) and torch.equal(wts, wts_r), case
        if case == "neginf":
            assert ids.cpu().tolist() == [0, 1, 2, 3] and np.allclose(wts.cpu().numpy(), 0.25)
        assert torch.isfinite(out.float()).all()
