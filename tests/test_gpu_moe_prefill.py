"""GPU parity of moe_prefill_qgemm_int4 (expert-sorted gather GEMMs) against the fp64
oracle's prefill MoE, through the C ABI.

Tolerances are the GEMM/MoE ones: bf16 outputs per element 2^-7 |y| + 2^-16 a (a the
oracle's magnitude including what h carries into the down product), float32 outputs
relative L2 <= 1e-5.  Router ids are integer inputs drawn by the oracle's router from
seeded N(0,1) logits, except where the device router produces them.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import check, dev_matrix, lib, nan_like, oracle_threads, require_gpu

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _route(logits, k):
    pairs = [oracle.router_topk(row.astype(np.float64), k) for row in logits]
    ids = np.array([p[0] for p in pairs], dtype=np.int64)
    wts = np.array([p[1] for p in pairs], dtype=np.float32)
    return ids, wts


def _run(d, ids, wts, out_dt="bf16", residual=True, ldx=None, mats=None):
    q = lib()
    gate, up, down = mats or (dev_matrix(d["gate"]), dev_matrix(d["up"]), dev_matrix(d["down"]))
    T, hidden = d["x"].shape
    inter = d["gate"].n_out
    ldx = ldx or hidden
    x = torch.full((T, ldx), float("nan"), dtype=torch.bfloat16, device="cuda")
    x[:, :hidden] = synth.to_torch(d["x"], "bf16")
    res = synth.to_torch(d["residual"], "bf16").to(TD[out_dt]) if residual else None
    out = nan_like((T, hidden), TD[out_dt])
    nb = q.moe_prefill_qgemm_int4_workspace_bytes(T, ids.shape[1], d["gate"].n_experts, hidden, inter)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    q.moe_prefill_qgemm_int4(gate, up, down, x, torch.tensor(ids.astype(np.int32), device="cuda"),
                             torch.tensor(wts, device="cuda"), out, ws, residual=res)
    torch.cuda.synchronize()
    return out


def _expect(d, ids, wts, residual=True, out_dt="bf16", tokens=None):
    res = None
    if residual:
        res = d["residual"] if out_dt == "bf16" else synth.bf16_bits_to_f32(d["residual"])
    return oracle.moe_prefill(d["gate"], d["up"], d["down"], d["x"], ids, wts, res,
                              res_dtype=out_dt, tokens=tokens, threads=oracle_threads())


def _check_rows(out, ref, a, tokens, what):
    for i, t in enumerate(tokens):
        check(out[t], ref[i], a[i], "%s token %d" % (what, t))


@pytest.mark.parametrize("T", [1, 5, 33, 200])
@pytest.mark.parametrize("top_k", [1, 4, 8])
def test_moe_prefill_small_layers(T, top_k):
    d = synth.moe_prefill_layer(seed=T * 10 + top_k, T=T, n_experts=16, hidden=256, inter=128)
    ids, wts = _route(d["logits"], top_k)
    out = _run(d, ids, wts)
    ref, a = _expect(d, ids, wts)
    _check_rows(out, ref, a, range(T), "T=%d k=%d" % (T, top_k))


@pytest.mark.parametrize("out_dt,residual", [("f32", True), ("f32", False), ("bf16", False)])
def test_moe_prefill_dtypes_and_no_residual(out_dt, residual):
    d = synth.moe_prefill_layer(seed=77, T=40, n_experts=8, hidden=512, inter=192)
    ids, wts = _route(d["logits"], 4)
    out = _run(d, ids, wts, out_dt=out_dt, residual=residual, ldx=512 + 32)
    ref, a = _expect(d, ids, wts, residual=residual, out_dt=out_dt)
    if out_dt == "f32":
        check(out, ref, a, "f32 out")
    else:
        _check_rows(out, ref, a, range(40), "bf16 no residual")


def test_moe_prefill_skewed_routing_and_invalid_ids():
    """All tokens on few experts (several row tiles per expert, a 128-row tile height),
    with some ids out of range (those slots contribute nothing)."""
    T, k = 300, 2
    d = synth.moe_prefill_layer(seed=5, T=T, n_experts=6, hidden=256, inter=128)
    rng = np.random.default_rng(5)
    ids = rng.choice([0, 1, 1, 1, 4], size=(T, k))
    ids[::7, 1] = 6          # == n_experts
    ids[::11, 0] = 1 << 30   # far out of range
    wts = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    out = _run(d, ids, wts)
    ref, a = _expect(d, ids, wts)
    _check_rows(out, ref, a, range(T), "skewed")


def test_moe_prefill_one_expert_and_many_experts():
    """E = 1 (every pair in one segment) and E = 1000 with few tokens (mostly 1-row tiles)."""
    d = synth.moe_prefill_layer(seed=8, T=70, n_experts=1, hidden=128, inter=64)
    ids = np.zeros((70, 1), np.int64)
    wts = np.full((70, 1), 0.75, np.float32)
    out = _run(d, ids, wts)
    ref, a = _expect(d, ids, wts)
    _check_rows(out, ref, a, range(70), "E=1")
    d = synth.moe_prefill_layer(seed=9, T=12, n_experts=1000, hidden=128, inter=64)
    ids, wts = _route(d["logits"], 8)
    out = _run(d, ids, wts)
    ref, a = _expect(d, ids, wts)
    _check_rows(out, ref, a, range(12), "E=1000")


def test_moe_prefill_fed_by_device_router():
    """moe_router_topk output used directly (no host round trip)."""
    q = lib()
    T = 48
    d = synth.moe_prefill_layer(seed=10, T=T, n_experts=32, hidden=256, inter=128)
    logits = torch.tensor(d["logits"], device="cuda")
    ids = torch.empty((T, 8), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, 8), dtype=torch.float32, device="cuda")
    q.moe_router_topk(logits, 8, ids, wts)
    gate, up, down = (dev_matrix(d[k]) for k in ("gate", "up", "down"))
    x = synth.to_torch(d["x"], "bf16")
    res = synth.to_torch(d["residual"], "bf16")
    out = nan_like((T, 256), torch.bfloat16)
    ws = torch.empty(q.moe_prefill_qgemm_int4_workspace_bytes(T, 8, 32, 256, 128), dtype=torch.uint8,
                     device="cuda")
    q.moe_prefill_qgemm_int4(gate, up, down, x, ids, wts, out, ws, residual=res)
    torch.cuda.synchronize()
    ref_ids, _ = _route(d["logits"], 8)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ref, a = _expect(d, ref_ids, wts.cpu().numpy())
    _check_rows(out, ref, a, range(T), "router-fed")


@pytest.mark.parametrize("T", [256, 1024, 4096])
def test_moe_prefill_full_layer(T):
    """128 experts, hidden 2048, inter 768, top-8 at the measured prefill lengths (32/64/128-row
    tiles): every output of every token against the oracle."""
    d = synth.moe_prefill_layer(seed=6, T=T)
    ids, wts = _route(d["logits"], 8)
    out = _run(d, ids, wts)
    ref, a = _expect(d, ids, wts)
    check(out, ref, a, "full layer T=%d" % T)
