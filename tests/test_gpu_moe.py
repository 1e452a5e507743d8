"""GPU parity of moe_gather_qgemv_int4 against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import check, dev_matrix, lib, nan_like, oracle_threads, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _run(d, ids, wts, residual, act="bf16", tok=0):
    q = lib()
    gate, up, down = (dev_matrix(d[k]) for k in ("gate", "up", "down"))
    hidden, inter = d["gate"].k_in, d["gate"].n_out
    x = synth.to_torch(d["x"][tok], act)
    res = None if residual is None else synth.to_torch(residual, act)
    ids_t = torch.tensor(np.asarray(ids, dtype=np.int64).astype(np.uint32).view(np.int32),
                         device="cuda")
    wts_t = torch.tensor(np.asarray(wts, dtype=np.float32), device="cuda")
    ws = torch.empty(q.moe_gather_qgemv_int4_workspace_bytes(down, len(ids)), dtype=torch.uint8,
                     device="cuda")
    out = nan_like(hidden, torch.bfloat16 if act == "bf16" else torch.float32)
    q.moe_gather_qgemv_int4(gate, up, down, x, ids_t, wts_t, out, ws, residual=res)
    torch.cuda.synchronize()
    return out


def test_moe_decode_workload():
    """128 experts, hidden 2048, inter 768, top-8 from softmax router, residual add."""
    d = synth.moe_layer()
    ids, wts = oracle.router_topk(d["logits"][0], 8)
    wts32 = wts.astype(np.float32)
    out = _run(d, ids, wts32, d["residual"][0])
    ref, a_ref = oracle.moe(d["gate"], d["up"], d["down"], d["x"][0], ids, wts32,
                            d["residual"][0], "bf16", threads=oracle_threads())
    rel = check(out, ref, a_ref, "moe top-8")
    print("moe max rel %.3e ids %s" % (rel, ids.tolist()))


@pytest.mark.parametrize("top_k", [1, 3, 8])
@pytest.mark.parametrize("with_residual", [True, False])
def test_moe_small_topk_variants(top_k, with_residual):
    d = synth.moe_layer(seed=40 + top_k, n_experts=16, hidden=512, inter=256, group_size=64)
    ids, wts = oracle.router_topk(d["logits"][0], top_k)
    wts32 = wts.astype(np.float32)
    res = d["residual"][0] if with_residual else None
    out = _run(d, ids, wts32, res)
    ref, a_ref = oracle.moe(d["gate"], d["up"], d["down"], d["x"][0], ids, wts32, res, "bf16")
    check(out, ref, a_ref, "moe k=%d res=%s" % (top_k, with_residual))


def test_moe_float32_activations_group32():
    d = synth.moe_layer(seed=50, n_experts=8, hidden=256, inter=96, group_size=32)
    x32 = synth.bf16_bits_to_f32(d["x"][0])
    r32 = synth.bf16_bits_to_f32(d["residual"][0])
    d2 = dict(d)
    d2["x"] = x32[None, :]
    ids, wts = oracle.router_topk(d["logits"][0], 4)
    wts32 = wts.astype(np.float32)
    out = _run(d2, ids, wts32, r32, act="f32")
    ref, a_ref = oracle.moe(d["gate"], d["up"], d["down"], x32, ids, wts32, r32, "f32")
    check(out, ref, a_ref, "moe f32")


def test_moe_repeated_and_invalid_ids():
    """Duplicate ids accumulate twice; ids >= n_experts contribute nothing."""
    d = synth.moe_layer(seed=60, n_experts=8, hidden=512, inter=128, group_size=64)
    ids = [3, 3, 9, 0, 1000, 7]
    wts = np.array([0.25, 0.25, 0.5, 0.125, 0.5, 0.0625], np.float32)
    out = _run(d, ids, wts, d["residual"][0])
    ref, a_ref = oracle.moe(d["gate"], d["up"], d["down"], d["x"][0], ids, wts, d["residual"][0],
                            "bf16")
    check(out, ref, a_ref, "moe invalid ids")


def test_moe_expert_slab_selection_matches_single_gemv_path():
    """Expert 2 of a 4-expert stack, weight 1, no residual: equals the dense path on that slab."""
    q = lib()
    d = synth.moe_layer(seed=70, n_experts=4, hidden=1024, inter=256, group_size=64)
    out = _run(d, [2], np.array([1.0], np.float32), None)
    slab = {k: synth.QMatrix(codes=d[k].codes[2].copy(), scales=d[k].scales[2].copy(),
                             biases=d[k].biases[2].copy(), sb_dtype="bf16", group_size=64,
                             n_out=d[k].n_out, k_in=d[k].k_in) for k in ("gate", "up", "down")}
    x = synth.to_torch(d["x"][0], "bf16")
    h = nan_like(256, torch.float32)
    y = nan_like(1024, torch.bfloat16)
    q.qgemv_int4_multi([dev_matrix(slab["gate"]), dev_matrix(slab["up"])], x, [h],
                       epilogue=q.EPI_SWIGLU_PAIR)
    q.qgemv_int4(dev_matrix(slab["down"]), h, y)
    torch.cuda.synchronize()
    y_ref, a_y, _, _ = oracle.dense_ffn(slab["gate"], slab["up"], slab["down"], d["x"][0], "bf16")
    check(out, y_ref, a_y, "moe expert 2")
    check(y, y_ref, a_y, "dense on slab 2")
