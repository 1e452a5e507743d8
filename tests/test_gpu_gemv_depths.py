"""GPU parity of every GEMV ring form: one pass with depth 1, 2 and 4 (including a wave that
has fewer steps than its ring) and the streaming ring, for each launch that has them.

Each case asserts, through the library's host-only plan query for the device it runs on, the
form it was chosen for (tests/test_gemv_plan.py checks the same tables on the CPU for 256 CUs)."""
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


# (n_out, k_in, x dtype, ring depth, steps of the busiest wave)
GEMV_CASES = [
    (8, 2048, "bf16", 1, 1),
    (14000, 1024, "bf16", 2, 2),
    (28250, 1024, "bf16", 4, 4),
    (30000, 512, "bf16", 4, 3),
    (25000, 512, "bf16", 0, 5),
    (8, 1024, "f32", 1, 1),
    (16000, 1024, "f32", 2, 2),
    (27750, 1024, "f32", 4, 4),
]


@pytest.mark.parametrize("n_out,k_in,x_dt,depth,steps", GEMV_CASES)
def test_gemv_ring_forms(n_out, k_in, x_dt, depth, steps):
    q = lib()
    f = q.plan_qgemv([n_out], k_in, x_dtype=x_dt)
    assert (f["kernel"], f["ring_depth"], f["busiest_wave_steps"]) == ("ring", depth, steps)
    rng = np.random.default_rng(n_out + 7 * k_in)
    w = synth.draw_matrix(rng, n_out, k_in, 64, "bf16")
    x = synth.draw_activation(rng, (k_in,), x_dt)
    y = nan_like(n_out, torch.bfloat16)
    q.qgemv_int4(dev_matrix(w), synth.to_torch(x, x_dt), y)
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.gemv(w, x, x_dt, threads=oracle_threads())
    check(y, y_ref, a_ref, "gemv %dx%d %s depth %d" % (n_out, k_in, x_dt, depth))


# (T, n_out, k_in, ring depth, steps); k_in not a multiple of 512, so that the
# small-M call runs the GEMV rings rather than the MFMA form
SMALLM_CASES = [
    (2, 64, 256, 1, 1),
    (2, 8, 2304, 2, 2),
    (4, 2000, 2304, 4, 3),
    (4, 5000, 2304, 0, 9),
]


@pytest.mark.parametrize("T,n_out,k_in,depth,steps", SMALLM_CASES)
def test_smallm_ring_forms(T, n_out, k_in, depth, steps):
    q = lib()
    f = q.plan_qgemv([n_out], k_in, T=T, call=q.CALL_SMALLM)
    assert (f["kernel"], f["ring_depth"], f["busiest_wave_steps"]) == ("ring", depth, steps)
    rng = np.random.default_rng(T * 1000 + n_out)
    w = synth.draw_matrix(rng, n_out, k_in, 64, "bf16")
    x = synth.draw_activation(rng, (T, k_in), "bf16")
    y = torch.full((T, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    q.qgemv_int4_smallm([dev_matrix(w)], synth.to_torch(x, "bf16"), [y])
    torch.cuda.synchronize()
    for t in range(T):
        ref, a = oracle.gemv(w, x[t], "bf16", threads=oracle_threads())
        check(y[t], ref, a, "smallm T=%d t=%d depth %d" % (T, t, depth))


# (n_out, k_in, ring depth, steps): the gate/up pair, two code streams per row
SWIGLU_CASES = [
    (8, 2048, 1, 1),
    (8000, 2048, 2, 2),
    (500, 2112, 4, 3),
    (2000, 1280, 0, 5),
]


@pytest.mark.parametrize("n_out,k_in,depth,steps", SWIGLU_CASES)
def test_swiglu_ring_forms(n_out, k_in, depth, steps):
    q = lib()
    f = q.plan_qgemv([n_out, n_out], k_in, epilogue=q.EPI_SWIGLU_PAIR)
    assert (f["kernel"], f["ring_depth"], f["busiest_wave_steps"]) == ("ring", depth, steps)
    rng = np.random.default_rng(n_out * 3 + k_in)
    gate = synth.draw_matrix(rng, n_out, k_in, 64, "bf16")
    up = synth.draw_matrix(rng, n_out, k_in, 64, "bf16")
    x = synth.draw_activation(rng, (k_in,), "bf16")
    h = nan_like(n_out, torch.bfloat16)
    q.qgemv_int4_multi([dev_matrix(gate), dev_matrix(up)], synth.to_torch(x, "bf16"), [h],
                       epilogue=q.EPI_SWIGLU_PAIR)
    torch.cuda.synchronize()
    h_ref, a_h = oracle.swiglu_pair(gate, up, x, "bf16")
    check(h, h_ref, a_h, "swiglu %dx%d depth %d" % (n_out, k_in, depth))


# (hidden, inter, top_k, residual, gate/up depth, down depth)
MOE_CASES = [
    (256, 64, 1, True, 1, 1),
    (256, 512, 3, True, 1, 2),
    (256, 96, 1, True, 1, 4),
    (256, 96, 3, True, 1, 0),
    (2048, 1024, 8, True, 2, 4),
    (2048, 2048, 8, False, 0, 0),
]


@pytest.mark.parametrize("hidden,inter,top_k,residual,d_gu,d_down", MOE_CASES)
def test_moe_ring_forms(hidden, inter, top_k, residual, d_gu, d_down):
    q = lib()
    gu, dn = q.plan_moe_gather(hidden, inter, top_k, group_size=64 if inter % 64 == 0 else 32,
                               residual=residual)
    assert (gu["ring_depth"], dn["ring_depth"]) == (d_gu, d_down)
    d = synth.moe_layer(seed=hidden + inter + top_k, n_experts=16, hidden=hidden, inter=inter,
                        group_size=64 if inter % 64 == 0 else 32)
    ids, wts = oracle.router_topk(d["logits"][0], top_k)
    wts32 = wts.astype(np.float32)
    res = d["residual"][0] if residual else None
    gate, up, down = (dev_matrix(d[k]) for k in ("gate", "up", "down"))
    x = synth.to_torch(d["x"][0], "bf16")
    ids_t = torch.tensor(np.asarray(ids, dtype=np.int64).astype(np.int32), device="cuda")
    wts_t = torch.tensor(wts32, device="cuda")
    ws = torch.empty(q.moe_gather_qgemv_int4_workspace_bytes(down, top_k), dtype=torch.uint8,
                     device="cuda")
    out = nan_like(hidden, torch.bfloat16)
    q.moe_gather_qgemv_int4(gate, up, down, x, ids_t, wts_t, out, ws,
                            residual=None if res is None else synth.to_torch(res, "bf16"))
    torch.cuda.synchronize()
    ref, a_ref = oracle.moe(d["gate"], d["up"], d["down"], d["x"][0], ids, wts32, res, "bf16",
                            threads=oracle_threads())
    check(out, ref, a_ref, "moe h%d i%d k%d depths %d/%d" % (hidden, inter, top_k, d_gu, d_down))
