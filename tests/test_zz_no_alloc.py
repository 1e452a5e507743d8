"""moe_gather_qgemv_int4_noalloc (the library's static per-device scratch instead of a
caller workspace) against moe_gather_qgemv_int4 through the C ABI: bit-identical outputs
on two calls in a row, the second with a smaller input (fewer experts kept, a narrower
expert), and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from tests.gpu_common import dev_matrix, lib, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _layer(seed, E, hidden, inter):
    m = synth.moe_layer(seed=seed, n_experts=E, hidden=hidden, inter=inter)
    return m, [dev_matrix(m[k]) for k in ("gate", "up", "down")]


def _both(q, mats, m, ids, wts, hidden, residual=True):
    x = synth.to_torch(m["x"][0], "bf16")
    res = synth.to_torch(m["residual"][0], "bf16") if residual else None
    ids_d = torch.tensor(ids, dtype=torch.int32, device="cuda")
    wts_d = torch.tensor(wts, dtype=torch.float32, device="cuda")
    out_ws = torch.full((hidden,), float("nan"), dtype=torch.bfloat16, device="cuda")
    out_na = torch.full((hidden,), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(q.moe_gather_qgemv_int4_workspace_bytes(mats[2], len(ids)), dtype=torch.uint8,
                     device="cuda")
    q.moe_gather_qgemv_int4(*mats, x, ids_d, wts_d, out_ws, ws, residual=res)
    q.moe_gather_qgemv_int4_noalloc(*mats, x, ids_d, wts_d, out_na, residual=res)
    torch.cuda.synchronize()
    return out_ws, out_na


def test_noalloc_matches_workspace_entry_two_calls():
    q = lib()
    # first call: top-8 of 128 experts, hidden 2048, inter 768 (the decode MoE shape)
    m1, mats1 = _layer(3, 128, 2048, 768)
    rng = np.random.default_rng(5)
    ids1 = rng.choice(128, size=8, replace=False)
    w1 = rng.uniform(0.05, 0.3, size=8).astype(np.float32)
    a, b = _both(q, mats1, m1, ids1, w1, 2048)
    assert not torch.isnan(a.float()).any()
    assert torch.equal(a, b)
    # second call, smaller: top-3 of 16 experts, hidden 512, inter 256, no residual;
    # the scratch still holds the first call's larger intermediates
    m2, mats2 = _layer(4, 16, 512, 256)
    ids2 = np.array([7, 2, 11])
    w2 = np.array([0.5, 0.3, 0.2], np.float32)
    a, b = _both(q, mats2, m2, ids2, w2, 512, residual=False)
    assert not torch.isnan(a.float()).any()
    assert torch.equal(a, b)


def test_noalloc_rejects_oversize():
    """top_k * inter * 4 above the scratch size: a status error, nothing launched."""
    q = lib()
    inter = q.NOALLOC_SCRATCH_BYTES // (4 * 8) + 32
    m, mats = _layer(6, 2, 256, 64)
    g, _, d = mats
    # descriptors with an inflated inter: validation rejects them before any launch
    gate = q.CMatrix(g.c().codes, g.c().scales, g.c().biases, inter, 256, 64, 2, 1, 0)
    assert gate.n_out == inter
    out = torch.empty(256, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(256, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(8, dtype=torch.int32, device="cuda")
    wts = torch.zeros(8, dtype=torch.float32, device="cuda")
    rc = q.load().moe_gather_qgemv_int4_noalloc(
        ctypes.byref(gate), ctypes.byref(gate), ctypes.byref(d.c()), x.data_ptr(), ids.data_ptr(),
        wts.data_ptr(), 8, None, out.data_ptr(), q.BF16, None)
    assert rc == 6, rc
    assert b"scratch" in q.load().qint4_last_error()
