"""GPU parity of the activation-stationary GEMV form (float32 activations, one matrix, k_in from
4096 to 32768) against the fp64 oracle, through the C ABI.  Each case first asserts, through the
library's plan query, that the call takes that form, so the edges below stay on it: fewer rows
than CUs (one row per workgroup), rows not a multiple of the grid, a last wave with only a few
lanes holding a chunk, sixteen waves, and 256 rows per workgroup."""
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


def _n_cu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _run(w, x, y_dt):
    q = lib()
    f = q.plan_qgemv([w.n_out], w.k_in, group_size=w.group_size, x_dtype="f32")
    assert f["kernel"] == "xs", f
    y = nan_like(w.n_out, TD[y_dt])
    q.qgemv_int4(dev_matrix(w), synth.to_torch(x, "f32"), y)
    torch.cuda.synchronize()
    return y, f


# (n_out, k_in, group size): 100 rows < CUs; 333 rows, 1-2 per workgroup; 4160 = 130 chunks, the
# third wave holding 2; 6144 / g128; 17408 (the dense down projection) with ragged rows;
# 32768 = 16 waves
SHAPES = [(100, 6144, 128), (333, 4096, 32), (5000, 4160, 64), (1000, 17408, 64), (257, 32768, 64)]


@pytest.mark.parametrize("n_out,k_in,g", SHAPES)
@pytest.mark.parametrize("sb_dt,y_dt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
def test_xs_shapes_and_dtypes(n_out, k_in, g, sb_dt, y_dt):
    rng = np.random.default_rng(n_out * 17 + k_in + g)
    w = synth.draw_matrix(rng, n_out, k_in, g, sb_dt)
    x = synth.draw_activation(rng, (k_in,), "f32")
    y, f = _run(w, x, y_dt)
    y_ref, a_ref = oracle.gemv(w, x, "f32", threads=oracle_threads())
    check(y, y_ref, a_ref, "xs gemv %dx%d g%d %s/%s (grid %d, %d waves)" %
          (n_out, k_in, g, sb_dt, y_dt, f["grid"], f["waves"]))


def test_xs_most_rows_per_workgroup():
    """256 rows per workgroup (the form's limit) on a 4096-wide matrix."""
    n_out = 256 * _n_cu()
    rng = np.random.default_rng(4242)
    w = synth.draw_matrix(rng, n_out, 4096, 64, "bf16")
    x = synth.draw_activation(rng, (4096,), "f32")
    y, f = _run(w, x, "f32")
    assert f["busiest_wave_steps"] == 256
    y_ref, a_ref = oracle.gemv(w, x, "f32", threads=oracle_threads())
    check(y, y_ref, a_ref, "xs gemv %dx4096 (256 rows per workgroup)" % n_out)


def test_xs_unpack_identity_probe():
    """s = 1, b = 0 and x = e_k for k at the start, middle and end of every wave's slice: y[o]
    equals code k of row o exactly."""
    q = lib()
    rng = np.random.default_rng(31)
    n_out, k_in = 300, 4160
    raw = rng.integers(0, 16, size=(n_out, k_in), dtype=np.uint8)
    groups = k_in // 64
    w = synth.QMatrix(codes=synth.pack_codes(raw), scales=np.ones((n_out, groups), np.float32),
                      biases=np.zeros((n_out, groups), np.float32), sb_dtype="f32", group_size=64,
                      n_out=n_out, k_in=k_in)
    dw = dev_matrix(w)
    assert q.plan_qgemv([n_out], k_in, x_dtype="f32")["kernel"] == "xs"
    for k in (0, 1, 7, 31, 32, 2047, 2048, 2049, 4095, 4096, 4127, 4128, 4159):
        x = np.zeros(k_in, np.float32)
        x[k] = 1.0
        y = nan_like(n_out, torch.float32)
        q.qgemv_int4(dw, synth.to_torch(x, "f32"), y)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().astype(np.float64), raw[:, k].astype(np.float64)), k


def test_xs_repeatable_and_matches_itself_across_calls():
    """Two calls on the same inputs give the same bits (fixed reduction order)."""
    q = lib()
    rng = np.random.default_rng(77)
    w = synth.draw_matrix(rng, 5120, 17408, 64, "bf16")
    x = synth.draw_activation(rng, (17408,), "f32")
    dw = dev_matrix(w)
    xt = synth.to_torch(x, "f32")
    y1 = nan_like(5120, torch.float32)
    y2 = nan_like(5120, torch.float32)
    q.qgemv_int4(dw, xt, y1)
    q.qgemv_int4(dw, xt, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
