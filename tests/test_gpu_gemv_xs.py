"""GPU parity of the activation-stationary GEMV form (qgemv_int4 on one matrix, float32 or bf16
activations, qgemv_int4_multi on the gate/up pair; k_in from 4096 to 32768, at least 2^25 codes)
against the fp64 oracle, through the C ABI.  Each case first asserts, through the library's plan
query, that the call takes that form, so the edges below stay on it: rows not a multiple of the
grid, fewer rows than workgroups (one row each), a last wave with few lanes holding a chunk, 32
and 64 lanes a row, sixteen waves, one and two workgroups per CU, and 256 rows per workgroup."""
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


def _run_single(w, x, x_dt, y_dt):
    q = lib()
    f = q.plan_qgemv([w.n_out], w.k_in, group_size=w.group_size, x_dtype=x_dt)
    assert f["kernel"] == "xs", f
    y = nan_like(w.n_out, TD[y_dt])
    q.qgemv_int4(dev_matrix(w), synth.to_torch(x, x_dt), y)
    torch.cuda.synchronize()
    return y, f


# (n_out, k_in, group size): 5000 rows, 19 or 20 per workgroup, 32 lanes a row; 8320 = 260
# chunks, the ninth wave holding 4 per row group; 16384 / g128, 16 waves of 32 lanes; 17408 (the
# dense down projection), 64 lanes a row; 32768, 16 waves of 64 lanes; 5120 columns, five waves,
# two workgroups per CU; 2048 columns, two waves, four workgroups per CU
SINGLE = [(5000, 8192, 64), (4100, 8320, 32), (2100, 16384, 128), (2000, 17408, 64), (2049, 32768, 64),
          (7001, 5120, 64), (12801, 2048, 64)]


@pytest.mark.parametrize("n_out,k_in,g", SINGLE)
@pytest.mark.parametrize("sb_dt,y_dt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("x_dt", ["f32", "bf16"])
def test_xs_single_shapes_and_dtypes(n_out, k_in, g, sb_dt, y_dt, x_dt):
    rng = np.random.default_rng(n_out * 17 + k_in + g)
    w = synth.draw_matrix(rng, n_out, k_in, g, sb_dt)
    x = synth.draw_activation(rng, (k_in,), x_dt)
    y, f = _run_single(w, x, x_dt, y_dt)
    if k_in == 5120:
        assert f["grid"] == 2 * _n_cu()
    y_ref, a_ref = oracle.gemv(w, x, x_dt, threads=oracle_threads())
    check(y, y_ref, a_ref, "xs gemv %dx%d g%d x %s, %s/%s (grid %d, %d waves of %d lanes)" %
          (n_out, k_in, g, x_dt, sb_dt, y_dt, f["grid"], f["waves"], f["lanes"]))


def test_xs_most_rows_per_workgroup():
    """256 rows per workgroup (the form's limit) on an 8320-wide matrix (nine waves, one
    workgroup per CU)."""
    n_out = 256 * _n_cu()
    rng = np.random.default_rng(4242)
    w = synth.draw_matrix(rng, n_out, 8320, 64, "bf16")
    x = synth.draw_activation(rng, (8320,), "f32")
    y, f = _run_single(w, x, "f32", "f32")
    assert f["busiest_wave_steps"] == 256 and f["grid"] == _n_cu()
    y_ref, a_ref = oracle.gemv(w, x, "f32", threads=oracle_threads())
    check(y, y_ref, a_ref, "xs gemv %dx8320 (256 rows per workgroup)" % n_out)


def test_xs_grid_grows_past_256_rows_per_workgroup():
    """A matrix whose rows would give a workgroup more than 256 at two per CU (an LM-head-like
    2 * 256 * n_cu + 1 rows over 5120 columns): the grid grows to keep every workgroup at 256 or
    fewer.  Every 61st row, and the last rows, against the oracle on those rows."""
    q = lib()
    n_out, k_in = 2 * 256 * _n_cu() + 1, 5120
    f = q.plan_qgemv([n_out], k_in, x_dtype="bf16")
    assert f["kernel"] == "xs" and f["grid"] == -(-n_out // 256) and f["busiest_wave_steps"] <= 256, f
    rng = np.random.default_rng(515)
    w = synth.draw_matrix(rng, n_out, k_in, 64, "bf16")
    x = synth.draw_activation(rng, (k_in,), "bf16")
    y = nan_like(n_out, torch.float32)
    q.qgemv_int4(dev_matrix(w), synth.to_torch(x, "bf16"), y)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, n_out, 61), np.arange(n_out - 300, n_out)]))
    sub = synth.QMatrix(codes=w.codes[rows], scales=w.scales[rows], biases=w.biases[rows],
                        sb_dtype="bf16", group_size=64, n_out=len(rows), k_in=k_in)
    y_ref, a_ref = oracle.gemv(sub, x, "bf16", threads=oracle_threads())
    check(y[torch.from_numpy(rows).cuda()], y_ref, a_ref,
          "xs gemv %dx%d (grid %d), %d sampled rows" % (n_out, k_in, f["grid"], len(rows)))


@pytest.mark.parametrize("lo,hi", [(-100, -60), (-20, 100)])
def test_xs_float32_activation_range(lo, hi):
    """Float32 activations across the exponent range the scaled form keeps exact (codes as f16
    subnormals times activations scaled by 2^24 / 2^20): each 32-value chunk in its own binade
    between 2^lo and 2^hi (products stay normal floats), against the oracle."""
    n_out, k_in = 2048, 16384
    rng = np.random.default_rng(99 + hi)
    w = synth.draw_matrix(rng, n_out, k_in, 64, "f32")
    x = synth.draw_activation(rng, (k_in,), "f32")
    binade = np.repeat(rng.integers(lo, hi + 1, size=k_in // 32), 32).astype(np.float64)
    x = (x.astype(np.float64) * np.exp2(binade)).astype(np.float32)
    y, f = _run_single(w, x, "f32", "f32")
    y_ref, a_ref = oracle.gemv(w, x, "f32", threads=oracle_threads())
    check(y, y_ref, a_ref, "xs gemv %dx%d, activations from 2^%d to 2^%d" % (n_out, k_in, lo, hi))


# matrices sharing x with stored outputs, each with its own workgroups: q/k/v of a 5120
# activation; three odd sizes (37 rows: one workgroup); eight matrices over 4608 columns (five
# waves, the last half full); single matrices at the threshold (5120 x 5120 codes)
MULTI = [([5120, 1024, 1024], 5120), ([3001, 37, 1499], 8192), ([800] * 8, 4608), ([5120], 5120),
         ([2560], 10240)]


@pytest.mark.parametrize("n_outs,k_in", MULTI)
@pytest.mark.parametrize("x_dt,sb_dt,y_dt", [("bf16", "bf16", "bf16"), ("bf16", "f32", "f32"),
                                             ("f32", "bf16", "f32")])
def test_xs_multi(n_outs, k_in, x_dt, sb_dt, y_dt):
    q = lib()
    f = q.plan_qgemv(n_outs, k_in, x_dtype=x_dt)
    assert f["kernel"] == "xs", f
    rng = np.random.default_rng(sum(n_outs) + k_in + len(n_outs))
    ws = [synth.draw_matrix(rng, n, k_in, 64, sb_dt) for n in n_outs]
    x = synth.draw_activation(rng, (k_in,), x_dt)
    ys = [nan_like(n, TD[y_dt]) for n in n_outs]
    q.qgemv_int4_multi([dev_matrix(w) for w in ws], synth.to_torch(x, x_dt), ys)
    torch.cuda.synchronize()
    for i, (w, y) in enumerate(zip(ws, ys)):
        y_ref, a_ref = oracle.gemv(w, x, x_dt, threads=oracle_threads())
        check(y, y_ref, a_ref, "xs multi %s x %d, matrix %d, x %s %s/%s (grid %d)" %
              (n_outs, k_in, i, x_dt, sb_dt, y_dt, f["grid"]))


# (n_out, k_in, x dtype): the dense FFN gate/up pair 17408 x 5120 (three workgroups per CU);
# 6144 and 8192 columns (two per CU), 5 or 6 and 4 or 5 rows per workgroup; 1000 rows over 32768
# columns (16 waves of 64 lanes, one workgroup per CU); float32 activations over 17408 columns;
# 2048 and 3072 columns (two and three waves, four workgroups per CU)
PAIRS = [(17408, 5120, "bf16"), (3000, 6144, "bf16"), (2100, 8192, "bf16"), (1000, 32768, "bf16"),
         (2048, 17408, "f32"), (8192, 2048, "bf16"), (6000, 3072, "f32")]


@pytest.mark.parametrize("n_out,k_in,x_dt", PAIRS)
@pytest.mark.parametrize("sb_dt,h_dt", [("bf16", "f32"), ("f32", "bf16")])
def test_xs_gate_up_pair(n_out, k_in, x_dt, sb_dt, h_dt):
    q = lib()
    f = q.plan_qgemv([n_out, n_out], k_in, x_dtype=x_dt, epilogue=q.EPI_SWIGLU_PAIR)
    assert f["kernel"] == "xs", f
    rng = np.random.default_rng(n_out * 5 + k_in)
    gate = synth.draw_matrix(rng, n_out, k_in, 64, sb_dt)
    up = synth.draw_matrix(rng, n_out, k_in, 64, sb_dt)
    x = synth.draw_activation(rng, (k_in,), x_dt)
    h = nan_like(n_out, TD[h_dt])
    q.qgemv_int4_multi([dev_matrix(gate), dev_matrix(up)], synth.to_torch(x, x_dt), [h],
                       epilogue=q.EPI_SWIGLU_PAIR)
    torch.cuda.synchronize()
    h_ref, a_ref = oracle.swiglu_pair(gate, up, x, x_dt, threads=oracle_threads())
    check(h, h_ref, a_ref, "xs gate/up pair %dx%d %s %s/%s (grid %d, %d waves of %d lanes)" %
          (n_out, k_in, x_dt, sb_dt, h_dt, f["grid"], f["waves"], f["lanes"]))


def test_xs_unpack_identity_probe():
    """s = 1, b = 0 and x = e_k for k at the start, middle and end of the waves' slices: y[o]
    equals code k of row o exactly."""
    q = lib()
    rng = np.random.default_rng(31)
    n_out, k_in = 4100, 8320
    raw = rng.integers(0, 16, size=(n_out, k_in), dtype=np.uint8)
    groups = k_in // 64
    w = synth.QMatrix(codes=synth.pack_codes(raw), scales=np.ones((n_out, groups), np.float32),
                      biases=np.zeros((n_out, groups), np.float32), sb_dtype="f32", group_size=64,
                      n_out=n_out, k_in=k_in)
    dw = dev_matrix(w)
    for x_dt in ("f32", "bf16"):
        assert q.plan_qgemv([n_out], k_in, x_dtype=x_dt)["kernel"] == "xs"
        for k in (0, 1, 2, 3, 4, 5, 6, 7, 31, 32, 1023, 1024, 1025, 4095, 4096, 8191, 8192, 8287, 8288, 8319):
            x = np.zeros(k_in, np.float32)
            x[k] = 1.0
            y = nan_like(n_out, torch.float32)
            q.qgemv_int4(dw, synth.to_torch(x if x_dt == "f32" else synth.f32_to_bf16_bits(x), x_dt), y)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy().astype(np.float64), raw[:, k].astype(np.float64)), (x_dt, k)


def test_xs_pair_repeatable():
    """The gate/up pair (a block of rows per workgroup, some workgroups without rows): two calls
    on the same inputs give the same bits."""
    q = lib()
    rng = np.random.default_rng(78)
    n_out, k_in = 17408, 5120
    f = q.plan_qgemv([n_out, n_out], k_in, epilogue=q.EPI_SWIGLU_PAIR)
    assert f["kernel"] == "xs" and -(-n_out // f["busiest_wave_steps"]) < f["grid"], f
    gate = dev_matrix(synth.draw_matrix(rng, n_out, k_in, 64, "bf16"))
    up = dev_matrix(synth.draw_matrix(rng, n_out, k_in, 64, "bf16"))
    x = synth.to_torch(synth.draw_activation(rng, (k_in,), "bf16"), "bf16")
    h1 = nan_like(n_out, torch.float32)
    h2 = nan_like(n_out, torch.float32)
    q.qgemv_int4_multi([gate, up], x, [h1], epilogue=q.EPI_SWIGLU_PAIR)
    q.qgemv_int4_multi([gate, up], x, [h2], epilogue=q.EPI_SWIGLU_PAIR)
    torch.cuda.synchronize()
    assert torch.isfinite(h1).all() and torch.equal(h1, h2)


def test_xs_repeatable():
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
