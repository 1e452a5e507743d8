"""GPU parity of qgemv_int4 and qgemv_int4_multi against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import (check, check_f32, dev_matrix, lib, nan_like, oracle_threads, require_gpu,
                              to_np64)

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def _run_gemv(w, x_np, x_dt, y_dt):
    q = lib()
    dw = dev_matrix(w)
    x = synth.to_torch(x_np, x_dt)
    y = nan_like(w.n_out, TD[y_dt])
    q.qgemv_int4(dw, x, y)
    torch.cuda.synchronize()
    return y


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def test_single_gemv_workload_fp32():
    """1024x1024, g64, fp32 scales/biases, fp32 x and y (seed 0)."""
    d = synth.single_gemv()
    y = _run_gemv(d["w"], d["x"], "f32", "f32")
    y_ref, a_ref = oracle.gemv(d["w"], d["x"], "f32", threads=oracle_threads())
    err = check(y, y_ref, a_ref, "single gemv")
    print("single gemv rel L2 %.3e" % err)


@pytest.mark.parametrize("n_out,k_in,g", [(1, 64, 64), (7, 96, 32), (64, 256, 64), (100, 1024, 128),
                                          (33, 768, 64), (257, 5120, 64), (130, 2048, 32),
                                          (50, 17408, 64), (9, 160, 32)])
@pytest.mark.parametrize("x_dt,sb_dt,y_dt", [("f32", "f32", "f32"), ("bf16", "bf16", "bf16"),
                                             ("bf16", "f32", "f32"), ("f32", "bf16", "bf16")])
def test_gemv_shapes_and_dtypes(n_out, k_in, g, x_dt, sb_dt, y_dt):
    rng = np.random.default_rng(n_out * 131 + k_in + g)
    w = synth.draw_matrix(rng, n_out, k_in, g, sb_dt)
    x = synth.draw_activation(rng, (k_in,), x_dt)
    y = _run_gemv(w, x, x_dt, y_dt)
    y_ref, a_ref = oracle.gemv(w, x, x_dt)
    check(y, y_ref, a_ref, "gemv %dx%d g%d %s/%s/%s" % (n_out, k_in, g, x_dt, sb_dt, y_dt))


@pytest.mark.parametrize("x_dt", ["f32", "bf16"])
def test_unpack_bit_exact_identity_probe(x_dt):
    """s = 1, b = 0, x = e_k: y[o] equals code k of row o exactly, for every k."""
    q = lib()
    rng = np.random.default_rng(17)
    n_out, k_in = 96, 256
    raw = rng.integers(0, 16, size=(n_out, k_in), dtype=np.uint8)
    ones = np.ones((n_out, k_in // 64), np.float32)
    zeros = np.zeros((n_out, k_in // 64), np.float32)
    sb_dt = "f32" if x_dt == "f32" else "bf16"
    conv = (lambda a: a) if sb_dt == "f32" else synth.f32_to_bf16_bits
    w = synth.QMatrix(codes=synth.pack_codes(raw), scales=conv(ones), biases=conv(zeros),
                      sb_dtype=sb_dt, group_size=64, n_out=n_out, k_in=k_in)
    dw = dev_matrix(w)
    eye = np.eye(k_in, dtype=np.float32)
    xs = synth.to_torch(eye if x_dt == "f32" else synth.f32_to_bf16_bits(eye), x_dt)
    got = np.empty((k_in, n_out), np.float64)
    for k in range(k_in):
        y = nan_like(n_out, torch.float32)
        q.qgemv_int4(dw, xs[k].contiguous(), y)
        got[k] = to_np64(y)
    torch.cuda.synchronize()
    assert np.array_equal(got.T, raw.astype(np.float64))


def test_determinism_and_power_of_two_scaling():
    q = lib()
    rng = np.random.default_rng(23)
    w = synth.draw_matrix(rng, 512, 4096, 64, "bf16")
    x = synth.draw_activation(rng, (4096,), "f32")
    dw = dev_matrix(w)
    xt = synth.to_torch(x, "f32")
    y1 = nan_like(512, torch.float32)
    y2 = nan_like(512, torch.float32)
    y3 = nan_like(512, torch.float32)
    q.qgemv_int4(dw, xt, y1)
    q.qgemv_int4(dw, xt, y2)
    q.qgemv_int4(dw, (2 * xt).contiguous(), y3)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y3, 2 * y1)


def test_qkv_multi_workload():
    """q/k/v projections of one bf16 input in one launch (4096 -> 4096/1024/1024)."""
    q = lib()
    d = synth.qkv_multi()
    dws = [dev_matrix(w) for w in d["ws"]]
    x = synth.to_torch(d["x"], "bf16")
    ys = [nan_like(w.n_out, torch.bfloat16) for w in d["ws"]]
    q.qgemv_int4_multi(dws, x, ys)
    torch.cuda.synchronize()
    refs = oracle.multi(d["ws"], d["x"], "bf16", threads=oracle_threads())
    for name, y, (y_ref, a_ref) in zip("qkv", ys, refs):
        rel = check(y, y_ref, a_ref, "qkv " + name)
        print("qkv %s max rel %.3e" % (name, rel))


def test_multi_ragged_rows_many_matrices():
    """Eight matrices with ragged row counts share one input."""
    q = lib()
    rng = np.random.default_rng(29)
    outs = [1, 7, 64, 33, 128, 5, 250, 16]
    ws = [synth.draw_matrix(rng, n, 512, 64, "bf16") for n in outs]
    x = synth.draw_activation(rng, (512,), "bf16")
    ys = [nan_like(n, torch.float32) for n in outs]
    q.qgemv_int4_multi([dev_matrix(w) for w in ws], synth.to_torch(x, "bf16"), ys)
    torch.cuda.synchronize()
    for i, (w, y) in enumerate(zip(ws, ys)):
        y_ref, a_ref = oracle.gemv(w, x, "bf16")
        check(y, y_ref, a_ref, "multi[%d]" % i)


@pytest.mark.parametrize("h_dt", ["f32", "bf16"])
def test_swiglu_pair_small(h_dt):
    q = lib()
    rng = np.random.default_rng(31)
    gate = synth.draw_matrix(rng, 200, 640, 64, "bf16")
    up = synth.draw_matrix(rng, 200, 640, 64, "bf16")
    x = synth.draw_activation(rng, (640,), "bf16")
    h = nan_like(200, TD[h_dt])
    q.qgemv_int4_multi([dev_matrix(gate), dev_matrix(up)], synth.to_torch(x, "bf16"), [h],
                       epilogue=q.EPI_SWIGLU_PAIR)
    torch.cuda.synchronize()
    h_ref, a_h = oracle.swiglu_pair(gate, up, x, "bf16")
    if h_dt == "f32":
        # h is a float32 SwiGLU of float32 sums: bound by the propagated accumulation noise
        got = to_np64(h)
        check_f32(got, h_ref, "swiglu pair h", a_ref=a_h)
    else:
        check(h, h_ref, a_h, "swiglu bf16")


def test_dense_layer_workload():
    """Gate/up 5120->17408 with SwiGLU (fp32 h), then down 17408->5120 (bf16 y)."""
    q = lib()
    d = synth.dense_layer()
    gate, up, down = (dev_matrix(d[k]) for k in ("gate", "up", "down"))
    x = synth.to_torch(d["x"], "bf16")
    h = nan_like(d["gate"].n_out, torch.float32)
    y = nan_like(d["down"].n_out, torch.bfloat16)
    q.qgemv_int4_multi([gate, up], x, [h], epilogue=q.EPI_SWIGLU_PAIR)
    q.qgemv_int4(down, h, y)
    torch.cuda.synchronize()
    y_ref, a_y, h_ref, a_h = oracle.dense_ffn(d["gate"], d["up"], d["down"], d["x"], "bf16",
                                              threads=oracle_threads())
    got_h = to_np64(h)
    check_f32(got_h, h_ref, "dense h (fp32 SwiGLU)", a_ref=a_h)
    rel = check(y, y_ref, a_y, "dense down")
    print("dense layer max rel %.3e" % rel)
