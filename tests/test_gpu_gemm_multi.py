"""GPU parity of qgemm_int4_padT_multi (the prefill GEMM of several matrices that share
one activation block, one launch) against the fp64 oracle, through the C ABI.

Each output is compared with oracle.gemm of its own matrix (weights rounded once to
bf16); the kernel's float32 dequantisation step is covered by gemm_rounding_slack."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import (check_gemm, dev_matrix, gemm_rounding_slack, lib, oracle_threads,
                              require_gpu, to_np64)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _run(ws, X, y_dt=torch.bfloat16, ldys=None, fill=float("nan")):
    q = lib()
    T = X.shape[0]
    xs = synth.to_torch(X, "bf16")
    bufs = [torch.full((T, (ldys[i] if ldys else w.n_out)), fill, dtype=y_dt, device="cuda")
            for i, w in enumerate(ws)]
    ys = [b[:, :w.n_out] for b, w in zip(bufs, ws)]
    q.qgemm_int4_padT_multi([dev_matrix(w) for w in ws], xs, ys)
    torch.cuda.synchronize()
    return bufs


@pytest.mark.parametrize("T", [1, 17, 64, 65, 100, 257, 300, 2049])
@pytest.mark.parametrize("g,sbd,y_dt", [(64, "bf16", torch.bfloat16), (32, "f32", torch.float32),
                                        (128, "bf16", torch.float32)])
def test_multi_small_ragged(T, g, sbd, y_dt):
    """Three matrices of ragged widths (one tile each or less, one over two tiles)."""
    rng = np.random.default_rng(T * 13 + g)
    k_in = 384 if g != 128 else 512
    ws = [synth.draw_matrix(rng, n, k_in, g, sbd) for n in (96, 32, 288)]
    X = synth.draw_activation(rng, (T, k_in), "bf16")
    ys = _run(ws, X, y_dt)
    for i, (w, y) in enumerate(zip(ws, ys)):
        Y, A = oracle.gemm(w, X, "bf16", round_w=True, threads=oracle_threads())
        slack, n_sites = gemm_rounding_slack(w, X)
        if sbd == "bf16":
            assert n_sites == 0
        check_gemm(y, Y, A, "multi T=%d m=%d" % (T, i), slack=slack)


@pytest.mark.parametrize("T", [130, 2050])
def test_multi_canaries_strides_and_eight_matrices(T):
    """Eight matrices with row strides above n_out: columns past n_out keep their canary."""
    rng = np.random.default_rng(501 + T)
    k_in = 256
    outs = [32, 64, 256, 32, 96, 544, 32, 160]
    ws = [synth.draw_matrix(rng, n, k_in, 64, "bf16") for n in outs]
    X = synth.draw_activation(rng, (T, k_in), "bf16")
    ldys = [n + 24 for n in outs]
    ys = _run(ws, X, torch.bfloat16, ldys=ldys, fill=5.0)
    for i, (w, y) in enumerate(zip(ws, ys)):
        Y, A = oracle.gemm(w, X, "bf16", round_w=True)
        check_gemm(y[:, :w.n_out], Y, A, "multi8 m=%d" % i)
        assert torch.all(y[:, w.n_out:] == 5.0)


@pytest.mark.parametrize("T", [200, 2100])
def test_multi_equals_single_calls_bit_for_bit(T):
    """For T > 64 each output equals qgemm_int4_padT of its matrix alone (same tiles)."""
    q = lib()
    rng = np.random.default_rng(502)
    ws = [synth.draw_matrix(rng, n, 1024, 64, "bf16") for n in (256, 128, 128)]
    X = synth.draw_activation(rng, (T, 1024), "bf16")
    ys = _run(ws, X, torch.float32)
    xs = synth.to_torch(X, "bf16")
    for w, y in zip(ws, ys):
        y1 = torch.full((T, w.n_out), float("nan"), dtype=torch.float32, device="cuda")
        q.qgemm_int4_padT(dev_matrix(w), xs, y1)
        torch.cuda.synchronize()
        assert torch.equal(y, y1)


@pytest.mark.parametrize("T", [32, 256, 1024])
def test_multi_qkv_workload(T):
    """q/k/v of a 4096-wide block: 4096 -> 4096 / 1024 / 1024, g64, bf16 scales and outputs;
    every output against the oracle."""
    d = synth.qkv_multi()
    X = synth.draw_activation(np.random.default_rng(600 + T), (T, 4096), "bf16")
    ys = _run(d["ws"], X, torch.bfloat16)
    for name, w, y in zip("qkv", d["ws"], ys):
        Y, A = oracle.gemm(w, X, "bf16", round_w=True, threads=oracle_threads())
        check_gemm(y, Y, A, "qkv prefill T=%d %s" % (T, name))
