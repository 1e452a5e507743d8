"""GPU parity of quantize_int4 against the oracle quantiser (through the C ABI).

Codes, scales and biases are integer/bit decisions and must match exactly: both
sides take them in float32 (min/max, (max - min) / 15, bf16 rounding to nearest
even, (w - b') / s' correctly rounded, rint ties to even).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import check, dev_matrix, lib, nan_like, require_gpu

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int32).numpy().view(np.uint32)


def _as_bits(a: np.ndarray, dt: str) -> np.ndarray:
    return a.view(np.uint16) if dt == "bf16" else np.ascontiguousarray(a, np.float32).view(np.uint32)


def _quantize(W: np.ndarray, w_dt: str, group: int, sb_dt: str):
    q = lib()
    m = q.quantize_int4(synth.to_torch(W, w_dt), group, TD[sb_dt])
    torch.cuda.synchronize()
    return m


def _compare(W, w_dt, group, sb_dt):
    m = _quantize(W, w_dt, group, sb_dt)
    codes, s, b = oracle.quantize(W, w_dt, group, sb_dt)
    got_c = _bits(m.codes)
    assert np.array_equal(got_c, codes), "codes differ at %d words" % np.count_nonzero(got_c != codes)
    assert np.array_equal(_bits(m.scales), _as_bits(s, sb_dt))
    assert np.array_equal(_bits(m.biases), _as_bits(b, sb_dt))
    return m


@pytest.mark.parametrize("n_out,k_in,group", [(1, 32, 32), (3, 64, 64), (17, 256, 128), (100, 1024, 64),
                                              (257, 5120, 64), (9, 17408, 64), (64, 96, 32)])
@pytest.mark.parametrize("w_dt,sb_dt", [("f32", "bf16"), ("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_quantize_bit_exact(n_out, k_in, group, w_dt, sb_dt):
    rng = np.random.default_rng(n_out * 7 + k_in + group)
    W = synth.draw_float_weights(rng, (n_out, k_in), w_dt)
    _compare(W, w_dt, group, sb_dt)


def test_quantize_full_dense_matrix():
    """The measured workload: 17408 x 5120 float32 weights -> g64 codes with bf16 scales."""
    rng = np.random.default_rng(11)
    W = synth.draw_float_weights(rng, (17408, 5120), "f32")
    _compare(W, "f32", 64, "bf16")


def test_quantize_expert_stack_and_special_groups():
    """A 3-D expert stack; constant groups, wide-range groups and exact ties (x.5 quotients)."""
    rng = np.random.default_rng(12)
    W = synth.draw_float_weights(rng, (4, 48, 256), "f32")
    W[0, 0, :64] = 0.25                     # constant group: s = 0, codes 0
    W[1, 2, 64:128] = np.linspace(-3e4, 5e4, 64, dtype=np.float32)
    W[2, 5, :64] = np.arange(64, dtype=np.float32) * 0.5  # many (w - b) / s ties at .5
    _compare(W, "f32", 64, "bf16")
    _compare(W, "f32", 64, "f32")


def test_quantized_matrix_feeds_the_gemv():
    """quantize_int4 output used directly by qgemv_int4 matches the oracle GEMV of the oracle's
    quantisation of the same weights."""
    q = lib()
    rng = np.random.default_rng(13)
    W = synth.draw_float_weights(rng, (640, 2048), "bf16")
    m = _quantize(W, "bf16", 64, "bf16")
    x = synth.draw_activation(rng, (2048,), "bf16")
    y = nan_like(640, torch.bfloat16)
    q.qgemv_int4(m, synth.to_torch(x, "bf16"), y)
    torch.cuda.synchronize()
    codes, s, b = oracle.quantize(W, "bf16", 64, "bf16")
    ref_w = synth.QMatrix(codes=codes, scales=s, biases=b, sb_dtype="bf16", group_size=64,
                          n_out=640, k_in=2048)
    ref, a = oracle.gemv(ref_w, x, "bf16")
    check(y, ref, a, "quantised gemv")
