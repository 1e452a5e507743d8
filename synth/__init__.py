"""Seeded synthetic inputs for the int4 group-affine GEMV/GEMM path.

This module only *draws* data: packed 4-bit codes, per-group scales and
biases, activations, residuals and router logits.  It holds none of the
method's arithmetic (no unpacking, no dequantisation, no products); both the
fp64 CPU oracle and the HIP path consume what it produces.

Storage format (the FFAI pages, PR #14, batched-QKV precondition commit:
a packed weight has ``in_dim = shape[1] * 8``, i.e. 8 codes per u32 along
``in_dim``):

* ``codes``  -- uint32 ``[E][n_out][k_in/8]`` (E omitted for a plain matrix).
  Code ``k`` of a row sits in word ``k // 8`` at bits ``4*(k % 8)`` ..
  ``4*(k % 8)+3`` (low nibble first).  The pages never print the nibble order;
  this is the plainest reading (the first code in the least significant bits).
* ``scales``/``biases`` -- ``[E][n_out][k_in/group_size]``, either float32 or
  bfloat16.  bfloat16 arrays are held as their raw uint16 bit patterns because
  numpy has no bfloat16 type.

Value recipe (the single-GEMV workload's, reused by every workload):
codes uniform in 0..15, scales uniform in [0.005, 0.02], biases
``-8*scale + N(0, 0.001)``, activations N(0, 1).  Draw order per seed:
for each matrix in order: codes, scales, bias noise; then x, then residual,
then router logits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even) via torch's cast.

    Returns the uint16 bit patterns.  Used only to *store* generated data in
    bfloat16; it plays no part in the computation under test.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for data recipes only)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class QMatrix:
    """One packed int4 matrix, or a stack of ``n_experts`` of them."""

    codes: np.ndarray            # uint32 [E?][n_out][k_in//8]
    scales: np.ndarray           # float32, or uint16 bf16 bits, [E?][n_out][k_in//g]
    biases: np.ndarray
    sb_dtype: str                # "f32" | "bf16"
    group_size: int
    n_out: int
    k_in: int
    n_experts: int = 1           # 1 => plain matrix (no leading E axis)
    raw_codes: Optional[np.ndarray] = field(default=None, repr=False)  # uint8 [E?][n_out][k_in]

    @property
    def weight_bytes(self) -> int:
        return int(self.codes.nbytes + self.scales.nbytes + self.biases.nbytes)


def pack_codes(raw: np.ndarray) -> np.ndarray:
    """Pack uint8 codes (values 0..15) along the last axis, 8 per little-endian u32.

    Two codes share a byte (even index in the low nibble), and four bytes form
    a word in little-endian order, so code k lands at bits 4*(k%8) of word k//8.
    """
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    if raw.shape[-1] % 8:
        raise ValueError("last axis must be a multiple of 8")
    if raw.size and int(raw.max()) > 15:
        raise ValueError("codes must lie in 0..15")
    byte = (raw[..., 0::2] | (raw[..., 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(byte).view("<u4").astype(np.uint32, copy=False)


def draw_matrix(rng: np.random.Generator, n_out: int, k_in: int, group_size: int,
                sb_dtype: str, n_experts: int = 1, keep_raw: bool = False,
                scale_lo: float = 0.005, scale_hi: float = 0.02,
                bias_noise: float = 0.001) -> QMatrix:
    """Draw one matrix (or expert stack) with the value recipe above."""
    if k_in % group_size or k_in % 8:
        raise ValueError("k_in must be a multiple of group_size and of 8")
    lead = (n_experts,) if n_experts > 1 else ()
    groups = k_in // group_size
    raw = rng.integers(0, 16, size=lead + (n_out, k_in), dtype=np.uint8)
    codes = pack_codes(raw)
    s = rng.uniform(scale_lo, scale_hi, size=lead + (n_out, groups)).astype(np.float32)
    noise = rng.normal(0.0, bias_noise, size=lead + (n_out, groups))
    if sb_dtype == F32:
        scales = s
        biases = (-8.0 * s.astype(np.float64) + noise).astype(np.float32)
    elif sb_dtype == BF16:
        scales = f32_to_bf16_bits(s)
        s_r = bf16_bits_to_f32(scales).astype(np.float64)
        biases = f32_to_bf16_bits((-8.0 * s_r + noise).astype(np.float32))
    else:
        raise ValueError(sb_dtype)
    return QMatrix(codes=codes, scales=scales, biases=biases, sb_dtype=sb_dtype,
                   group_size=group_size, n_out=n_out, k_in=k_in, n_experts=n_experts,
                   raw_codes=raw if keep_raw else None)


def draw_activation(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) activations: float32 array, or uint16 bf16 bits when dtype is bf16."""
    a = rng.standard_normal(size=shape).astype(np.float32)
    return a if dtype == F32 else f32_to_bf16_bits(a)


def draw_float_weights(rng: np.random.Generator, shape, dtype: str, std: float = 0.02) -> np.ndarray:
    """Unquantised weights N(0, std^2) (the quantiser's input), float32 or bf16 bits."""
    a = (std * rng.standard_normal(size=shape)).astype(np.float32)
    return a if dtype == F32 else f32_to_bf16_bits(a)


def draw_norm_weight(rng: np.random.Generator, n: int, dtype: str) -> np.ndarray:
    """RMSNorm weight [n]: uniform in [0.5, 1.5], stored in dtype (bf16 as bits)."""
    g = rng.uniform(0.5, 1.5, size=n).astype(np.float32)
    return g if dtype == F32 else f32_to_bf16_bits(g)


# --------------------------------------------------------------------------
# Workload recipes.  Default sizes are the decode/prefill shapes measured;
# tests pass smaller sizes to the same recipes.
# --------------------------------------------------------------------------

def single_gemv(seed: int = 0, n_out: int = 1024, k_in: int = 1024, group_size: int = 64,
                sb_dtype: str = F32, x_dtype: str = F32, keep_raw: bool = False) -> dict:
    """Single int4 GEMV at T=1 (1024x1024, g64, fp32 scales/biases, fp32 x and y)."""
    rng = np.random.default_rng(seed)
    w = draw_matrix(rng, n_out, k_in, group_size, sb_dtype, keep_raw=keep_raw)
    x = draw_activation(rng, (k_in,), x_dtype)
    return {"w": w, "x": x, "x_dtype": x_dtype}


def qkv_multi(seed: int = 1, hidden: int = 4096, outs=(4096, 1024, 1024), group_size: int = 64,
              keep_raw: bool = False) -> dict:
    """Three projections sharing one bf16 input (q/k/v at T=1), bf16 scales/biases."""
    rng = np.random.default_rng(seed)
    ws = [draw_matrix(rng, n, hidden, group_size, BF16, keep_raw=keep_raw) for n in outs]
    x = draw_activation(rng, (hidden,), BF16)
    return {"ws": ws, "x": x, "x_dtype": BF16}


def rms_qkv(seed: int = 5, hidden: int = 4096, outs=(4096, 1024, 1024), group_size: int = 64,
            eps: float = 1e-6) -> dict:
    """The q/k/v projection set behind an RMSNorm of its bf16 input: the qkv_multi
    recipe, then the norm weight (bf16, uniform in [0.5, 1.5]); eps is the
    float32 value passed to the library."""
    rng = np.random.default_rng(seed)
    ws = [draw_matrix(rng, n, hidden, group_size, BF16) for n in outs]
    x = draw_activation(rng, (hidden,), BF16)
    gamma = draw_norm_weight(rng, hidden, BF16)
    return {"ws": ws, "x": x, "gamma": gamma, "eps": float(np.float32(eps)), "x_dtype": BF16}


def dense_layer(seed: int = 2, hidden: int = 5120, inter: int = 17408, group_size: int = 64,
                keep_raw: bool = False) -> dict:
    """Dense decoder-layer GEMV set: gate/up hidden->inter, down inter->hidden."""
    rng = np.random.default_rng(seed)
    gate = draw_matrix(rng, inter, hidden, group_size, BF16, keep_raw=keep_raw)
    up = draw_matrix(rng, inter, hidden, group_size, BF16, keep_raw=keep_raw)
    down = draw_matrix(rng, hidden, inter, group_size, BF16, keep_raw=keep_raw)
    x = draw_activation(rng, (hidden,), BF16)
    return {"gate": gate, "up": up, "down": down, "x": x, "x_dtype": BF16}


def moe_layer(seed: int = 3, n_experts: int = 128, hidden: int = 2048, inter: int = 768,
              group_size: int = 64, n_tokens: int = 1, keep_raw: bool = False) -> dict:
    """Top-K MoE decode: stacked experts, bf16 x and residual, N(0,1) router logits.

    ``n_tokens`` rows of (x, residual, logits) are drawn, one per decode step.
    """
    rng = np.random.default_rng(seed)
    gate = draw_matrix(rng, inter, hidden, group_size, BF16, n_experts=n_experts, keep_raw=keep_raw)
    up = draw_matrix(rng, inter, hidden, group_size, BF16, n_experts=n_experts, keep_raw=keep_raw)
    down = draw_matrix(rng, hidden, inter, group_size, BF16, n_experts=n_experts, keep_raw=keep_raw)
    x = draw_activation(rng, (n_tokens, hidden), BF16)
    residual = draw_activation(rng, (n_tokens, hidden), BF16)
    logits = rng.standard_normal(size=(n_tokens, n_experts)).astype(np.float32)
    return {"gate": gate, "up": up, "down": down, "x": x, "residual": residual,
            "logits": logits, "x_dtype": BF16}


def moe_prefill_layer(seed: int = 6, T: int = 256, n_experts: int = 128, hidden: int = 2048,
                      inter: int = 768, group_size: int = 64) -> dict:
    """Top-K MoE prefill: the moe_layer recipe with T rows of x, residual and
    N(0,1) router logits (the decode workload's per-token draws, T at once)."""
    return moe_layer(seed=seed, n_experts=n_experts, hidden=hidden, inter=inter,
                     group_size=group_size, n_tokens=T)


PREFILL_T = (32, 256, 1000, 1024, 4096)


def prefill_gemm(seed: int = 4, T: int = 32, n_out: int = 17408, k_in: int = 5120,
                 group_size: int = 64, keep_raw: bool = False) -> dict:
    """Prefill dequant GEMM: one int4 matrix and a bf16 activation block [T][k_in]."""
    rng = np.random.default_rng(seed)
    w = draw_matrix(rng, n_out, k_in, group_size, BF16, keep_raw=keep_raw)
    X = draw_activation(rng, (T, k_in), BF16)
    return {"w": w, "X": X, "x_dtype": BF16, "T": T}


# --------------------------------------------------------------------------
# Device-side pools for throughput runs.  A pool holds R distinct weight
# copies so that back-to-back calls stream from HBM rather than from the
# 256 MB last-level cache.  Uniform random 32-bit words have independent
# uniform nibbles, i.e. codes uniform in 0..15, as in the recipe above.
# --------------------------------------------------------------------------

def torch_matrix(n_out: int, k_in: int, group_size: int, sb_dtype: str, n_experts: int = 1,
                 seed: int = 0, device: str = "cuda"):
    """Draw one matrix (or expert stack) directly on ``device`` with torch.

    Returns a dict of tensors: ``codes`` int32 [E?][n_out][k_in/8], ``scales`` and
    ``biases`` (float32 or bfloat16) [E?][n_out][k_in/g].
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    lead = (n_experts,) if n_experts > 1 else ()
    codes = torch.randint(-(2 ** 31), 2 ** 31, lead + (n_out, k_in // 8), generator=g,
                          device=device, dtype=torch.int64).to(torch.int32)
    groups = k_in // group_size
    s = torch.rand(lead + (n_out, groups), generator=g, device=device) * 0.015 + 0.005
    noise = torch.randn(lead + (n_out, groups), generator=g, device=device) * 0.001
    if sb_dtype == BF16:
        s = s.to(torch.bfloat16)
        b = (-8.0 * s.float() + noise).to(torch.bfloat16)
    else:
        b = -8.0 * s + noise
    return {"codes": codes, "scales": s.contiguous(), "biases": b.contiguous()}


# --------------------------------------------------------------------------
# numpy -> torch marshalling (device placement only, values unchanged)
# --------------------------------------------------------------------------

def to_torch(a: np.ndarray, dtype: str, device: str = "cuda"):
    """float32 array, or uint16 bf16 bit patterns, as a torch tensor on ``device``."""
    import torch

    a = np.ascontiguousarray(a)
    if dtype == BF16:
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be uint16 bit patterns")
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif dtype == F32:
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    else:
        raise ValueError(dtype)
    return t.to(device)


def matrix_to_torch(w: QMatrix, device: str = "cuda") -> dict:
    """Codes (as int32 bit patterns), scales and biases of ``w`` on ``device``."""
    import torch

    codes = torch.from_numpy(np.ascontiguousarray(w.codes).view(np.int32)).to(device)
    return {"codes": codes, "scales": to_torch(w.scales, w.sb_dtype, device),
            "biases": to_torch(w.biases, w.sb_dtype, device), "group_size": w.group_size}
