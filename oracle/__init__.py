"""fp64 CPU oracle for group-affine int4 GEMV / multi-GEMV / MoE / prefill GEMM.

TEST INFRASTRUCTURE ONLY.  This package is the checker for the HIP library:
only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import it.  It shares no code with the HIP path; the seeded generators in
``synth`` are the only thing both sides use.

Sources, cited by page title and passage:

* [FFAI #14]  thewafflehaus/FFAI pull 14, "feat(everything-bagel): clean
  migration of PR #9 + #10 onto updated dev".
* [FFAI #9]   thewafflehaus/FFAI pull 9, "Everything Bagel".
* [ds4 #844]  antirez/ds4 pull 844, "Ornith 1.5 + Qwen 3.8 27B hybrid runtime +
  DFlash speculative decoding on Metal".

The integer and product arithmetic lives in ``oracle.c`` (plain double loops);
this module widens stored values exactly to float64, and composes the steps
the pages describe (SwiGLU, router top-K, expert gather, weighted combine) in
plain float64 numpy.

Pinning: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms, exact rational brute force, library routines or the
worked router example the pages print.  No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32 = "f32"
BF16 = "bf16"


# --------------------------------------------------------------------------
# build / load
# --------------------------------------------------------------------------

def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
               "-fPIC", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.orc_unpack.argtypes = [P, I64, I64, P]
        lib.orc_dequant.argtypes = [P, P, P, I64, I64, I64, P]
        lib.orc_gemv.argtypes = [P, P, P, I64, I64, I64, P, P, P, ctypes.c_int]
        lib.orc_gemv_absw.argtypes = [P, P, P, I64, I64, I64, P, P, ctypes.c_int]
        lib.orc_round_bf16.argtypes = [ctypes.c_double]
        lib.orc_round_bf16.restype = ctypes.c_double
        lib.orc_round_bf16_array.argtypes = [P, I64, P]
        lib.orc_gemm_entries.argtypes = [P, P, P, I64, I64, I64, P, I64, P, P, I64,
                                         ctypes.c_int, P, P, ctypes.c_int]
        lib.orc_gemm.argtypes = [P, P, P, I64, I64, I64, P, I64, ctypes.c_int, P, P,
                                 ctypes.c_int]
        lib.orc_gemm.restype = ctypes.c_int
        lib.orc_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().orc_max_threads())


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# exact widening of stored values
# --------------------------------------------------------------------------

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly.

    bfloat16 is the upper half of an IEEE binary32 word, so its bit pattern
    shifted left by 16 is the float32 of the same value; float32 -> float64 is
    exact.
    """
    if dtype == BF16:
        a = np.asarray(a)
        if a.dtype != np.uint16:
            raise TypeError("bf16 arrays are passed as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def _slab(w, expert: Optional[int]):
    """(codes, scales, biases) of one matrix, or of expert ``expert`` of a stack."""
    if w.n_experts > 1 or expert is not None:
        e = 0 if expert is None else int(expert)
        if w.n_experts > 1:
            return w.codes[e], w.scales[e], w.biases[e]
        if e != 0:
            raise IndexError("plain matrix has only expert 0")
    return w.codes, w.scales, w.biases


# --------------------------------------------------------------------------
# unpack / dequant / GEMV
# --------------------------------------------------------------------------

def unpack(codes: np.ndarray, k_in: int) -> np.ndarray:
    """Codes uint32 [..., rows, k_in/8] -> uint8 [..., rows, k_in] (word k//8, nibble k%8)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    lead = codes.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    q = np.empty(lead + (k_in,), dtype=np.uint8)
    _load().orc_unpack(_p(codes), rows, k_in, _p(q))
    return q


def dequant(w, expert: Optional[int] = None) -> np.ndarray:
    """float64 [n_out, k_in] weights w = s * q + b of one matrix / expert."""
    c, s, b = _slab(w, expert)
    c = np.ascontiguousarray(c, dtype=np.uint32)
    sd = np.ascontiguousarray(widen(s, w.sb_dtype))
    bd = np.ascontiguousarray(widen(b, w.sb_dtype))
    out = np.empty((w.n_out, w.k_in), dtype=np.float64)
    _load().orc_dequant(_p(c), _p(sd), _p(bd), w.n_out, w.k_in, w.group_size, _p(out))
    return out


def gemv_f64(w, x64: np.ndarray, expert: Optional[int] = None,
             threads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """y = W x and a = sum |w x| in float64, x already float64 [k_in]."""
    c, s, b = _slab(w, expert)
    c = np.ascontiguousarray(c, dtype=np.uint32)
    sd = np.ascontiguousarray(widen(s, w.sb_dtype))
    bd = np.ascontiguousarray(widen(b, w.sb_dtype))
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    if x64.shape != (w.k_in,):
        raise ValueError("x must have shape (k_in,)")
    y = np.empty(w.n_out, dtype=np.float64)
    a = np.empty(w.n_out, dtype=np.float64)
    _load().orc_gemv(_p(c), _p(sd), _p(bd), w.n_out, w.k_in, w.group_size, _p(x64),
                     _p(y), _p(a), int(threads))
    return y, a


def gemv(w, x: np.ndarray, x_dtype: str, expert: Optional[int] = None,
         threads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Single int4 GEMV on stored x (float32 or bf16 bits)."""
    return gemv_f64(w, widen(x, x_dtype), expert=expert, threads=threads)


def multi(ws: Sequence, x: np.ndarray, x_dtype: str, threads: int = 1):
    """Several projections of one shared input ([FFAI #14], batched QKV / 4-way
    qgemv commits: one input, N outputs).  Returns a list of (y, a)."""
    x64 = widen(x, x_dtype)
    return [gemv_f64(w, x64, threads=threads) for w in ws]


# --------------------------------------------------------------------------
# RMSNorm prologue
# --------------------------------------------------------------------------

def rms_norm(x: np.ndarray, x_dtype: str, gamma: np.ndarray, eps: float) -> np.ndarray:
    """xn[k] = x[k] * gamma[k] / sqrt(mean_j x[j]^2 + eps) in float64.

    [FFAI #14], commit wrapping the RMSNorm-fused qgemv: the normalised
    activation feeds the int4 dequant GEMV directly.  [ds4 #844], commit
    unifying the norm kernels: the normaliser is 1 / sqrt(mean + eps).  gamma
    is stored in x's dtype; eps is used as given (callers pass the float32
    value the library receives).
    """
    x64 = widen(x, x_dtype)
    g64 = widen(gamma, x_dtype)
    if x64.shape != g64.shape or x64.ndim != 1:
        raise ValueError("x and gamma must be equal-length vectors")
    ms = np.mean(x64 * x64)
    return x64 * g64 / np.sqrt(ms + float(eps))


def rms_norm_multi(ws: Sequence, x: np.ndarray, x_dtype: str, gamma: np.ndarray, eps: float,
                   threads: int = 1):
    """Projections of one RMS-normalised input; a list of (y, a) as in multi()."""
    xn = rms_norm(x, x_dtype, gamma, eps)
    return [gemv_f64(w, xn, threads=threads) for w in ws]


def rms_norm_swiglu_pair(gate, up, x: np.ndarray, x_dtype: str, gamma: np.ndarray, eps: float,
                         threads: int = 1):
    """silu(gate xn) * (up xn) of the RMS-normalised input; (h, a_h) as in swiglu_pair()."""
    xn = rms_norm(x, x_dtype, gamma, eps)
    g, ag = gemv_f64(gate, xn, threads=threads)
    u, au = gemv_f64(up, xn, threads=threads)
    return swiglu(g, u), 1.1 * np.abs(u) * ag + np.abs(silu(g)) * au


# --------------------------------------------------------------------------
# SwiGLU, dense FFN, router, MoE
# --------------------------------------------------------------------------

def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in float64; exp overflow for g << 0 gives -0."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(gate) * up ([FFAI #9], commit fusing silu and mul into one swiglu)."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def swiglu_pair(gate, up, x: np.ndarray, x_dtype: str, threads: int = 1):
    """Gate and up projections of one input followed by SwiGLU.

    Returns (h, a_h) where a_h bounds |h| error propagation:
    |dh| <= |silu'(g)| |u| |dg| + |silu(g)| |du| is reported through
    a_h = |u| a_g + |silu(g)| a_u (silu' is bounded by 1.1).
    """
    x64 = widen(x, x_dtype)
    g, ag = gemv_f64(gate, x64, threads=threads)
    u, au = gemv_f64(up, x64, threads=threads)
    h = swiglu(g, u)
    a_h = 1.1 * np.abs(u) * ag + np.abs(silu(g)) * au
    return h, a_h


def gemv_absw(w, v64: np.ndarray, expert: Optional[int] = None, threads: int = 1) -> np.ndarray:
    """m = |W| v for a non-negative float64 vector v (error propagation bound)."""
    c, s, b = _slab(w, expert)
    c = np.ascontiguousarray(c, dtype=np.uint32)
    sd = np.ascontiguousarray(widen(s, w.sb_dtype))
    bd = np.ascontiguousarray(widen(b, w.sb_dtype))
    v64 = np.ascontiguousarray(v64, dtype=np.float64)
    m = np.empty(w.n_out, dtype=np.float64)
    _load().orc_gemv_absw(_p(c), _p(sd), _p(bd), w.n_out, w.k_in, w.group_size, _p(v64),
                          _p(m), int(threads))
    return m


def dense_ffn(gate, up, down, x: np.ndarray, x_dtype: str, threads: int = 1):
    """down( silu(gate x) * (up x) ) in float64.

    Returns (y, a_y, h, a_h): a_y = sum|w_down h| + |W_down| a_h, the magnitude
    against which a float32 implementation's rounding noise is measured
    (including what its float32 h carries into the down projection).
    """
    h, a_h = swiglu_pair(gate, up, x, x_dtype, threads=threads)
    y, a = gemv_f64(down, h, threads=threads)
    a_y = a + gemv_absw(down, a_h, threads=threads)
    return y, a_y, h, a_h


def router_topk(logits: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Router: softmax over all experts, keep the top-k, renormalise.

    Ordering is by probability descending, ties by expert index ascending
    ([FFAI #9], commit replacing the full sort in MoERouter.topKIndices with a
    k-heap while keeping the (value desc, index asc) tie-break).  Returns
    (ids int64 [k], weights float64 [k]) in that order.
    """
    z = np.asarray(logits, dtype=np.float64)
    p = np.exp(z - z.max())
    p = p / p.sum()
    order = np.lexsort((np.arange(z.size), -p))  # primary key -p, secondary index
    ids = order[:k].astype(np.int64)
    kept = p[ids]
    return ids, kept / kept.sum()


def combine(residual64: Optional[np.ndarray], scalars: Sequence[float],
            values: Sequence[np.ndarray]) -> np.ndarray:
    """Weighted accumulate: out = residual + sum_k scalars[k] * values[k].

    The scalar-broadcast FMA chain of [FFAI #14] (commit adding scalarFMA,
    scalarFMAMany and the 8-way scalarFMAChain8: out[i] = base[i] +
    scalar * value[i], applied once per kept expert).
    """
    out = np.zeros_like(np.asarray(values[0], dtype=np.float64))
    if residual64 is not None:
        out = out + residual64
    for a, v in zip(scalars, values):
        out = out + float(a) * np.asarray(v, dtype=np.float64)
    return out


def moe(gate, up, down, x: np.ndarray, ids: Sequence[int], wts: Sequence[float],
        residual: Optional[np.ndarray], x_dtype: str, threads: int = 1):
    """Top-K MoE decode step on stacked experts.

    For each kept slot k with expert e = ids[k] ([FFAI #14], expert-indexed GEMV
    commit: e selects a slab of the stacked [nExperts, outDim, inDim/8] tensor):
      h_k = silu(W_gate[e] x) * (W_up[e] x);  d_k = W_down[e] h_k;
    then out = residual + sum_k wts[k] * d_k ([FFAI #14], chain8 down+SwiGLU+
    accumulate commit).  Expert ids outside [0, n_experts) contribute nothing
    (the library's documented contract for untrusted device ids).

    Returns (out, a_out) where a_out = |residual| + sum_k |wts_k| a_k bounds
    the accumulation noise.
    """
    x64 = widen(x, x_dtype)
    res64 = None if residual is None else widen(residual, x_dtype)
    ds, scal, mags = [], [], []
    for e, a_k in zip(ids, wts):
        e = int(e)
        if e < 0 or e >= gate.n_experts:
            continue
        g, ag = gemv_f64(gate, x64, expert=e, threads=threads)
        u, au = gemv_f64(up, x64, expert=e, threads=threads)
        h = swiglu(g, u)
        a_h = 1.1 * np.abs(u) * ag + np.abs(silu(g)) * au
        d, ad = gemv_f64(down, h, expert=e, threads=threads)
        ad = ad + gemv_absw(down, a_h, expert=e, threads=threads)
        ds.append(d)
        scal.append(float(a_k))
        mags.append(abs(float(a_k)) * ad)
    if not ds:
        zero = np.zeros(down.n_out, dtype=np.float64)
        return (zero if res64 is None else res64.copy()), (np.zeros_like(zero) if res64 is None
                                                             else np.abs(res64))
    out = combine(res64, scal, ds)
    a_out = np.sum(mags, axis=0) + (0.0 if res64 is None else np.abs(res64))
    return out, a_out


# --------------------------------------------------------------------------
# quantiser
# --------------------------------------------------------------------------

def _bf16_bits_of(v32: np.ndarray) -> np.ndarray:
    """Bit patterns of float32 values that are already bfloat16 values (upper halves)."""
    return (np.ascontiguousarray(v32, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def quantize(w: np.ndarray, w_dtype: str, group_size: int, sb_dtype: str):
    """Min/max group-affine int4 quantiser.  Returns (codes uint32 [..., k_in/8],
    scales, biases [..., k_in/group_size] stored in sb_dtype, bf16 as bits).

    [ds4 #844], PR body (verification list): the codes come from the stored
    (bf16-rounded) scale and bias.  Per group: s = (max - min) / 15, b = min,
    s' and b' their stored values, q = clamp(rint((w - b') / s'), 0, 15)
    (0 where s' == 0).  The integer decision is taken in float32, the
    precision the device kernel computes it in: numpy float32 subtraction and
    division are IEEE operations rounded to nearest, and rint rounds ties to
    even.
    """
    w32 = widen(w, w_dtype).astype(np.float32)  # exact: the stored values
    k_in = w32.shape[-1]
    if k_in % group_size:
        raise ValueError("k_in must be a multiple of group_size")
    G = w32.reshape(w32.shape[:-1] + (k_in // group_size, group_size))
    lo = G.min(axis=-1)
    hi = G.max(axis=-1)
    s = (hi - lo) / np.float32(15.0)
    b = lo
    if sb_dtype == BF16:
        s = round_bf16(s.astype(np.float64)).astype(np.float32)
        b = round_bf16(b.astype(np.float64)).astype(np.float32)
    sn, bn = s[..., None], b[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.rint((G - bn) / np.where(sn > 0, sn, np.float32(1.0)))
    q = np.where(sn > 0, np.clip(t, 0, 15), 0).astype(np.uint32).reshape(w32.shape)
    # pack: code k of a row at bits 4 * (k % 8) of word k // 8
    qw = q.reshape(q.shape[:-1] + (k_in // 8, 8))
    codes = np.zeros(qw.shape[:-1], dtype=np.uint32)
    for k in range(8):
        codes |= qw[..., k] << np.uint32(4 * k)
    if sb_dtype == BF16:
        return codes, _bf16_bits_of(s), _bf16_bits_of(b)
    return codes, s.astype(np.float32), b.astype(np.float32)


# --------------------------------------------------------------------------
# prefill GEMM
# --------------------------------------------------------------------------

def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    _load().orc_round_bf16_array(_p(v), v.size, _p(out))
    return out


def gemm_f64(w, X64: np.ndarray, round_w: bool = True, expert: Optional[int] = None,
             threads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Y[t][o] = sum_k w'[o][k] X64[t][k] and A = sum_k |w' X| for float64 rows X64
    (w' = the exact weight s q + b rounded once to the nearest bfloat16, ties to even,
    when round_w); one matrix or expert ``expert`` of a stack."""
    c, s, b = _slab(w, expert)
    c = np.ascontiguousarray(c, dtype=np.uint32)
    sd = np.ascontiguousarray(widen(s, w.sb_dtype))
    bd = np.ascontiguousarray(widen(b, w.sb_dtype))
    X64 = np.ascontiguousarray(X64, dtype=np.float64)
    if X64.ndim != 2 or X64.shape[1] != w.k_in:
        raise ValueError("X must be [T][k_in]")
    T = X64.shape[0]
    Y = np.empty((T, w.n_out), dtype=np.float64)
    A = np.empty((T, w.n_out), dtype=np.float64)
    rc = _load().orc_gemm(_p(c), _p(sd), _p(bd), w.n_out, w.k_in, w.group_size, _p(X64), T,
                          int(bool(round_w)), _p(Y), _p(A), int(threads))
    if rc != 0:
        raise MemoryError("orc_gemm: row buffer allocation failed")
    return Y, A


def gemm(w, X: np.ndarray, x_dtype: str = BF16, round_w: bool = True,
         threads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Full Y[t][o] = sum_k w'[o][k] X[t][k] for all T rows (small sizes).

    Padding T up to a multiple of 32 appends zero rows whose outputs are sliced
    away ([FFAI #9], dequantGemmDynamicM T-padding driver), so the result for
    the T real rows is this plain product.  When round_w, w' is the weight
    dequantised to bfloat16 before the product ([FFAI #9], the padded dequant GEMM
    multiplies bf16 weight tiles): the exact s q + b rounded once to the nearest
    bfloat16, ties to even.
    """
    return gemm_f64(w, widen(X, x_dtype), round_w=round_w, threads=threads)


def moe_prefill(gate, up, down, X: np.ndarray, ids: np.ndarray, wts: np.ndarray,
                residual: Optional[np.ndarray], res_dtype: str = BF16,
                tokens: Optional[Sequence[int]] = None, threads: int = 1):
    """T tokens through the top-K MoE in the prefill form.

    [FFAI #9], batched MoE commits: the T * topK (token, slot) rows are fanned
    into one GEMM per gate / up / down, grouped by expert id, then unpermuted by
    a scatter-sum.  Here the rows of each expert go through that expert's
    prefill GEMMs (gemm(), weights w' = RNE_bf16(s q + b)) in one call each;
    grouping changes no row's value, so each token's output is the decode step
    of moe() with the prefill weights:
      h_k = silu(W'_gate[e] x) * (W'_up[e] x),  out = residual + sum_k w_k W'_down[e] h_k,
    e = ids[t][k]; ids outside [0, n_experts) contribute nothing.  X is bf16
    [T][hidden]; residual (or None) is [T][hidden] in res_dtype.

    Returns (out [n][hidden], a_out [n][hidden]) for the rows ``tokens``
    (default: all), a_out bounding the float32 accumulation noise as in moe():
    the down product's own sum |w' h| plus sum |w'| a_h, what the error bound a_h
    of the float32 intermediate h carries through it.
    """
    X64 = widen(X, BF16)
    T = X64.shape[0]
    tokens = list(range(T)) if tokens is None else [int(t) for t in tokens]
    ids = np.asarray(ids)
    n, top_k, hidden = len(tokens), ids.shape[1], down.n_out
    D = np.zeros((n, top_k, hidden))
    AD = np.zeros((n, top_k, hidden))
    valid = np.zeros((n, top_k), bool)
    tok_idx = np.repeat(np.arange(n), top_k)          # (token position, slot) rows
    slot_idx = np.tile(np.arange(top_k), n)
    expert = ids[np.asarray(tokens, dtype=np.int64)].reshape(-1).astype(np.int64)
    for e in np.unique(expert):
        if e < 0 or e >= gate.n_experts:
            continue
        sel = np.nonzero(expert == e)[0]
        Xe = X64[np.asarray(tokens)[tok_idx[sel]]]
        g, ag = gemm_f64(gate, Xe, expert=int(e), threads=threads)
        u, au = gemm_f64(up, Xe, expert=int(e), threads=threads)
        h = swiglu(g, u)
        a_h = 1.1 * np.abs(u) * ag + np.abs(silu(g)) * au
        d, ad = gemm_f64(down, h, expert=int(e), threads=threads)
        _, carried = gemm_f64(down, a_h, expert=int(e), threads=threads)  # sum |w'| a_h
        D[tok_idx[sel], slot_idx[sel]] = d
        AD[tok_idx[sel], slot_idx[sel]] = ad + carried
        valid[tok_idx[sel], slot_idx[sel]] = True
    outs, mags = [], []
    for i, t in enumerate(tokens):
        res64 = None if residual is None else widen(residual[t], res_dtype)
        ks = [k for k in range(top_k) if valid[i, k]]
        if ks:
            out = combine(res64, [float(wts[t][k]) for k in ks], [D[i, k] for k in ks])
            a = sum(abs(float(wts[t][k])) * AD[i, k] for k in ks)
            a = a + (0.0 if res64 is None else np.abs(res64))
        else:
            out = np.zeros(hidden) if res64 is None else res64.copy()
            a = np.zeros(hidden) if res64 is None else np.abs(res64)
        outs.append(out)
        mags.append(a)
    return np.array(outs), np.array(mags)


def gemm_entries(w, X: np.ndarray, t_idx: np.ndarray, o_idx: np.ndarray,
                 x_dtype: str = BF16, round_w: bool = True,
                 threads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Selected entries Y[t_idx[i]][o_idx[i]] of the prefill GEMM."""
    c = np.ascontiguousarray(w.codes, dtype=np.uint32)
    sd = np.ascontiguousarray(widen(w.scales, w.sb_dtype))
    bd = np.ascontiguousarray(widen(w.biases, w.sb_dtype))
    X64 = np.ascontiguousarray(widen(X, x_dtype))
    t_idx = np.ascontiguousarray(t_idx, dtype=np.int64)
    o_idx = np.ascontiguousarray(o_idx, dtype=np.int64)
    if t_idx.shape != o_idx.shape:
        raise ValueError("index arrays must match")
    if t_idx.size and (t_idx.min() < 0 or t_idx.max() >= X64.shape[0]
                       or o_idx.min() < 0 or o_idx.max() >= w.n_out):
        raise IndexError("entry index out of range")
    y = np.empty(t_idx.size, dtype=np.float64)
    a = np.empty(t_idx.size, dtype=np.float64)
    _load().orc_gemm_entries(_p(c), _p(sd), _p(bd), w.n_out, w.k_in, w.group_size, _p(X64),
                             X64.shape[1], _p(t_idx), _p(o_idx), t_idx.size,
                             int(bool(round_w)), _p(y), _p(a), int(threads))
    return y, a
