"""Python binding of libqint4.so: int4 group-affine GEMV/GEMM for MI355X (gfx950).

Argument marshalling only: every computation runs in the HIP kernels of
``libqint4.so`` through its C ABI (``include/qint4.h``).  PyTorch provides
device memory and the current stream; nothing here computes on the CPU and
there is no fallback path -- if the library is missing, importing the
functions raises.

The names and arguments mirror the C entry points:

* :func:`qgemv_int4`                 -- y = W x (T = 1)
* :func:`qgemv_int4_multi`           -- several projections of one input, one launch;
                                        optional SwiGLU pairing (gate, up -> h)
* :func:`qgemv_int4_smallm`          -- the same for T = 1..8 activation rows at once
* :func:`moe_gather_qgemv_int4`      -- top-K expert gather + SwiGLU + down +
                                        weighted 8-way combine + residual
* :func:`qgemm_int4_padT`            -- prefill GEMM with virtual T padding, bf16 MFMA
* :func:`qgemm_int4_padT_ws`         -- the same with a workspace (K split for T <= 64)
* :func:`moe_router_topk`            -- softmax top-K expert routing on the device
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch  # must load before libqint4.so so both share torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqint4.so")

F32 = 0
BF16 = 1
EPI_NONE = 0
EPI_SWIGLU_PAIR = 1
MULTI_MAX = 8
TOPK_MAX = 8

STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_DTYPE", 4: "ERR_ALIGN",
          5: "ERR_ALIAS", 6: "ERR_WORKSPACE", 7: "ERR_DEVICE", 8: "ERR_LAUNCH",
          9: "ERR_VALUE"}


class Int4Error(RuntimeError):
    """A non-OK qint4_status; ``status`` is its name, the message the library's detail."""

    def __init__(self, code: int, message: str):
        self.code = int(code)
        self.status = STATUS.get(int(code), str(code))
        super().__init__("%s: %s" % (self.status, message))


class CMatrix(ctypes.Structure):
    """Mirror of ``qint4_matrix``."""

    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("n_out", ctypes.c_int64),
                ("k_in", ctypes.c_int64), ("group_size", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("sb_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class CGemvForm(ctypes.Structure):
    """qint4_gemv_form of include/qint4.h."""
    _fields_ = [("kernel", ctypes.c_int32), ("tokens", ctypes.c_int32),
                ("launches", ctypes.c_int64), ("grid", ctypes.c_int64), ("tasks", ctypes.c_int64),
                ("waves", ctypes.c_int32), ("lanes", ctypes.c_int32),
                ("rows_per_task", ctypes.c_int32), ("steps_per_task", ctypes.c_int32),
                ("busiest_wave_steps", ctypes.c_int64), ("ring_depth", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}
        d["kernel"] = {FORM_RING: "ring", FORM_MFMA: "mfma", FORM_XS: "xs"}[self.kernel]
        return d


FORM_RING = 0
FORM_MFMA = 1
FORM_XS = 2
CALL_QGEMV = 0
CALL_RMS_NORM = 1
CALL_SMALLM = 2

_lib = None

# (name, restype, argtypes) of every symbol include/qint4.h declares
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
SIGNATURES = [
    ("qgemv_int4", _I32, [ctypes.POINTER(CMatrix), _P, _I32, _P, _I32, _P]),
    ("qgemv_int4_multi", _I32, [_I32, ctypes.POINTER(CMatrix), _P, _I32,
                                ctypes.POINTER(ctypes.c_void_p), _I32, _I32, _P]),
    ("qgemv_int4_smallm", _I32, [_I32, ctypes.POINTER(CMatrix), _P, _I32, _I64, _I64,
                                 ctypes.POINTER(ctypes.c_void_p), _I32, _I32, _P]),
    ("rms_norm_qgemv_int4", _I32, [_I32, ctypes.POINTER(CMatrix), _P, _I32, _P, ctypes.c_float,
                                   ctypes.POINTER(ctypes.c_void_p), _I32, _I32, _P]),
    ("moe_gather_qgemv_int4_workspace_bytes", ctypes.c_size_t, [ctypes.POINTER(CMatrix), _I32]),
    ("moe_gather_qgemv_int4", _I32, [ctypes.POINTER(CMatrix), ctypes.POINTER(CMatrix),
                                     ctypes.POINTER(CMatrix), _P, _P, _P, _I32, _P, _P, _I32,
                                     _P, ctypes.c_size_t, _P]),
    ("moe_gather_qgemv_int4_noalloc", _I32, [ctypes.POINTER(CMatrix), ctypes.POINTER(CMatrix),
                                             ctypes.POINTER(CMatrix), _P, _P, _P, _I32, _P, _P,
                                             _I32, _P]),
    ("moe_route_gather_qgemv_int4", _I32, [ctypes.POINTER(CMatrix), ctypes.POINTER(CMatrix),
                                           ctypes.POINTER(CMatrix), _P, _P, _I32, _I32, _P, _P, _I32,
                                           _P, _P, _P, ctypes.c_size_t, _P]),
    ("qgemm_int4_padT", _I32, [ctypes.POINTER(CMatrix), _P, _I64, _I64, _P, _I64, _I32, _P]),
    ("qgemm_int4_padT_ws", _I32, [ctypes.POINTER(CMatrix), _P, _I64, _I64, _P, _I64, _I32, _P,
                                  ctypes.c_size_t, _P]),
    ("qgemm_int4_padT_workspace_bytes", ctypes.c_size_t, [_I64, _I64, _I64]),
    ("qgemm_int4_padT_multi", _I32, [_I32, ctypes.POINTER(CMatrix), _P, _I64, _I64,
                                     ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int64),
                                     _I32, _P]),
    ("moe_router_topk", _I32, [_P, _I32, _I64, _I32, _I32, _P, _P, _P]),
    ("moe_prefill_qgemm_int4_workspace_bytes", ctypes.c_size_t, [_I64, _I32, _I32, _I64, _I64]),
    ("moe_prefill_qgemm_int4", _I32, [ctypes.POINTER(CMatrix), ctypes.POINTER(CMatrix),
                                      ctypes.POINTER(CMatrix), _P, _I64, _I64, _P, _P, _I32, _P, _P,
                                      _I32, _P, ctypes.c_size_t, _P]),
    ("quantize_int4", _I32, [_P, _I32, _I64, _I64, _I32, _I32, _P, _P, _P, _P]),
    ("qint4_plan_qgemv", _I32, [_I32, _I32, ctypes.POINTER(ctypes.c_int64), _I64, _I32, _I32, _I64,
                                _I32, _I32, ctypes.POINTER(CGemvForm)]),
    ("qint4_plan_moe_gather", _I32, [_I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32,
                                     ctypes.POINTER(CGemvForm)]),
    ("qint4_status_string", ctypes.c_char_p, [_I32]),
    ("qint4_last_error", ctypes.c_char_p, []),
    ("qint4_abi_version", _I32, []),
]


def load(path: Optional[str] = None):
    """Load libqint4.so (built in-tree by ``build.py``) and declare its prototypes."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError("libqint4.so is not built (%s); run python -m dequant_matmul_int4_amd.build" % p)
    lib = ctypes.CDLL(p)
    for name, res, args in SIGNATURES:
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(code: int):
    if code != 0:
        msg = load().qint4_last_error()
        raise Int4Error(code, msg.decode() if msg else "")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


class QInt4Matrix:
    """Packed int4 matrix (or expert stack) in device memory.

    codes:  int32 tensor [E?][n_out][k_in/8] (the u32 words' bits)
    scales, biases: float32 or bfloat16 tensors [E?][n_out][k_in/group_size]
    """

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                 group_size: int):
        if codes.dtype not in (torch.int32, torch.uint32):
            raise TypeError("codes must be int32 (u32 bit patterns)")
        if scales.dtype != biases.dtype or scales.shape != biases.shape:
            raise ValueError("scales and biases must share dtype and shape")
        if codes.dim() not in (2, 3) or scales.dim() != codes.dim():
            raise ValueError("codes/scales must be [n_out, *] or [E, n_out, *]")
        self.codes, self.scales, self.biases = codes, scales, biases
        self.group_size = int(group_size)
        self.n_experts = codes.shape[0] if codes.dim() == 3 else 1
        self.n_out = codes.shape[-2]
        self.k_in = codes.shape[-1] * 8
        self.sb_dtype = _dt(scales)

    @property
    def weight_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.scales, self.biases))

    def c(self) -> CMatrix:
        return CMatrix(_dev(self.codes, "codes"), _dev(self.scales, "scales"),
                       _dev(self.biases, "biases"), self.n_out, self.k_in, self.group_size,
                       self.n_experts, self.sb_dtype, 0)


def qgemv_int4(w: QInt4Matrix, x: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """y = W x.  x: [k_in] float32/bfloat16; y: [n_out] float32/bfloat16."""
    cm = w.c()
    _check(load().qgemv_int4(ctypes.byref(cm), _dev(x, "x"), _dt(x), _dev(y, "y"), _dt(y),
                             _stream(stream)))


def qgemv_int4_multi(ws: Sequence[QInt4Matrix], x: torch.Tensor, ys: Sequence[torch.Tensor],
                     epilogue: int = EPI_NONE, stream=None) -> None:
    """ys[i] = W_i x in one launch; with EPI_SWIGLU_PAIR, ys[0] = silu(W_0 x) * (W_1 x)."""
    n = len(ws)
    arr = (CMatrix * max(n, 1))(*[w.c() for w in ws])
    if len(ys) < 1:
        raise ValueError("need at least one output")
    ptrs = (ctypes.c_void_p * max(len(ys), n))(*[_dev(y, "ys[%d]" % i) for i, y in enumerate(ys)])
    y_dt = _dt(ys[0])
    if any(_dt(y) != y_dt for y in ys):
        raise TypeError("all outputs must share one dtype")
    _check(load().qgemv_int4_multi(n, arr, _dev(x, "x"), _dt(x), ptrs, y_dt, int(epilogue),
                                   _stream(stream)))


def rms_norm_qgemv_int4(ws: Sequence[QInt4Matrix], x: torch.Tensor, gamma: torch.Tensor, eps: float,
                        ys: Sequence[torch.Tensor], epilogue: int = EPI_NONE, stream=None) -> None:
    """ys[i] = W_i (x * gamma / sqrt(mean(x^2) + eps)) in one launch (EPI_SWIGLU_PAIR as in
    qgemv_int4_multi).  x, gamma: [k_in], one dtype (float32 or bfloat16)."""
    n = len(ws)
    arr = (CMatrix * max(n, 1))(*[w.c() for w in ws])
    if len(ys) < 1:
        raise ValueError("need at least one output")
    if gamma.dtype != x.dtype:
        raise TypeError("gamma must have x's dtype")
    ptrs = (ctypes.c_void_p * max(len(ys), n))(*[_dev(y, "ys[%d]" % i) for i, y in enumerate(ys)])
    y_dt = _dt(ys[0])
    if any(_dt(y) != y_dt for y in ys):
        raise TypeError("all outputs must share one dtype")
    _check(load().rms_norm_qgemv_int4(n, arr, _dev(x, "x"), _dt(x), _dev(gamma, "gamma"),
                                      float(eps), ptrs, y_dt, int(epilogue), _stream(stream)))


def quantize_int4(w: torch.Tensor, group_size: int = 64, sb_dtype: torch.dtype = torch.bfloat16,
                  stream=None) -> QInt4Matrix:
    """Quantise float weights [n_out][k_in] (or an expert stack [E][n_out][k_in]) on the device
    into a new QInt4Matrix (codes from the stored scale/bias; see quantize_int4 in qint4.h)."""
    if w.dim() not in (2, 3):
        raise ValueError("w must be [n_out, k_in] or [E, n_out, k_in]")
    k_in = w.shape[-1]
    if k_in % group_size:
        raise ValueError("k_in must be a multiple of group_size")
    lead = tuple(w.shape[:-1])
    codes = torch.empty(lead + (k_in // 8,), dtype=torch.int32, device=w.device)
    scales = torch.empty(lead + (k_in // group_size,), dtype=sb_dtype, device=w.device)
    biases = torch.empty_like(scales)
    n_rows = math.prod(lead)
    _check(load().quantize_int4(_dev(w, "w"), _dt(w), n_rows, k_in, int(group_size), _dt(scales),
                                codes.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                                _stream(stream)))
    return QInt4Matrix(codes, scales, biases, group_size)


def moe_prefill_qgemm_int4_workspace_bytes(T: int, top_k: int, n_experts: int, hidden: int,
                                           inter: int) -> int:
    return int(load().moe_prefill_qgemm_int4_workspace_bytes(int(T), int(top_k), int(n_experts),
                                                              int(hidden), int(inter)))


def moe_prefill_qgemm_int4(gate: QInt4Matrix, up: QInt4Matrix, down: QInt4Matrix, x: torch.Tensor,
                           ids: torch.Tensor, wts: torch.Tensor, out: torch.Tensor,
                           workspace: torch.Tensor, residual: Optional[torch.Tensor] = None,
                           stream=None) -> None:
    """out[t] = residual[t] + sum_k wts[t,k] * down[ids[t,k]] (silu(gate[.] x[t]) * up[.] x[t])
    for all T rows of x ([T][ldx] bf16) at once; ids int32/uint32 [T][top_k], wts float32 [T][top_k],
    out (and residual) [T][hidden] float32/bfloat16, workspace of
    moe_prefill_qgemm_int4_workspace_bytes(...) bytes."""
    if x.dim() != 2 or x.stride(1) != 1 or x.device.type != "cuda":
        raise ValueError("x must be a 2-D device tensor [T][ldx] with contiguous rows")
    if ids.dtype not in (torch.int32, torch.uint32) or ids.dim() != 2 or ids.shape[0] != x.shape[0]:
        raise ValueError("ids must be int32/uint32 [T][top_k]")
    if wts.dtype != torch.float32 or wts.shape != ids.shape:
        raise ValueError("wts must be float32 of ids' shape")
    if residual is not None and residual.dtype != out.dtype:
        raise TypeError("residual must have out's dtype")
    g, u, d = gate.c(), up.c(), down.c()
    _check(load().moe_prefill_qgemm_int4(
        ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), x.data_ptr(), x.shape[0], x.stride(0),
        _dev(ids, "ids"), _dev(wts, "wts"), ids.shape[1],
        None if residual is None else _dev(residual, "residual"), _dev(out, "out"), _dt(out),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_route_gather_qgemv_int4(gate: QInt4Matrix, up: QInt4Matrix, down: QInt4Matrix,
                                x: torch.Tensor, logits: torch.Tensor, top_k: int,
                                ids: torch.Tensor, wts: torch.Tensor, out: torch.Tensor,
                                workspace: torch.Tensor, residual: Optional[torch.Tensor] = None,
                                stream=None) -> None:
    """moe_router_topk + moe_gather_qgemv_int4 for one token, routed inside the gate/up launch.
    logits: [n_experts] float32/bfloat16 (n_experts <= 256); ids (int32/uint32) and wts
    (float32) [top_k] are outputs."""
    if ids.dtype not in (torch.int32, torch.uint32) or wts.dtype != torch.float32:
        raise TypeError("ids must be int32/uint32 and wts float32")
    if residual is not None and residual.dtype != x.dtype:
        raise TypeError("residual must have x's dtype")
    g, u, d = gate.c(), up.c(), down.c()
    _check(load().moe_route_gather_qgemv_int4(
        ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), _dev(x, "x"), _dev(logits, "logits"),
        _dt(logits), int(top_k), None if residual is None else _dev(residual, "residual"),
        _dev(out, "out"), _dt(x), _dev(ids, "ids"), _dev(wts, "wts"), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


SMALLM_MAX = 16  # QINT4_SMALLM_MAX of include/qint4.h


def qgemv_int4_smallm(ws: Sequence[QInt4Matrix], x: torch.Tensor, ys: Sequence[torch.Tensor],
                      epilogue: int = EPI_NONE, stream=None) -> None:
    """ys[i][t] = W_i x[t] for T = x.shape[0] rows (1..16) sharing the weight stream; with
    EPI_SWIGLU_PAIR, ys[0][t] = silu(W_0 x[t]) * (W_1 x[t]).

    x: [T][ldx] bfloat16 (row stride may exceed k_in; float32 only for T = 1);
    ys[i]: [T][n_out_i] contiguous, float32 or bfloat16.
    """
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D [T][ldx] with contiguous rows")
    if x.device.type != "cuda":
        raise ValueError("x must be a device tensor")
    n = len(ws)
    arr = (CMatrix * max(n, 1))(*[w.c() for w in ws])
    if len(ys) < 1:
        raise ValueError("need at least one output")
    ptrs = (ctypes.c_void_p * max(len(ys), n))(*[_dev(y, "ys[%d]" % i) for i, y in enumerate(ys)])
    y_dt = _dt(ys[0])
    if any(_dt(y) != y_dt for y in ys):
        raise TypeError("all outputs must share one dtype")
    _check(load().qgemv_int4_smallm(n, arr, x.data_ptr(), _dt(x), x.shape[0], x.stride(0), ptrs,
                                    y_dt, int(epilogue), _stream(stream)))


def moe_gather_qgemv_int4_workspace_bytes(down: QInt4Matrix, top_k: int) -> int:
    """Workspace bytes of a moe_gather_qgemv_int4 call with this down stack and top_k."""
    m = down.c()
    return int(load().moe_gather_qgemv_int4_workspace_bytes(ctypes.byref(m), int(top_k)))


def moe_gather_qgemv_int4(gate: QInt4Matrix, up: QInt4Matrix, down: QInt4Matrix,
                          x: torch.Tensor, ids: torch.Tensor, wts: torch.Tensor,
                          out: torch.Tensor, workspace: torch.Tensor,
                          residual: Optional[torch.Tensor] = None, stream=None) -> None:
    """out = residual + sum_k wts[k] * down[ids[k]] (silu(gate[ids[k]] x) * up[ids[k]] x).

    ids: int32/uint32 [top_k] on the device; wts: float32 [top_k]; workspace: any
    device tensor of at least moe_gather_qgemv_int4_workspace_bytes(down, top_k) bytes.
    """
    if ids.dtype not in (torch.int32, torch.uint32):
        raise TypeError("ids must be int32/uint32")
    if wts.dtype != torch.float32:
        raise TypeError("wts must be float32")
    if ids.numel() != wts.numel():
        raise ValueError("ids and wts must have the same length")
    g, u, d = gate.c(), up.c(), down.c()
    res_p = _dev(residual, "residual") if residual is not None else None
    if residual is not None and residual.dtype != out.dtype:
        raise TypeError("residual and out must share a dtype")
    if x.dtype != out.dtype:
        raise TypeError("x and out must share a dtype")
    _check(load().moe_gather_qgemv_int4(
        ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), _dev(x, "x"), _dev(ids, "ids"),
        _dev(wts, "wts"), ids.numel(), res_p, _dev(out, "out"), _dt(out),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_gather_qgemv_int4_noalloc(gate: QInt4Matrix, up: QInt4Matrix, down: QInt4Matrix,
                                  x: torch.Tensor, ids: torch.Tensor, wts: torch.Tensor,
                                  out: torch.Tensor, residual: Optional[torch.Tensor] = None,
                                  stream=None) -> None:
    """moe_gather_qgemv_int4 with the library's static per-device scratch instead of a
    workspace (for callers that cannot allocate); top_k * inter * 4 bytes must fit in
    NOALLOC_SCRATCH_BYTES.  Calls that overlap on one GPU race on that scratch."""
    if ids.dtype not in (torch.int32, torch.uint32):
        raise TypeError("ids must be int32/uint32")
    if wts.dtype != torch.float32:
        raise TypeError("wts must be float32")
    if ids.numel() != wts.numel():
        raise ValueError("ids and wts must have the same length")
    g, u, d = gate.c(), up.c(), down.c()
    res_p = _dev(residual, "residual") if residual is not None else None
    if residual is not None and residual.dtype != out.dtype:
        raise TypeError("residual and out must share a dtype")
    if x.dtype != out.dtype:
        raise TypeError("x and out must share a dtype")
    _check(load().moe_gather_qgemv_int4_noalloc(
        ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), _dev(x, "x"), _dev(ids, "ids"),
        _dev(wts, "wts"), ids.numel(), res_p, _dev(out, "out"), _dt(out), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 1 << 20  # QINT4_NOALLOC_SCRATCH_BYTES of include/qint4.h


def _gemm_args(x: torch.Tensor, y: torch.Tensor) -> None:
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if x.dim() != 2 or y.dim() != 2 or x.shape[0] != y.shape[0]:
        raise ValueError("x and y must be 2-D with the same number of rows")
    if x.stride(1) != 1 or y.stride(1) != 1:
        raise ValueError("rows of x and y must be contiguous")
    if x.device.type != "cuda" or y.device.type != "cuda":
        raise ValueError("x and y must be device tensors")


def qgemm_int4_padT(w: QInt4Matrix, x: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """Y[t] = bf16(W) X[t] for t < T.  x: bfloat16 [T][ldx] (row stride may exceed k_in);
    y: [T][ldy] float32/bfloat16."""
    _gemm_args(x, y)
    cm = w.c()
    _check(load().qgemm_int4_padT(ctypes.byref(cm), x.data_ptr(), x.shape[0], x.stride(0),
                                  y.data_ptr(), y.stride(0), _dt(y), _stream(stream)))


def qgemm_int4_padT_multi(ws: Sequence[QInt4Matrix], x: torch.Tensor, ys: Sequence[torch.Tensor],
                          stream=None) -> None:
    """Y_i[t] = bf16(W_i) X[t] for t < T and every matrix i, in one launch.  x: bfloat16
    [T][ldx]; ys[i]: [T][ldy_i] float32/bfloat16, all of one dtype."""
    if len(ws) != len(ys) or not ws:
        raise ValueError("one output per matrix")
    for y in ys:
        _gemm_args(x, y)
    if len({y.dtype for y in ys}) != 1:
        raise TypeError("all outputs must share a dtype")
    arr = (CMatrix * len(ws))(*[w.c() for w in ws])
    yp = (ctypes.c_void_p * len(ys))(*[y.data_ptr() for y in ys])
    ld = (ctypes.c_int64 * len(ys))(*[y.stride(0) for y in ys])
    _check(load().qgemm_int4_padT_multi(len(ws), arr, x.data_ptr(), x.shape[0], x.stride(0), yp,
                                        ld, _dt(ys[0]), _stream(stream)))


def qgemm_int4_padT_workspace_bytes(T: int, n_out: int, k_in: int) -> int:
    """Workspace bytes for the full K split of qgemm_int4_padT_ws on the current device."""
    return int(load().qgemm_int4_padT_workspace_bytes(int(T), int(n_out), int(k_in)))


def qgemm_int4_padT_ws(w: QInt4Matrix, x: torch.Tensor, y: torch.Tensor,
                       workspace: Optional[torch.Tensor], stream=None) -> None:
    """qgemm_int4_padT with a scratch workspace (device tensor, 256-byte aligned, or None):
    for T <= 64 the K range is split over workgroups into float32 partials."""
    _gemm_args(x, y)
    cm = w.c()
    ws_p = _dev(workspace, "workspace") if workspace is not None else None
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().qgemm_int4_padT_ws(ctypes.byref(cm), x.data_ptr(), x.shape[0], x.stride(0),
                                     y.data_ptr(), y.stride(0), _dt(y), ws_p, ws_n,
                                     _stream(stream)))


def moe_router_topk(logits: torch.Tensor, top_k: int, ids: torch.Tensor, wts: torch.Tensor,
                    stream=None) -> None:
    """ids[t], wts[t] = top-K experts of softmax(logits[t]) and their renormalised weights.

    logits: float32/bfloat16 [n_experts] or [n_tokens][n_experts]; ids: int32/uint32 and
    wts: float32, each [top_k] or [n_tokens][top_k] (all on the device).
    """
    if ids.dtype not in (torch.int32, torch.uint32):
        raise TypeError("ids must be int32/uint32")
    if wts.dtype != torch.float32:
        raise TypeError("wts must be float32")
    n_experts = logits.shape[-1]
    n_tokens = logits.numel() // max(n_experts, 1)
    if ids.numel() != n_tokens * top_k or wts.numel() != n_tokens * top_k:
        raise ValueError("ids and wts must hold n_tokens * top_k elements")
    _check(load().moe_router_topk(_dev(logits, "logits"), _dt(logits), n_tokens, n_experts,
                                  int(top_k), _dev(ids, "ids"), _dev(wts, "wts"),
                                  _stream(stream)))


__all__ = ["QInt4Matrix", "Int4Error", "qgemv_int4", "qgemv_int4_multi", "qgemv_int4_smallm",
           "moe_gather_qgemv_int4", "moe_gather_qgemv_int4_workspace_bytes", "qgemm_int4_padT",
           "qgemm_int4_padT_ws", "qgemm_int4_padT_workspace_bytes", "qgemm_int4_padT_multi",
           "moe_router_topk", "rms_norm_qgemv_int4", "quantize_int4",
           "moe_prefill_qgemm_int4", "moe_prefill_qgemm_int4_workspace_bytes",
           "moe_route_gather_qgemv_int4", "moe_gather_qgemv_int4_noalloc", "NOALLOC_SCRATCH_BYTES",
           "load", "F32", "BF16", "EPI_NONE", "EPI_SWIGLU_PAIR", "LIB_PATH", "SIGNATURES"]


_DTYPE_CODES = {"f32": 0, "bf16": 1, torch.float32: 0, torch.bfloat16: 1}


def plan_qgemv(n_outs: Sequence[int], k_in: int, group_size: int = 64, x_dtype="bf16", T: int = 1,
               epilogue: int = EPI_NONE, call: int = CALL_QGEMV, n_cu: int = 0) -> dict:
    """The launch form of a qgemv_int4 / _multi (call CALL_QGEMV), rms_norm_qgemv_int4
    (CALL_RMS_NORM) or qgemv_int4_smallm (CALL_SMALLM) call with these shapes, planned by
    the library's own planner (host only; n_cu = 0 plans for the current device)."""
    n = len(n_outs)
    arr = (ctypes.c_int64 * max(n, 1))(*[int(v) for v in n_outs])
    form = CGemvForm()
    _check(load().qint4_plan_qgemv(int(call), n, arr, int(k_in), int(group_size),
                                   _DTYPE_CODES[x_dtype], int(T), int(epilogue), int(n_cu),
                                   ctypes.byref(form)))
    return form.as_dict()


def plan_moe_gather(hidden: int, inter: int, top_k: int, group_size: int = 64, act_dtype="bf16",
                    routed: bool = False, residual: bool = True, n_cu: int = 0):
    """(gate/up form, down form) of a moe_gather_qgemv_int4 (routed: moe_route_gather_qgemv_int4)
    call with these shapes, planned by the library's own planner (host only)."""
    forms = (CGemvForm * 2)()
    _check(load().qint4_plan_moe_gather(int(hidden), int(inter), int(top_k), int(group_size),
                                        _DTYPE_CODES[act_dtype], int(bool(routed)),
                                        int(bool(residual)), int(n_cu), forms))
    return forms[0].as_dict(), forms[1].as_dict()
