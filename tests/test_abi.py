"""The C ABI loads, exports every declared symbol, and rejects bad arguments (CPU only).

Every call here fails validation before anything is enqueued, so no kernel is
launched even when a GPU is present; pointers are fake addresses that are
never dereferenced.  The one case that passes validation (and would need a
device) runs only where no GPU exists.
"""
import ctypes
import os
import re

import pytest

import dequant_matmul_int4_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qint4.h")

A = 0x7F0000000000  # fake, 256-byte aligned device-looking addresses


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)  # preprocessor lines (macros)
    return sorted(set(re.findall(r"\b([A-Za-z_0-9]+)\s*\(", text)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q.LIB_PATH):
        pytest.skip("libqint4.so not built")
    return q.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert set(names) == {n for n, _, _ in q.SIGNATURES}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.qint4_abi_version() == 1


def test_status_strings(lib):
    for code in range(10):
        assert lib.qint4_status_string(code)
    assert lib.qint4_status_string(99) == b"unknown status"


def _m(codes=A, scales=A + 0x100000, biases=A + 0x200000, n_out=64, k_in=256, g=64, e=1, sb=1):
    return q.CMatrix(codes, scales, biases, n_out, k_in, g, e, sb, 0)


def _gemv(lib, m, x=A + 0x300000, y=A + 0x400000, xdt=1, ydt=1):
    return lib.qgemv_int4(ctypes.byref(m) if m is not None else None, x, xdt, y, ydt, None)


def _err(lib):
    return lib.qint4_last_error().decode()


def test_gemv_validation(lib):
    assert _gemv(lib, None) == 1
    assert _gemv(lib, _m(codes=0)) == 1
    assert _gemv(lib, _m(), x=0) == 1
    assert _gemv(lib, _m(g=48)) == 2 and "group_size 48" in _err(lib)
    assert _gemv(lib, _m(k_in=96, g=64)) == 2
    assert _gemv(lib, _m(n_out=0)) == 2
    assert _gemv(lib, _m(e=2)) == 2
    assert _gemv(lib, _m(sb=5)) == 3
    assert _gemv(lib, _m(), xdt=7) == 3
    assert _gemv(lib, _m(codes=A + 4)) == 4
    assert _gemv(lib, _m(), x=A + 0x300002) == 4
    assert _gemv(lib, _m(scales=A + 0x100001)) == 4
    m = _m()
    m.reserved = 1
    assert _gemv(lib, m) == 2
    # y overlapping the codes
    assert _gemv(lib, _m(), y=A + 16) == 5 and "overlaps" in _err(lib)


def test_multi_validation(lib):
    ms = (q.CMatrix * 3)(_m(), _m(k_in=512, codes=A + 0x500000), _m(codes=A + 0x600000))
    ys = (ctypes.c_void_p * 3)(A + 0x700000, A + 0x710000, A + 0x720000)
    rc = lib.qgemv_int4_multi(3, ms, A + 0x300000, 1, ys, 1, 0, None)
    assert rc == 2
    msg = _err(lib)
    assert "ws[1].k_in = 512" in msg and "ws[0].k_in = 256" in msg and "64 words" in msg
    assert lib.qgemv_int4_multi(0, ms, A + 0x300000, 1, ys, 1, 0, None) == 2
    assert lib.qgemv_int4_multi(9, ms, A + 0x300000, 1, ys, 1, 0, None) == 2
    ms2 = (q.CMatrix * 2)(_m(), _m(n_out=32, codes=A + 0x500000))
    assert lib.qgemv_int4_multi(2, ms2, A + 0x300000, 1, ys, 1, 1, None) == 2  # swiglu n_out mismatch
    assert lib.qgemv_int4_multi(3, ms, A + 0x300000, 1, ys, 1, 1, None) == 2  # swiglu needs n == 2
    assert lib.qgemv_int4_multi(2, ms2, A + 0x300000, 1, ys, 1, 5, None) == 2  # bad epilogue
    ms3 = (q.CMatrix * 2)(_m(), _m(codes=A + 0x500000))
    ys_alias = (ctypes.c_void_p * 2)(A + 0x700000, A + 0x700010)
    assert lib.qgemv_int4_multi(2, ms3, A + 0x300000, 1, ys_alias, 1, 0, None) == 5


def _moe(lib, top_k=8, ws_bytes=None, ws=A + 0x900000, e=(16, 16, 16), out=A + 0x800000,
         residual=A + 0x880000):
    hidden, inter = 512, 128
    gate = _m(A, A + 0x10000, A + 0x20000, inter, hidden, 64, e[0], 1)
    up = _m(A + 0x100000, A + 0x110000, A + 0x120000, inter, hidden, 64, e[1], 1)
    down = _m(A + 0x200000, A + 0x210000, A + 0x220000, hidden, inter, 64, e[2], 1)
    need = lib.moe_gather_qgemv_int4_workspace_bytes(ctypes.byref(down), max(1, min(top_k, 8)))
    return lib.moe_gather_qgemv_int4(ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down),
                                     A + 0x300000, A + 0x310000, A + 0x320000, top_k, residual, out,
                                     1, ws, need if ws_bytes is None else ws_bytes, None)


def test_moe_validation(lib):
    down = _m(A, A + 0x10000, A + 0x20000, 2048, 768, 64, 128, 1)
    assert lib.moe_gather_qgemv_int4_workspace_bytes(ctypes.byref(down), 8) == 8 * 768 * 4
    assert lib.moe_gather_qgemv_int4_workspace_bytes(ctypes.byref(down), 9) == 0
    assert lib.moe_gather_qgemv_int4_workspace_bytes(None, 8) == 0
    assert _moe(lib, top_k=0) == 2
    assert _moe(lib, top_k=9) == 2
    assert _moe(lib, e=(16, 16, 8)) == 2
    assert _moe(lib, ws_bytes=16) == 6
    assert _moe(lib, ws=0) == 6
    assert _moe(lib, ws=A + 0x900004) == 4
    assert _moe(lib, out=A + 0x300000 + 64) == 5          # out overlaps x
    assert _moe(lib, ws=A + 0x800000 + 64) == 5           # workspace overlaps out


def _gemm(lib, m, T=32, ldx=256, ldy=64, x=A + 0x300000, y=A + 0x400000, ydt=1):
    return lib.qgemm_int4_padT(ctypes.byref(m), x, T, ldx, y, ldy, ydt, None)


def test_gemm_validation(lib):
    assert _gemm(lib, _m(n_out=48)) == 2 and "multiple of 32" in _err(lib)
    assert _gemm(lib, _m(), T=0) == 2
    assert _gemm(lib, _m(), ldx=128) == 2
    assert _gemm(lib, _m(), ldx=260) == 2
    assert _gemm(lib, _m(), ldy=32) == 2
    assert _gemm(lib, _m(), x=A + 0x300008) == 4
    assert _gemm(lib, _m(), y=A + 0x300000 + 128) == 5
    ws = lambda **k: lib.qgemm_int4_padT_ws(ctypes.byref(_m()), A + 0x300000, 32, 256,  # noqa: E731
                                            A + 0x400000, 64, 1, k.get("ws", A + 0x800000),
                                            k.get("n", 1 << 20), None)
    assert ws(ws=A + 0x800040) == 4                          # workspace not 256-byte aligned
    # sizes are device-dependent: without a device the query reports no split
    import torch
    if not torch.cuda.is_available():
        assert lib.qgemm_int4_padT_workspace_bytes(32, 17408, 5120) == 0
    assert lib.qgemm_int4_padT_workspace_bytes(65, 17408, 5120) == 0   # T > 64: no split
    assert lib.qgemm_int4_padT_workspace_bytes(0, 17408, 5120) == 0


def _smallm(lib, m, T=4, ldx=256, x=A + 0x300000, xdt=1, y=A + 0x400000, ydt=1, epi=0, n=1):
    ys = (ctypes.c_void_p * 1)(y)
    return lib.qgemv_int4_smallm(n, ctypes.byref(m), x, xdt, T, ldx, ys, ydt, epi, None)


def test_smallm_validation(lib):
    assert _smallm(lib, _m(), T=0) == 2
    assert _smallm(lib, _m(), T=17) == 2 and "T = 17" in _err(lib)
    assert _smallm(lib, _m(), xdt=0) == 3                      # float32 rows need T = 1
    assert _smallm(lib, _m(), ldx=128) == 2                    # ldx < k_in
    assert _smallm(lib, _m(), ldx=260) == 2                    # ldx not a multiple of 8
    assert _smallm(lib, _m(), y=A + 0x300000 + 2 * 512) == 5   # y overlaps row 2 of x
    assert _smallm(lib, _m(), n=0) == 2
    # rows more than 2 GiB apart: rejected before any path is chosen (k_in 17408 takes the
    # GEMV form, 4096 the MFMA form)
    for k in (17408, 4096):
        assert _smallm(lib, _m(k_in=k), T=2, ldx=1 << 30) == 2 and "2 GiB" in _err(lib)


def _rms(lib, m, n=1, x=A + 0x300000, gamma=A + 0x310000, eps=1e-6, y=A + 0x400000, xdt=1,
         ydt=1, epi=0):
    arr = (q.CMatrix * 2)(m, m)
    ys = (ctypes.c_void_p * 2)(y, y + 0x10000)
    return lib.rms_norm_qgemv_int4(n, arr, x, xdt, gamma, eps, ys, ydt, epi, None)


def test_rms_norm_validation(lib):
    assert _rms(lib, _m(), gamma=0) == 1 and "gamma" in _err(lib)
    assert _rms(lib, _m(), gamma=A + 0x310008) == 4              # gamma misaligned
    assert _rms(lib, _m(), eps=0.0) == 9 and "eps" in _err(lib)
    assert _rms(lib, _m(), eps=-1e-6) == 9
    assert _rms(lib, _m(), eps=float("nan")) == 9
    assert _rms(lib, _m(), eps=float("inf")) == 9
    assert _rms(lib, _m(), y=A + 0x310000 + 64) == 5             # y overlaps gamma
    assert _rms(lib, _m(), n=0) == 2
    assert _rms(lib, _m(), xdt=7) == 3
    assert _rms(lib, _m(), n=1, epi=1) == 2                      # SwiGLU needs two matrices


def _router(lib, logits=A + 0x300000, dt=0, n_tokens=1, n_experts=128, top_k=8, ids=A + 0x400000,
            wts=A + 0x410000):
    return lib.moe_router_topk(logits, dt, n_tokens, n_experts, top_k, ids, wts, None)


def test_router_validation(lib):
    assert _router(lib, logits=0) == 1
    assert _router(lib, ids=0) == 1
    assert _router(lib, dt=5) == 3
    assert _router(lib, top_k=0) == 2
    assert _router(lib, top_k=9) == 2
    assert _router(lib, n_experts=4, top_k=8) == 2 and "n_experts" in _err(lib)
    assert _router(lib, n_experts=4097) == 2
    assert _router(lib, n_tokens=0) == 2
    assert _router(lib, logits=A + 0x300002) == 4          # float32 logits misaligned
    assert _router(lib, ids=A + 0x300000 + 64) == 5        # ids overlap logits
    assert _router(lib, wts=A + 0x400000 + 8) == 5         # wts overlap ids


def test_valid_call_without_device_reports_device_error(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present; fake pointers must never reach a launch")
    assert _gemv(lib, _m()) == 7
    assert "device" in _err(lib)


def _quant(lib, w=A, wdt=0, n_rows=64, k_in=256, g=64, sbdt=1, codes=A + 0x100000,
           scales=A + 0x200000, biases=A + 0x210000):
    return lib.quantize_int4(w, wdt, n_rows, k_in, g, sbdt, codes, scales, biases, None)


def test_quantize_validation(lib):
    assert _quant(lib, w=0) == 1
    assert _quant(lib, biases=0) == 1
    assert _quant(lib, wdt=3) == 3
    assert _quant(lib, sbdt=2) == 3
    assert _quant(lib, g=48) == 2
    assert _quant(lib, k_in=96) == 2 and "k_in" in _err(lib)
    assert _quant(lib, n_rows=0) == 2
    assert _quant(lib, w=A + 8) == 4
    assert _quant(lib, scales=A + 0x200001) == 4
    assert _quant(lib, codes=A + 0x100) == 5                    # codes overlap w
    assert _quant(lib, biases=A + 0x200000 + 64) == 5           # biases overlap scales


def _moep(lib, T=4, top_k=2, E=4, hidden=256, inter=128, x=A + 0x300000, ldx=256, ids=A + 0x310000,
          wts=A + 0x320000, res=0, out=A + 0x400000, odt=1, ws=A + 0x1000000, ws_bytes=1 << 30):
    g = _m(n_out=inter, k_in=hidden, e=E)
    u = q.CMatrix(A + 0x500000, A + 0x600000, A + 0x700000, inter, hidden, 64, E, 1, 0)
    d = q.CMatrix(A + 0x800000, A + 0x900000, A + 0xA00000, hidden, inter, 64, E, 1, 0)
    return lib.moe_prefill_qgemm_int4(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), x, T, ldx,
                                      ids, wts, top_k, res, out, odt, ws, ws_bytes, None)


def test_moe_prefill_validation(lib):
    assert lib.moe_prefill_qgemm_int4_workspace_bytes(0, 8, 128, 2048, 768) == 0
    assert lib.moe_prefill_qgemm_int4_workspace_bytes(1 << 22, 8, 128, 2048, 768) == 0
    assert lib.moe_prefill_qgemm_int4_workspace_bytes(4, 8, 5000, 2048, 768) == 0
    assert lib.moe_prefill_qgemm_int4_workspace_bytes(256, 8, 128, 2048, 768) > 256 * 8 * (2048 + 768) * 4
    assert _moep(lib, x=0) == 1
    assert _moep(lib, top_k=9) == 2
    assert _moep(lib, T=0) == 2
    assert _moep(lib, ldx=200) == 2
    assert _moep(lib, odt=4) == 3
    assert _moep(lib, x=A + 0x300008) == 4
    assert _moep(lib, ws=A + 0x1000010) == 4
    assert _moep(lib, ws_bytes=1024) == 6
    assert _moep(lib, out=A + 0x300000 + 64) == 5                # out overlaps x


def test_route_gather_validation(lib):
    g = _m(n_out=128, k_in=256, e=8)
    u = q.CMatrix(A + 0x500000, A + 0x600000, A + 0x700000, 128, 256, 64, 8, 1, 0)
    d = q.CMatrix(A + 0x800000, A + 0x900000, A + 0xA00000, 256, 128, 64, 8, 1, 0)

    def call(logits=A + 0x300400, ldt=0, top_k=4, ids=A + 0x310000, wts=A + 0x320000, e=8):
        g.n_experts = u.n_experts = d.n_experts = e
        return lib.moe_route_gather_qgemv_int4(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                               A + 0x300000, logits, ldt, top_k, None, A + 0x400000,
                                               1, ids, wts, A + 0x1000000, 1 << 20, None)
    assert call(logits=0) == 1 and "logits" in _err(lib)
    assert call(ldt=5) == 3
    assert call(e=300) == 2 and "256" in _err(lib)
    assert call(top_k=9) == 2
    assert call(logits=A + 0x300402) == 4                   # float32 logits misaligned
    assert call(ids=A + 0x300400 + 8) == 5                  # ids (an output) overlaps logits
    assert call(ids=A + 0x400000) == 5                      # ids overlaps out


def _gemm_multi(lib, ms, x=A + 0x300000, T=100, ldx=None, ys=None, ldys=None, ydt=1):
    arr = (q.CMatrix * len(ms))(*ms)
    ys = ys or [A + 0x1000000 + 0x100000 * i for i in range(len(ms))]
    yp = (ctypes.c_void_p * len(ys))(*ys)
    ld = (ctypes.c_int64 * len(ms))(*(ldys or [m.n_out for m in ms]))
    return lib.qgemm_int4_padT_multi(len(ms), arr, x, T, ldx or ms[0].k_in, yp, ld, ydt, None)


def test_gemm_multi_validation(lib):
    m = [_m(), _m(n_out=32), _m(n_out=96)]
    assert lib.qgemm_int4_padT_multi(0, None, A, 4, 256, None, None, 1, None) == 2
    assert _gemm_multi(lib, [_m(n_out=48)]) == 2 and "multiple of 32" in _err(lib)
    assert _gemm_multi(lib, [_m(), _m(k_in=512)]) == 2 and "packed width" in _err(lib)
    assert _gemm_multi(lib, [_m(), _m(g=32)]) == 2
    assert _gemm_multi(lib, m, T=0) == 2
    assert _gemm_multi(lib, m, ldx=260) == 2
    assert _gemm_multi(lib, m, ldys=[64, 16, 96]) == 2                     # ldy < n_out
    assert _gemm_multi(lib, m, ys=[A + 0x300000, A + 0x2000000, A + 0x2100000]) == 5  # y over x
    assert _gemm_multi(lib, m, ys=[A + 0x2000000, A + 0x2000000 + 64, A + 0x2100000]) == 5
    assert _gemm_multi(lib, m, ydt=4) == 3
