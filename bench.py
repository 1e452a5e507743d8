#!/usr/bin/env python3
"""Throughput of the int4 group-affine GEMV/GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One "step" is one pass of the workload's hot path over one token (T=1 decode
workloads) or one T-row block (prefill).  Inputs live in HBM before timing
starts.  Each step uses the next copy of a rotating pool of distinct weight
sets whose total exceeds 1 GiB, so every step streams its weights from HBM
rather than from the 256 MB last-level cache.  The steps are captured once in
a HIP graph and replayed: at a few microseconds per kernel, host-side launch
cost would otherwise decide the rate.  Timing is HIP events around the replay
on the replay stream, bracketed by device synchronisation.

Workloads (default: qkv):
  single   1024x1024 g64 GEMV, fp32 scales/biases, fp32 x and y
  qkv      q/k/v projections of one bf16 4096-vector (4096/1024/1024 rows), one launch
  rmsqkv   the same launch with the RMSNorm of the input fused in front
  smallm   the q/k/v set for --T tokens (1..8, default 4) in one launch
  dense    gate/up 5120->17408 with SwiGLU (fp32 h), then down 17408->5120
  moe      top-8 of 128 experts, hidden 2048, inter 768, weighted combine + residual;
           each step routes its token's logits inside the gate/up launch (--router gpu: with the
           separate router kernel; --router pre-drawn: host-drawn ids)
  prefill  K=5120, N=17408 dequant GEMM on bf16 MFMA (--T rows, default 256)
  moeprefill  --T tokens through the 128-expert top-8 layer at once (router + sorted GEMMs)
  copy     calibration: a 256 MiB device copy (reference for the HBM byte counters)
  quant    the offline quantiser: 17408x5120 float32 -> g64 codes, bf16 scales/biases

Prints one JSON line.  ``value`` is weight GB/s for the decode workloads and
TFLOP/s for prefill.  ``roofline`` describes the dominant kernel, ``cpu_baseline``
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
POOL_BYTES = 1 << 30

# HBM traffic per step from rocprofv3 counters (one pass with FETCH_SIZE, one
# with WRITE_SIZE, KiB per dispatch, summed over the step's library kernels).
# Scale factors from the copy workload (256 MiB read + 256 MiB written per
# dispatch): FETCH_SIZE read 131,087 KiB -> x2.000; WRITE_SIZE 262,144 KiB -> x1.000.
# Valid only for the kernel sources they were taken with (SOURCE_HASH); any
# change to a kernel source makes the figure null until it is measured again.
TRAFFIC_FETCH_SCALE = 262144.0 / 131087.2
TRAFFIC_WRITE_SCALE = 1.0
TRAFFIC_SOURCE_HASH = "453a4df9fa0418eb"
TRAFFIC_KIB = {  # workload: (FETCH_SIZE KiB, WRITE_SIZE KiB) per step, unscaled
    "qkv_multi_t1": (7004.1, 16.0),
    "rms_qkv_multi_t1": (7056.7, 16.0),
    "dense_ffn_t1": (74536.3, 127.4),
    "moe_top8_t1": (10844.3, 32.1),
    "prefill_gemm_T32": (36086.0, 7616.0),
    "prefill_gemm_T256": (54164.6, 8704.0),
    "prefill_gemm_T1024": (219157.1, 34816.0),
    "prefill_gemm_T4096": (512334.2, 139694.0),
    "moe_prefill_top8_T256": (188023.1, 23585.5),
    "quantize_17408x5120_f32_g64": (174106.0, 48960.0),
}


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: line comments and whitespace do not count, so an edit
    that only touches comments keeps the measured traffic figures valid."""
    import glob
    import hashlib
    import re
    csrc = os.path.join(ROOT, "dequant_matmul_int4_amd", "csrc")
    files = sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h")) +
                   glob.glob(os.path.join(csrc, "*.cpp")))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            code = re.sub(r"//[^\n]*", "", fh.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def traffic_bytes(workload_name: str):
    """Measured HBM bytes per step, or None (not measured, or kernels changed since)."""
    t = TRAFFIC_KIB.get(workload_name)
    if t is None or kernel_source_hash() != TRAFFIC_SOURCE_HASH:
        return None
    return (t[0] * TRAFFIC_FETCH_SCALE + t[1] * TRAFFIC_WRITE_SCALE) * 1024.0
METRIC = "weight GB/s and % of HBM peak for T=1 int4 GEMV; tokens/s-equivalent"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="qkv",
                    choices=["single", "qkv", "rmsqkv", "smallm", "dense", "moe", "moeprefill", "prefill",
                             "quant", "copy"])
    ap.add_argument("--T", type=int, default=None,
                    help="prefill rows (default 256) or small-M tokens (default 4)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-time budget of the CPU oracle sample (0 disables)")
    ap.add_argument("--router", choices=("fused", "gpu", "pre-drawn"), default="fused",
                    help="moe: route each token inside the gate/up launch (default), with the "
                         "separate router kernel, or use pre-drawn ids/weights")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the steps one by one instead of replaying a HIP graph "
                         "(for counter collection; the timing then includes launch gaps)")
    ap.add_argument("--layers", type=int, default=64,
                    help="dense layers per token assumed for tokens/s-equivalent")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# workloads: build a pool, expose step(i) and byte/flop counts
# ---------------------------------------------------------------------------

class Workload:
    name = ""
    launches_per_step = 1
    dominant = ""           # kernel named in the roofline

    def weight_bytes(self) -> int: ...
    def algo_bytes(self) -> int: ...  # bytes the step's kernels must move (weights + activations)
    def step(self, i: int) -> None: ...


def _mat(q, synth, n_out, k_in, sb, seed, n_experts=1, g=64):
    d = synth.torch_matrix(n_out, k_in, g, sb, n_experts=n_experts, seed=seed)
    return q.QInt4Matrix(d["codes"], d["scales"], d["biases"], g)


class Single(Workload):
    name = "single_gemv_t1"
    dominant = "qgemv_kernel (EPI_STORE, f32 x)"

    def __init__(self, q, synth, torch):
        self.q = q
        one = _mat(q, synth, 1024, 1024, "f32", 0)
        self.wb = one.weight_bytes
        self.R = max(1, math.ceil(POOL_BYTES / self.wb))
        self.pool = [one] + [_mat(q, synth, 1024, 1024, "f32", 1 + r) for r in range(self.R - 1)]
        self.x = torch.randn(1024, device="cuda")
        self.y = torch.empty(1024, device="cuda")
        self.config = {"workload": self.name, "n_out": 1024, "in_dim": 1024, "group_size": 64,
                       "sb_dtype": "f32", "x_dtype": "f32", "y_dtype": "f32", "pool_copies": self.R}
        self.dtype = "f32"

    def weight_bytes(self):
        return self.wb

    def algo_bytes(self):
        return self.wb + 1024 * 4 * 2

    def step(self, i):
        self.q.qgemv_int4(self.pool[i % self.R], self.x, self.y)


class QKV(Workload):
    name = "qkv_multi_t1"
    dominant = "qgemv_kernel (EPI_STORE, bf16 x, 3 matrices)"

    def __init__(self, q, synth, torch):
        self.q = q
        outs = (4096, 1024, 1024)
        sets = []
        wb = None
        r = 0
        while True:
            s = [_mat(q, synth, n, 4096, "bf16", 100 * r + i) for i, n in enumerate(outs)]
            sets.append(s)
            wb = sum(m.weight_bytes for m in s)
            r += 1
            if r * wb >= POOL_BYTES:
                break
        self.pool, self.wb, self.R = sets, wb, len(sets)
        self.x = torch.randn(4096, device="cuda").to(torch.bfloat16)
        self.ys = [torch.empty(n, device="cuda", dtype=torch.bfloat16) for n in outs]
        self.config = {"workload": self.name, "in_dim": 4096, "out_dims": list(outs),
                       "group_size": 64, "sb_dtype": "bf16", "x_dtype": "bf16", "y_dtype": "bf16",
                       "pool_copies": self.R}
        self.dtype = "bf16"

    def weight_bytes(self):
        return self.wb

    def algo_bytes(self):
        return self.wb + 4096 * 2 + 6144 * 2

    def step(self, i):
        self.q.qgemv_int4_multi(self.pool[i % self.R], self.x, self.ys)


class SmallM(QKV):
    """The q/k/v projection set for T = 1..8 tokens in one launch (small-M products)."""

    def __init__(self, q, synth, torch, T):
        super().__init__(q, synth, torch)
        self.T = T
        self.name = "qkv_smallm_T%d" % T
        self.dominant = "qgemv_mfma_kernel (bf16 x, 3 matrices, %d tokens)" % T
        self.xT = torch.randn(T, 4096, device="cuda").to(torch.bfloat16)
        self.ysT = [torch.empty(T, n, device="cuda", dtype=torch.bfloat16) for n in (4096, 1024, 1024)]
        self.config = dict(self.config, workload=self.name, T=T)

    def algo_bytes(self):
        return self.wb + self.T * (4096 * 2 + 6144 * 2)

    def step(self, i):
        self.q.qgemv_int4_smallm(self.pool[i % self.R], self.xT, self.ysT)


class RmsQKV(QKV):
    """RMSNorm of the bf16 input fused into the q/k/v projection launch."""

    def __init__(self, q, synth, torch):
        super().__init__(q, synth, torch)
        self.name = "rms_qkv_multi_t1"
        self.dominant = "qgemv_kernel (EPI_STORE, RMSNorm prologue, bf16 x, 3 matrices)"
        self.gamma = (0.5 + torch.rand(4096, device="cuda")).to(torch.bfloat16)
        self.eps = 1e-6
        self.config = dict(self.config, workload=self.name, norm="rmsnorm", eps=self.eps)

    def algo_bytes(self):
        return super().algo_bytes() + 4096 * 2

    def step(self, i):
        self.q.rms_norm_qgemv_int4(self.pool[i % self.R], self.x, self.gamma, self.eps, self.ys)


class Quant(Workload):
    """The offline quantiser on the dense layer's gate matrix: 17408 x 5120 float32 weights
    -> g64 codes with bf16 scales/biases (bytes moved: weights read + packed matrix written)."""
    name = "quantize_17408x5120_f32_g64"
    dominant = "quantize_kernel (min/max group affine)"

    def __init__(self, q, synth, torch):
        self.q = q
        N, K = 17408, 5120
        gen = torch.Generator(device="cuda")
        gen.manual_seed(11)
        one = N * K * 4
        self.R = max(1, math.ceil(POOL_BYTES / one))
        self.pool = [0.02 * torch.randn(N, K, device="cuda", generator=gen) for _ in range(self.R)]
        self.out = q.quantize_int4(self.pool[0], 64, torch.bfloat16)
        self.wb = one
        self.out_bytes = self.out.weight_bytes
        self.config = {"workload": self.name, "n_out": N, "k_in": K, "group_size": 64,
                       "w_dtype": "f32", "sb_dtype": "bf16", "pool_copies": self.R}
        self.dtype = "f32"
        self.torch = torch

    def weight_bytes(self):
        return self.wb

    def algo_bytes(self):
        return self.wb + self.out_bytes

    def step(self, i):
        o = self.out
        self.q._check(self.q.load().quantize_int4(
            self.pool[i % self.R].data_ptr(), self.q.F32, 17408, 5120, 64, self.q.BF16,
            o.codes.data_ptr(), o.scales.data_ptr(), o.biases.data_ptr(),
            self.torch.cuda.current_stream().cuda_stream))


class Copy(Workload):
    """Calibration only: torch's device-to-device copy of a known number of bytes
    (256 MiB read + 256 MiB written per step), the reference for the HBM byte
    counters the roofline's traffic figures are scaled by."""
    name = "copy_256MiB"
    dominant = "torch elementwise copy"

    def __init__(self, q, synth, torch):
        self.nbytes = 256 << 20
        self.src = [torch.empty(self.nbytes // 4, device="cuda").uniform_() for _ in range(4)]
        self.dst = torch.empty_like(self.src[0])
        self.R = 4
        self.config = {"workload": self.name, "bytes_read": self.nbytes, "bytes_written": self.nbytes}
        self.dtype = "f32"

    def weight_bytes(self):
        return self.nbytes

    def algo_bytes(self):
        return 2 * self.nbytes

    def step(self, i):
        self.dst.copy_(self.src[i % self.R])


class Dense(Workload):
    name = "dense_ffn_t1"
    launches_per_step = 2
    dominant = "qgemv_kernel EPI_SWIGLU (gate/up) + EPI_STORE (down)"

    def __init__(self, q, synth, torch):
        self.q = q
        H, I = 5120, 17408
        sets = []
        r = 0
        while True:
            sets.append((_mat(q, synth, I, H, "bf16", 10 * r), _mat(q, synth, I, H, "bf16", 10 * r + 1),
                         _mat(q, synth, H, I, "bf16", 10 * r + 2)))
            r += 1
            wb = sum(m.weight_bytes for m in sets[0])
            if r * wb >= POOL_BYTES:
                break
        self.pool, self.wb, self.R = sets, wb, len(sets)
        self.x = torch.randn(H, device="cuda").to(torch.bfloat16)
        self.h = torch.empty(I, device="cuda")
        self.y = torch.empty(H, device="cuda", dtype=torch.bfloat16)
        self.config = {"workload": self.name, "hidden": H, "inter": I, "group_size": 64,
                       "sb_dtype": "bf16", "x_dtype": "bf16", "h_dtype": "f32", "y_dtype": "bf16",
                       "pool_copies": self.R}
        self.dtype = "bf16"

    def weight_bytes(self):
        return self.wb

    def algo_bytes(self):
        return self.wb + 5120 * 2 + 17408 * 4 * 2 + 5120 * 2

    def step(self, i):
        g, u, d = self.pool[i % self.R]
        self.q.qgemv_int4_multi([g, u], self.x, [self.h], epilogue=self.q.EPI_SWIGLU_PAIR)
        self.q.qgemv_int4(d, self.h, self.y)


class MoE(Workload):
    name = "moe_top8_t1"
    launches_per_step = 3
    dominant = "router_topk + qgemv_kernel EPI_SWIGLU (expert gate/up) + EPI_MOE_DOWN"

    def __init__(self, q, synth, torch, router="fused"):
        self.q = q
        self.router = router
        if router != "fused":
            self.name = "moe_top8_t1_%s_router" % router.replace("-", "")
        if router != "gpu":
            self.launches_per_step = 2
            self.dominant = "qgemv_kernel EPI_SWIGLU (expert gate/up%s) + EPI_MOE_DOWN" % (
                ", routing its token" if router == "fused" else "")
        E, H, I, K = 128, 2048, 768, 8
        stacks = []
        r = 0
        while True:
            stacks.append((_mat(q, synth, I, H, "bf16", 7 * r, n_experts=E),
                           _mat(q, synth, I, H, "bf16", 7 * r + 1, n_experts=E),
                           _mat(q, synth, H, I, "bf16", 7 * r + 2, n_experts=E)))
            r += 1
            if r * sum(m.weight_bytes for m in stacks[0]) >= POOL_BYTES:
                break
        self.pool, self.R = stacks, len(stacks)
        # 1024 router draws: logits ~ N(0,1) -> softmax -> top-8 -> renormalise
        gen = torch.Generator(device="cuda")
        gen.manual_seed(3)
        logits = torch.randn(1024, E, device="cuda", generator=gen)
        self.logits = logits.contiguous()
        p = torch.softmax(logits, dim=-1)
        top = torch.topk(p, K, dim=-1)
        self.ids = top.indices.to(torch.int32).contiguous()
        self.wts = (top.values / top.values.sum(-1, keepdim=True)).float().contiguous()
        self.ids_buf = torch.empty(K, dtype=torch.int32, device="cuda")
        self.wts_buf = torch.empty(K, dtype=torch.float32, device="cuda")
        self.x = torch.randn(H, device="cuda").to(torch.bfloat16)
        self.res = torch.randn(H, device="cuda").to(torch.bfloat16)
        self.out = torch.empty(H, device="cuda", dtype=torch.bfloat16)
        self.ws = torch.empty(q.moe_gather_qgemv_int4_workspace_bytes(I, K), dtype=torch.uint8,
                              device="cuda")
        per_expert = (I * H // 2 + 2 * 2 * I * H // 64)
        self.wb = 3 * K * per_expert            # gate + up + down of the 8 kept experts
        self.config = {"workload": self.name, "n_experts": E, "top_k": K, "hidden": H, "inter": I,
                       "group_size": 64, "sb_dtype": "bf16", "x_dtype": "bf16",
                       "router_draws": 1024, "router": router,
                       "pool_copies": self.R}
        self.dtype = "bf16"

    def weight_bytes(self):
        return self.wb

    def algo_bytes(self):
        return self.wb + 2048 * 2 * 3 + 8 * 768 * 4 * 2 + 8 * 8

    def step(self, i):
        g, u, d = self.pool[i % self.R]
        j = i % self.ids.shape[0]
        if self.router == "fused":  # routed inside the gate/up launch
            self.q.moe_route_gather_qgemv_int4(g, u, d, self.x, self.logits[j], 8, self.ids_buf,
                                               self.wts_buf, self.out, self.ws, residual=self.res)
            return
        if self.router == "gpu":  # route this token's logits on the device, then gather
            self.q.moe_router_topk(self.logits[j], 8, self.ids_buf, self.wts_buf)
            ids, wts = self.ids_buf, self.wts_buf
        else:
            ids, wts = self.ids[j], self.wts[j]
        self.q.moe_gather_qgemv_int4(g, u, d, self.x, ids, wts, self.out, self.ws,
                                     residual=self.res)


class MoEPrefill(Workload):
    """T tokens through the 128-expert top-8 layer at once: device router over the T rows,
    then the expert-sorted gather GEMMs (sort, gate/up + SwiGLU, down, combine)."""
    launches_per_step = 5
    dominant = "moe_gemm_kernel (gate/up SwiGLU, down) on bf16 MFMA"

    def __init__(self, q, synth, torch, T):
        self.q, self.T = q, T
        E, H, I, K = 128, 2048, 768, 8
        self.name = "moe_prefill_top8_T%d" % T
        stacks = []
        r = 0
        while True:
            stacks.append((_mat(q, synth, I, H, "bf16", 7 * r, n_experts=E),
                           _mat(q, synth, I, H, "bf16", 7 * r + 1, n_experts=E),
                           _mat(q, synth, H, I, "bf16", 7 * r + 2, n_experts=E)))
            r += 1
            if r * sum(m.weight_bytes for m in stacks[0]) >= POOL_BYTES:
                break
        self.pool, self.R = stacks, len(stacks)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(6)
        self.logits = torch.randn(T, E, device="cuda", generator=gen)
        self.x = torch.randn(T, H, device="cuda", generator=gen).to(torch.bfloat16)
        self.res = torch.randn(T, H, device="cuda", generator=gen).to(torch.bfloat16)
        self.out = torch.empty(T, H, device="cuda", dtype=torch.bfloat16)
        self.ids = torch.empty(T, K, dtype=torch.int32, device="cuda")
        self.wts = torch.empty(T, K, dtype=torch.float32, device="cuda")
        self.ws = torch.empty(q.moe_prefill_qgemm_int4_workspace_bytes(T, K, E, H, I),
                              dtype=torch.uint8, device="cuda")
        q.moe_router_topk(self.logits, K, self.ids, self.wts)
        touched = int(torch.unique(self.ids).numel())
        per_expert = 3 * (I * H // 2 + 2 * 2 * I * H // 64)
        self.wb = touched * per_expert              # weights of the experts the step touches
        self.flops = 6.0 * T * K * I * H
        self.config = {"workload": self.name, "T": T, "n_experts": E, "top_k": K, "hidden": H,
                       "inter": I, "group_size": 64, "sb_dtype": "bf16", "x_dtype": "bf16",
                       "experts_touched": touched, "router": "gpu", "pool_copies": self.R}
        self.dtype = "bf16"

    def weight_bytes(self):
        return self.wb

    def algo_bytes(self):
        return self.wb + self.T * 2048 * 2 * 3 + self.T * 128 * 4

    def step(self, i):
        g, u, d = self.pool[i % self.R]
        self.q.moe_router_topk(self.logits, 8, self.ids, self.wts)
        self.q.moe_prefill_qgemm_int4(g, u, d, self.x, self.ids, self.wts, self.out, self.ws,
                                      residual=self.res)


class Prefill(Workload):
    dominant = "qgemm_kernel (bf16 MFMA)"

    def __init__(self, q, synth, torch, T):
        self.q = q
        self.T = T
        N, K = 17408, 5120
        self.name = "prefill_gemm_T%d" % T
        one = _mat(q, synth, N, K, "bf16", 0)
        self.wb = one.weight_bytes
        self.R = max(1, math.ceil(POOL_BYTES / self.wb))
        self.pool = [one] + [_mat(q, synth, N, K, "bf16", 1 + r) for r in range(self.R - 1)]
        self.x = torch.randn(T, K, device="cuda").to(torch.bfloat16)
        self.y = torch.empty(T, N, device="cuda", dtype=torch.bfloat16)
        self.flops = 2.0 * T * K * N
        # T <= 64: the K-split stream kernel with its workspace (allocated once, outside
        # the timed steps), plus the partial-sum reduce; longer T: the LDS-tiled kernel
        nb = q.qgemm_int4_padT_workspace_bytes(T, N, K)
        self.ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
        if T <= 64:
            self.dominant = "qgemm_stream_kernel (bf16 MFMA, K split)" + (" + splitk_reduce" if nb else "")
            self.launches_per_step = 2 if nb else 1
        self.config = {"workload": self.name, "T": T, "T_padded": -(-T // 32) * 32, "K": K, "N": N,
                       "group_size": 64, "sb_dtype": "bf16", "x_dtype": "bf16", "y_dtype": "bf16",
                       "pool_copies": self.R, "workspace_bytes": nb}
        self.dtype = "bf16"

    def weight_bytes(self):
        return self.wb

    def algo_bytes(self):
        return self.wb + self.T * 5120 * 2 + self.T * 17408 * 2

    def step(self, i):
        self.q.qgemm_int4_padT_ws(self.pool[i % self.R], self.x, self.y, self.ws)


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def cpu_baseline(workload: str, budget_s: float, T: int):
    import numpy as np

    import oracle
    import synth

    threads = max(1, min(oracle.max_threads(), os.cpu_count() or 1))
    if workload == "single":
        d = synth.single_gemv()
        wb = d["w"].weight_bytes
        fn = lambda: oracle.gemv(d["w"], d["x"], "f32", threads=threads)
        sample = "full 1024x1024 GEMV (seed 0), repeated"
    elif workload == "qkv":
        d = synth.qkv_multi()
        wb = sum(w.weight_bytes for w in d["ws"])
        fn = lambda: oracle.multi(d["ws"], d["x"], "bf16", threads=threads)
        sample = "full q/k/v set (seed 1), repeated"
    elif workload == "rmsqkv":
        d = synth.rms_qkv()
        wb = sum(w.weight_bytes for w in d["ws"])
        fn = lambda: oracle.rms_norm_multi(d["ws"], d["x"], "bf16", d["gamma"], d["eps"],
                                           threads=threads)
        sample = "full RMSNorm + q/k/v set (seed 5), repeated"
    elif workload == "smallm":
        d = synth.qkv_multi()
        wb = sum(w.weight_bytes for w in d["ws"])
        xs = [synth.draw_activation(np.random.default_rng(100 + t), (4096,), "bf16") for t in range(T)]
        fn = lambda: [oracle.multi(d["ws"], x, "bf16", threads=threads) for x in xs]
        sample = "full q/k/v set (seed 1) for %d tokens, repeated" % T
    elif workload == "dense":
        d = synth.dense_layer()
        wb = sum(d[k].weight_bytes for k in ("gate", "up", "down"))
        fn = lambda: oracle.dense_ffn(d["gate"], d["up"], d["down"], d["x"], "bf16", threads=threads)
        sample = "full dense layer (seed 2), repeated"
    elif workload == "moe":
        d = synth.moe_layer()
        per = d["gate"].weight_bytes // d["gate"].n_experts
        wb = 3 * 8 * per

        def fn():
            ids, wts = oracle.router_topk(d["logits"][0], 8)
            return oracle.moe(d["gate"], d["up"], d["down"], d["x"][0], ids, wts.astype(np.float32),
                              d["residual"][0], "bf16", threads=threads)
        sample = "one token of the 128-expert layer (seed 3): router + top-8 experts, repeated"
    elif workload == "moeprefill":
        d = synth.moe_prefill_layer(T=max(T, 2))
        ntok = 2
        pairs = [oracle.router_topk(d["logits"][t].astype(np.float64), 8) for t in range(ntok)]
        ids = np.array([p_[0] for p_ in pairs])
        wts = np.array([p_[1] for p_ in pairs], dtype=np.float32)
        fn = lambda: oracle.moe_prefill(d["gate"], d["up"], d["down"], d["x"][:ntok], ids, wts,
                                        d["residual"][:ntok], threads=threads)
        flops_per_call = 6.0 * ntok * 8 * 768 * 2048
        sample = "%d tokens of the 128-expert layer (seed 6) per call: router + 8 experts each" % ntok
        t0 = time.perf_counter()
        n = 0
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
        return {"value": flops_per_call * n / el / 1e12, "unit": "TFLOP/s", "cores": threads,
                "kind": "oracle", "sample": sample + "; %d calls in %.1f s" % (n, el)}
    elif workload == "quant":
        rng = np.random.default_rng(11)
        rows = 512
        W = synth.draw_float_weights(rng, (rows, 5120), "f32")
        wb = W.nbytes
        fn = lambda: oracle.quantize(W, "f32", 64, "bf16")
        sample = "%d x 5120 rows of float32 weights per call (numpy float32, one thread)" % rows
        threads = 1
    else:
        d = synth.prefill_gemm(T=T)
        rows = 64
        rng = np.random.default_rng(0)
        t_idx = np.repeat(np.arange(min(T, 4)), rows // min(T, 4))
        o_idx = rng.integers(0, d["w"].n_out, t_idx.size)
        fn = lambda: oracle.gemm_entries(d["w"], d["X"], t_idx, o_idx, "bf16", threads=threads)
        flops_per_call = 2.0 * t_idx.size * 5120
        sample = "%d sampled output entries of the T=%d GEMM per call" % (t_idx.size, T)
        t0 = time.perf_counter()
        n = 0
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        el = time.perf_counter() - t0
        return {"value": flops_per_call * n / el / 1e12, "unit": "TFLOP/s", "cores": threads,
                "kind": "oracle", "sample": sample + "; %d calls in %.1f s" % (n, el)}
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": wb * n / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": sample + "; %d calls in %.1f s" % (n, el)}


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.T is None:
        args.T = 4 if args.workload == "smallm" else 256
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import dequant_matmul_int4_amd as q
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    q.load()

    if args.workload == "single":
        wl = Single(q, synth, torch)
    elif args.workload == "qkv":
        wl = QKV(q, synth, torch)
    elif args.workload == "rmsqkv":
        wl = RmsQKV(q, synth, torch)
    elif args.workload == "quant":
        wl = Quant(q, synth, torch)
    elif args.workload == "copy":
        wl = Copy(q, synth, torch)
    elif args.workload == "moeprefill":
        wl = MoEPrefill(q, synth, torch, args.T)
    elif args.workload == "dense":
        wl = Dense(q, synth, torch)
    elif args.workload == "smallm":
        wl = SmallM(q, synth, torch, args.T)
    elif args.workload == "moe":
        wl = MoE(q, synth, torch, router=args.router)
    else:
        wl = Prefill(q, synth, torch, args.T)
    torch.cuda.synchronize()
    print("# workload %s: pool %d copies, %.1f MB weights/step" % (
        wl.name, wl.R, wl.weight_bytes() / 1e6), file=sys.stderr, flush=True)

    K, W = args.steps, args.warmup
    stream = torch.cuda.Stream()
    # eager warm-up call (caches device properties, sets kernel attributes)
    with torch.cuda.stream(stream):
        wl.step(0)
    stream.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    if args.no_graph:
        with torch.cuda.stream(stream):
            for i in range(W):
                wl.step(i)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            ev0.record(stream)
            for i in range(K):
                wl.step(W + i)
            ev1.record(stream)
        torch.cuda.synchronize()
    else:
        g_warm = torch.cuda.CUDAGraph()
        g_main = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_warm, stream=stream):
            for i in range(W):
                wl.step(i)
        with torch.cuda.graph(g_main, stream=stream):
            for i in range(K):
                wl.step(W + i)
        torch.cuda.synchronize()

        with torch.cuda.stream(stream):
            g_warm.replay()
        torch.cuda.synchronize()

        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            ev0.record(stream)
            g_main.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / K
    print("# timed %d steps in %.3f ms" % (K, ms_total), file=sys.stderr, flush=True)

    out = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": W,
           "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded, device-generated pool)",
           "config": wl.config}
    if isinstance(wl, MoEPrefill):
        tflops = wl.flops / (ms_step * 1e-3) / 1e12
        gbs = wl.algo_bytes() / (ms_step * 1e-3) / 1e9
        out.update({"value": tflops, "unit": "TFLOP/s", "tokens_per_s": wl.T * 1e3 / ms_step,
                    "weight_GBps": wl.weight_bytes() / (ms_step * 1e-3) / 1e9})
        # the bound is whichever ideal time is longer: the touched weights at HBM peak or
        # the products at dense bf16 MFMA peak
        t_hbm = wl.algo_bytes() / (HBM_PEAK_GBS * 1e9)
        t_mfma = wl.flops / (BF16_MFMA_PEAK_TFLOPS * 1e12)
        if t_mfma >= t_hbm:
            out["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": tflops / BF16_MFMA_PEAK_TFLOPS,
                               "traffic": traffic_bytes(wl.name), "kernel": wl.dominant,
                               "launches_per_step": wl.launches_per_step}
        else:
            out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": gbs / HBM_PEAK_GBS, "traffic": traffic_bytes(wl.name), "kernel": wl.dominant,
                               "launches_per_step": wl.launches_per_step}
    elif isinstance(wl, Prefill):
        tflops = wl.flops / (ms_step * 1e-3) / 1e12
        gbs = wl.algo_bytes() / (ms_step * 1e-3) / 1e9
        out.update({"value": tflops, "unit": "TFLOP/s",
                    "weight_GBps": wl.weight_bytes() / (ms_step * 1e-3) / 1e9,
                    "mfma_util": tflops / BF16_MFMA_PEAK_TFLOPS})
        # bound: the longer of the ideal times (bytes at HBM peak, products at MFMA peak)
        if wl.flops / (BF16_MFMA_PEAK_TFLOPS * 1e12) >= wl.algo_bytes() / (HBM_PEAK_GBS * 1e9):
            out["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": tflops / BF16_MFMA_PEAK_TFLOPS}
        else:
            out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": gbs / HBM_PEAK_GBS}
        out["roofline"].update({"traffic": traffic_bytes(wl.name), "kernel": wl.dominant,
                                "launches_per_step": wl.launches_per_step})
    else:
        gbs = wl.weight_bytes() / (ms_step * 1e-3) / 1e9
        out.update({"value": gbs, "unit": "GB/s", "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
                    "calls_per_s": 1e3 / ms_step})
        if isinstance(wl, Dense):
            out["tokens_per_s_equiv"] = 1e3 / (ms_step * args.layers)
            out["tokens_per_s_equiv_layers"] = args.layers
        if isinstance(wl, MoE):
            out["tokens_per_s_equiv"] = 1e3 / (ms_step * 40)
            out["tokens_per_s_equiv_layers"] = 40
        if isinstance(wl, SmallM):
            out["tokens_per_call"] = wl.T
        # per launch of the step's kernels (one launch for single/qkv; for the
        # two-launch workloads the pair is timed as one unit)
        ach = wl.algo_bytes() / (ms_step * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS, "traffic": traffic_bytes(wl.name), "kernel": wl.dominant,
                           "launches_per_step": wl.launches_per_step}
    if args.cpu_seconds > 0 and args.workload != "copy":
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds, args.T)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
