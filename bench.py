#!/usr/bin/env python3
"""Throughput of the int4 group-affine GEMV/GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One "step" is one pass of the workload's hot path over one token (T=1 decode
workloads) or one T-row block (prefill).  Inputs live in HBM before timing
starts.  Each step uses the next copy of a rotating pool of distinct weight
sets whose total exceeds 1 GiB, so every step streams its weights from HBM
rather than from the 256 MB last-level cache.  The W warm-up steps and the K
timed steps are captured as two HIP graphs (at a few microseconds per kernel,
host-side launch cost would otherwise decide the rate).  One repetition is:
device synchronisation, the warm-up graph, an event, the K-step graph, an
event, device synchronisation -- so the timed region holds exactly the K steps
and the warm-up keeps the GPU busy while the timed graph is submitted.  The
line reports the median over 5 repetitions.

Each kernel launch of a step is also timed on its own (K launches of it in a
graph, same repetitions): ``roofline`` is the dominant kernel's algorithmic
bytes (or flops) per launch over its median launch duration.  Next to it, the
same run measures a stream-read ceiling (a plain read kernel over an equal
number of bytes, from a 1 GiB rotating pool) and, for the prefill GEMM,
torch's bf16 matmul of the same shape.

Workloads (default: dense):
  single   1024x1024 g64 GEMV, fp32 scales/biases, fp32 x and y
  qkv      q/k/v projections of one bf16 4096-vector (4096/1024/1024 rows), one launch
  qkvprefill  the q/k/v projections of --T rows in one multi-matrix GEMM launch
  rmsqkv   the same launch with the RMSNorm of the input fused in front
  smallm   the q/k/v set for --T tokens (1..16, default 4) in one call
  dense    gate/up 5120->17408 with SwiGLU (fp32 h), then down 17408->5120
  moe      top-8 of 128 experts, hidden 2048, inter 768, weighted combine + residual;
           each step routes its token's logits inside the gate/up launch (--router gpu: with the
           separate router kernel; --router pre-drawn: host-drawn ids)
  prefill  K=5120, N=17408 dequant GEMM on bf16 MFMA (--T rows, default 256)
  moeprefill  --T tokens through the 128-expert top-8 layer at once (router + sorted GEMMs)
  copy     calibration: a 256 MiB device copy (reference for the HBM byte counters)
  quant    the offline quantiser: 17408x5120 float32 -> g64 codes, bf16 scales/biases

Prints one JSON line.  ``value`` is weight GB/s for the decode workloads and
TFLOP/s for prefill.  ``cpu_baseline`` is the fp64 CPU oracle timed on a
bounded sample of the same workload, on one core and on all cores.
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

# HBM traffic from rocprofv3 counters (one pass with FETCH_SIZE, one with
# WRITE_SIZE, KiB per dispatch, calls launched one by one with --no-graph) for
# the unit the roofline describes: the dominant kernel where a step has several
# timed parts (dense: the gate/up launch), else the step's library kernels
# summed.  Scale factors from the copy workload (256 MiB read + 256 MiB written
# per dispatch): FETCH_SIZE read 131,084 KiB -> x2.000; WRITE_SIZE 262,144 KiB
# -> x1.000.  Each figure is valid only for the sources it was taken with: the
# hash covers the listed kernel sources (comments and whitespace excluded), and
# any change to them makes the figure null until it is measured again.
TRAFFIC_FETCH_SCALE = 262144.0 / 131084.1
TRAFFIC_WRITE_SCALE = 1.0
GEMV_SRC = ("kernels.h", "api.cpp", "qgemv.hip", "qgemv_xs.hip", "topk_wave.h")
SMALLM_SRC = ("kernels.h", "api.cpp", "qgemv_mfma.hip")
STREAM_SRC = ("kernels.h", "api.cpp", "qgemm_stream.hip")
GEMM_SRC = ("kernels.h", "api.cpp", "qgemm.hip")
MOEP_SRC = ("kernels.h", "api.cpp", "moe_prefill.hip", "router.hip", "topk_wave.h")
QUANT_SRC = ("kernels.h", "api.cpp", "quant.hip")
TRAFFIC = {  # workload: (sources, source hash, FETCH_SIZE KiB, WRITE_SIZE KiB), unscaled
    "dense_ffn_t1": (GEMV_SRC, "4854a9b2a3d12933", 49668.0, 88.7),
    "moe_top8_t1": (GEMV_SRC, "4854a9b2a3d12933", 10802.8, 32.1),
    "qkv_multi_t1": (GEMV_SRC, "4854a9b2a3d12933", 6997.6, 16.0),
    "rms_qkv_multi_t1": (GEMV_SRC, "4854a9b2a3d12933", 7057.1, 16.0),
    "qkv_smallm_T4": (SMALLM_SRC, "1945b2914096cd9e", 7086.6, 48.0),
    "qkv_smallm_T16": (SMALLM_SRC, "1945b2914096cd9e", 7502.6, 192.0),
    "prefill_gemm_T32": (STREAM_SRC, "fd3edbcac088e1cd", 36112.7, 7616.0),
    "prefill_gemm_T256": (GEMM_SRC, "111d8436f4badcf5", 34848.3, 8704.0),
    "prefill_gemm_T1024": (GEMM_SRC, "111d8436f4badcf5", 139596.3, 34816.0),
    "prefill_gemm_T4096": (GEMM_SRC, "111d8436f4badcf5", 515714.2, 139848.0),
    "qkv_prefill_T256": (GEMM_SRC, "111d8436f4badcf5", 12470.0, 1849.3),
    "qkv_prefill_T4096": (GEMM_SRC, "111d8436f4badcf5", 75757.6, 29650.2),
    "moe_prefill_top8_T256": (MOEP_SRC, "1fd358bb4ab7069d", 193672.9, 23585.8),
    "quantize_17408x5120_f32_g64": (QUANT_SRC, "957344c34d8c5002", 174101.4, 48960.1),
}


def kernel_source_hash(files) -> str:
    """Hash of the listed kernel sources' code: line comments and whitespace do not count,
    so an edit that only touches comments keeps the measured traffic figures valid."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "dequant_matmul_int4_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(files):
        h.update(name.encode())
        with open(os.path.join(csrc, name), encoding="utf-8") as fh:
            code = re.sub(r"//[^\n]*", "", fh.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def traffic_bytes(workload_name: str):
    """Measured HBM bytes per step, or None (not measured, or kernels changed since)."""
    t = TRAFFIC.get(workload_name)
    if t is None or kernel_source_hash(t[0]) != t[1]:
        return None
    return (t[2] * TRAFFIC_FETCH_SCALE + t[3] * TRAFFIC_WRITE_SCALE) * 1024.0


METRIC = "weight GB/s and % of HBM peak for T=1 int4 GEMV; tokens/s-equivalent"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dense",
                    choices=["single", "qkv", "rmsqkv", "smallm", "dense", "moe", "moeprefill", "prefill",
                             "qkvprefill", "quant", "copy"])
    ap.add_argument("--T", type=int, default=None,
                    help="prefill rows (default 256) or small-M tokens (default 4)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="wall-time budget of the CPU oracle sample (0 disables)")
    ap.add_argument("--router", choices=("fused", "gpu", "pre-drawn"), default="fused",
                    help="moe: route each token inside the gate/up launch (default), with the "
                         "separate router kernel, or use pre-drawn ids/weights")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the steps one by one instead of replaying a HIP graph "
                         "(for counter collection; the timing then includes launch gaps)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the stream-read (and bf16 GEMM) ceilings measured next to the workload")
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

    def parts(self):
        """The step's library calls, each timed on its own: (kernel label, fn(i), algorithmic
        bytes per call, algorithmic flops per call, kernel launches per call).  The first
        is the dominant one, the kernel ``roofline`` describes."""
        return [(self.dominant, self.step, self.algo_bytes(), float(getattr(self, "flops", 0.0)),
                 self.launches_per_step)]


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
    dominant = "qgemv_xs_kernel (gate/up pair with SwiGLU, then down)"

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

    def gate_up(self, i):
        g, u, _ = self.pool[i % self.R]
        self.q.qgemv_int4_multi([g, u], self.x, [self.h], epilogue=self.q.EPI_SWIGLU_PAIR)

    def down(self, i):
        self.q.qgemv_int4(self.pool[i % self.R][2], self.h, self.y)

    def step(self, i):
        self.gate_up(i)
        self.down(i)

    def parts(self):
        g, u, d = self.pool[0]
        return [("qgemv_xs_kernel (gate/up pair with SwiGLU, bf16 x, fp32 h)", self.gate_up,
                 g.weight_bytes + u.weight_bytes + 5120 * 2 + 17408 * 4, 0.0, 1),
                ("qgemv_xs_kernel (down, fp32 h, bf16 y)", self.down,
                 d.weight_bytes + 17408 * 4 + 5120 * 2, 0.0, 1)]


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
        self.ws = torch.empty(q.moe_gather_qgemv_int4_workspace_bytes(stacks[0][2], K), dtype=torch.uint8,
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


class QKVPrefill(QKV):
    """q/k/v prefill: T rows of a 4096-wide bf16 block through the 4096 -> 4096/1024/1024
    projections in one qgemm_int4_padT_multi launch (timed beside three qgemm_int4_padT calls)."""

    def __init__(self, q, synth, torch, T):
        super().__init__(q, synth, torch)
        self.T = T
        self.name = "qkv_prefill_T%d" % T
        self.dominant = "qgemm_int4_padT_multi (q/k/v, one launch, bf16 MFMA)"
        self.xT = torch.randn(T, 4096, device="cuda").to(torch.bfloat16)
        self.ysT = [torch.empty(T, n, device="cuda", dtype=torch.bfloat16) for n in (4096, 1024, 1024)]
        self.flops = 2.0 * T * 4096 * 6144
        self.config = dict(self.config, workload=self.name, T=T)

    def algo_bytes(self):
        return self.wb + self.T * (4096 * 2 + 6144 * 2)

    def step(self, i):
        self.q.qgemm_int4_padT_multi(self.pool[i % self.R], self.xT, self.ysT)

    def separate(self, i):
        for w, y in zip(self.pool[i % self.R], self.ysT):
            self.q.qgemm_int4_padT(w, self.xT, y)

    def parts(self):
        return [(self.dominant, self.step, self.algo_bytes(), self.flops, 1),
                ("three qgemm_int4_padT calls (q, k, v)", self.separate, self.algo_bytes(), self.flops, 3)]


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_sample(workload: str, T: int, threads: int):
    """(fn, amount per call, unit, description, fixed thread count or None) for the oracle on
    a bounded sample of the workload: amount is weight bytes (GB/s) or flops (TFLOP/s)."""
    import numpy as np

    import oracle
    import synth

    if workload == "single":
        d = synth.single_gemv()
        return (lambda: oracle.gemv(d["w"], d["x"], "f32", threads=threads), d["w"].weight_bytes,
                "GB/s", "full 1024x1024 GEMV (seed 0), repeated", None)
    if workload in ("qkv", "rmsqkv", "smallm"):
        if workload == "rmsqkv":
            d = synth.rms_qkv()
            fn = lambda: oracle.rms_norm_multi(d["ws"], d["x"], "bf16", d["gamma"], d["eps"],
                                               threads=threads)
            desc = "full RMSNorm + q/k/v set (seed 5), repeated"
        elif workload == "qkv":
            d = synth.qkv_multi()
            fn = lambda: oracle.multi(d["ws"], d["x"], "bf16", threads=threads)
            desc = "full q/k/v set (seed 1), repeated"
        else:
            d = synth.qkv_multi()
            xs = [synth.draw_activation(np.random.default_rng(100 + t), (4096,), "bf16")
                  for t in range(T)]
            fn = lambda: [oracle.multi(d["ws"], x, "bf16", threads=threads) for x in xs]
            desc = "full q/k/v set (seed 1) for %d tokens, repeated" % T
        return fn, sum(w.weight_bytes for w in d["ws"]), "GB/s", desc, None
    if workload == "dense":
        d = synth.dense_layer()
        return (lambda: oracle.dense_ffn(d["gate"], d["up"], d["down"], d["x"], "bf16", threads=threads),
                sum(d[k].weight_bytes for k in ("gate", "up", "down")), "GB/s",
                "full dense layer (seed 2): gate/up + SwiGLU + down, repeated", None)
    if workload == "moe":
        d = synth.moe_layer()
        per = d["gate"].weight_bytes // d["gate"].n_experts

        def fn():
            ids, wts = oracle.router_topk(d["logits"][0], 8)
            return oracle.moe(d["gate"], d["up"], d["down"], d["x"][0], ids, wts.astype(np.float32),
                              d["residual"][0], "bf16", threads=threads)
        return fn, 3 * 8 * per, "GB/s", ("one token of the 128-expert layer (seed 3): router + top-8 "
                                         "experts, repeated"), None
    if workload == "moeprefill":
        d = synth.moe_prefill_layer(T=max(T, 2))
        ntok = 2
        pairs = [oracle.router_topk(d["logits"][t].astype(np.float64), 8) for t in range(ntok)]
        ids = np.array([p_[0] for p_ in pairs])
        wts = np.array([p_[1] for p_ in pairs], dtype=np.float32)
        return (lambda: oracle.moe_prefill(d["gate"], d["up"], d["down"], d["x"][:ntok], ids, wts,
                                           d["residual"][:ntok], threads=threads),
                6.0 * ntok * 8 * 768 * 2048, "TFLOP/s",
                "%d tokens of the 128-expert layer (seed 6) per call: router + 8 experts each" % ntok,
                None)
    if workload == "quant":
        rng = np.random.default_rng(11)
        rows = 512
        W = synth.draw_float_weights(rng, (rows, 5120), "f32")
        return (lambda: oracle.quantize(W, "f32", 64, "bf16"), W.nbytes, "GB/s",
                "%d x 5120 rows of float32 weights per call (numpy float32, one thread)" % rows, 1)
    if workload == "qkvprefill":
        d = synth.qkv_multi()
        X = synth.draw_activation(np.random.default_rng(600 + T), (T, 4096), "bf16")
        rng = np.random.default_rng(0)
        t_idx = np.repeat(np.arange(min(T, 4)), 64 // min(T, 4))
        picks = [(w, rng.integers(0, w.n_out, t_idx.size)) for w in d["ws"]]
        return (lambda: [oracle.gemm_entries(w, X, t_idx, o, "bf16", threads=threads) for w, o in picks],
                3 * 2.0 * t_idx.size * 4096, "TFLOP/s",
                "%d sampled output entries of each of q, k, v (T=%d) per call" % (t_idx.size, T), None)
    d = synth.prefill_gemm(T=T)
    rows = 64
    rng = np.random.default_rng(0)
    t_idx = np.repeat(np.arange(min(T, 4)), rows // min(T, 4))
    o_idx = rng.integers(0, d["w"].n_out, t_idx.size)
    return (lambda: oracle.gemm_entries(d["w"], d["X"], t_idx, o_idx, "bf16", threads=threads),
            2.0 * t_idx.size * 5120, "TFLOP/s",
            "%d sampled output entries of the T=%d GEMM per call" % (t_idx.size, T), None)


def _rate(fn, amount, unit, budget_s):
    fn()  # first call outside the clock (library load, caches)
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    return amount * n / el / scale, n, el


def cpu_baseline(workload: str, budget_s: float, T: int):
    """The fp64 oracle as it stands on the host: all cores (the reported value), then one
    core, each for about budget_s / 2 seconds."""
    import oracle

    all_threads = max(1, min(oracle.max_threads(), os.cpu_count() or 1))
    fn, amount, unit, desc, fixed = _oracle_sample(workload, T, all_threads)
    threads = fixed or all_threads
    v, n, el = _rate(fn, amount, unit, budget_s / 2)
    out = {"value": v, "unit": unit, "cores": threads, "kind": "oracle",
           "sample": desc + "; %d calls in %.1f s on %d thread(s)" % (n, el, threads),
           "cpu_model": _cpu_model(), "host_cores": os.cpu_count()}
    if threads > 1:
        fn1, amount1, _, _, _ = _oracle_sample(workload, T, 1)
        v1, n1, el1 = _rate(fn1, amount1, unit, budget_s / 2)
        out["value_1core"] = v1
        out["sample_1core"] = "%d calls in %.1f s on 1 thread" % (n1, el1)
    else:
        out["value_1core"] = v
    return out


# ---------------------------------------------------------------------------

REPS = 5


class Timer:
    """Median-of-REPS graph timing of a per-step callable on one stream (see the module
    docstring for the shape of one repetition)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def ms_per_step(self, fn, K, W, first=0, no_graph=False):
        torch, stream = self.torch, self.stream
        times = []
        if no_graph:  # launches one by one (for counter collection)
            for _ in range(REPS):
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(stream):
                    for i in range(W):
                        fn(first + i)
                    e0.record(stream)
                    for i in range(K):
                        fn(first + W + i)
                    e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) / K)
        else:
            g_warm, g_main = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_warm, stream=stream):
                for i in range(W):
                    fn(first + i)
            with torch.cuda.graph(g_main, stream=stream):
                for i in range(K):
                    fn(first + W + i)
            torch.cuda.synchronize()
            for _ in range(REPS):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                with torch.cuda.stream(stream):
                    if W:
                        g_warm.replay()
                    e0.record(stream)
                    g_main.replay()
                    e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) / K)
            del g_warm, g_main
        s = sorted(times)
        return s[len(s) // 2], times


def stream_ceiling(torch, timer, nbytes, K, W):
    """Median time of a plain 128-bit read of nbytes (next buffer of a >= 1 GiB pool per
    launch), best over a few grid sizes; None when the calibration library is missing."""
    import ctypes
    path = os.path.join(ROOT, "dequant_matmul_int4_amd", "libqint4_calib.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.qint4_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_void_p]
    nb = (nbytes + 15) // 16 * 16
    R = max(2, math.ceil(POOL_BYTES / nb))
    pool = [torch.empty(nb, dtype=torch.uint8, device="cuda").random_(0, 256) for _ in range(R)]
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    best = None
    for grid in (1024, 2048, 4096, 8192):
        def fn(i, grid=grid):
            rc = lib.qint4_calib_stream_read(pool[i % R].data_ptr(), nb, sink.data_ptr(), grid,
                                             torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError("stream read launch failed: %d" % rc)
        ms, _ = timer.ms_per_step(fn, K, W)
        if best is None or ms < best[0]:
            best = (ms, grid)
    del pool
    ms, grid = best
    return {"bytes": nb, "us": ms * 1e3, "GBps": nb / (ms * 1e-3) / 1e9,
            "frac_of_peak": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "grid": grid,
            "kernel": "stream_read_kernel (libqint4_calib.so, 128-bit loads)"}


def gemm_ceiling(torch, timer, T, K_, W_steps):
    """torch's bf16 matmul (hipBLASLt) of the same shape, T x 5120 @ 5120 x 17408, over 6
    rotating weight copies: the measured dense bf16 GEMM rate on this GPU."""
    a = torch.randn(T, 5120, device="cuda").to(torch.bfloat16)
    ws = [torch.randn(17408, 5120, device="cuda").to(torch.bfloat16) for _ in range(6)]
    y = torch.empty(T, 17408, device="cuda", dtype=torch.bfloat16)

    def fn(i):
        torch.matmul(a, ws[i % 6].t(), out=y)
    # one eager call first: hipBLASLt sets itself up on its first product, which
    # is not allowed inside a graph capture
    with torch.cuda.stream(timer.stream):
        fn(0)
    torch.cuda.synchronize()
    ms, _ = timer.ms_per_step(fn, K_, W_steps)
    del ws
    return {"us": ms * 1e3, "TFLOPs": 2.0 * T * 5120 * 17408 / (ms * 1e-3) / 1e12,
            "kernel": "torch.matmul bf16 (hipBLASLt)"}


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
    elif args.workload == "qkvprefill":
        wl = QKVPrefill(q, synth, torch, args.T)
    elif args.workload == "moe":
        wl = MoE(q, synth, torch, router=args.router)
    else:
        wl = Prefill(q, synth, torch, args.T)
    torch.cuda.synchronize()
    print("# workload %s: pool %d copies, %.1f MB weights/step" % (
        wl.name, wl.R, wl.weight_bytes() / 1e6), file=sys.stderr, flush=True)

    K, W = args.steps, args.warmup
    stream = torch.cuda.Stream()
    timer = Timer(torch, stream)
    # eager warm-up call (caches device properties, sets kernel attributes)
    with torch.cuda.stream(stream):
        wl.step(0)
    stream.synchronize()

    ms_step, reps = timer.ms_per_step(wl.step, K, W, no_graph=args.no_graph)
    print("# %d steps x %d repetitions: %s ms/step" % (K, REPS, ", ".join("%.5f" % t for t in reps)),
          file=sys.stderr, flush=True)

    out = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": W,
           "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded, device-generated pool)",
           "config": wl.config, "repetitions": REPS, "ms_per_step_reps": reps}

    # each library call of the step on its own: K calls in a graph, same repetitions
    parts = []
    for label, fn, nbytes, flops, launches in wl.parts():
        if len(wl.parts()) == 1:
            ms = ms_step
        else:
            ms, _ = timer.ms_per_step(fn, K, W, no_graph=args.no_graph)
        parts.append({"kernel": label, "us": ms * 1e3, "bytes": nbytes, "flops": flops,
                      "GBps": nbytes / (ms * 1e-3) / 1e9,
                      "TFLOPs": flops / (ms * 1e-3) / 1e12 if flops else None,
                      "launches": launches})
    if len(parts) > 1:
        out["kernels"] = parts
    dom = parts[0]

    gemm_like = isinstance(wl, (Prefill, MoEPrefill, QKVPrefill))
    if gemm_like:
        tflops = wl.flops / (ms_step * 1e-3) / 1e12
        out.update({"value": tflops, "unit": "TFLOP/s",
                    "weight_GBps": wl.weight_bytes() / (ms_step * 1e-3) / 1e9,
                    "mfma_util": tflops / BF16_MFMA_PEAK_TFLOPS})
        if isinstance(wl, MoEPrefill):
            out["tokens_per_s"] = wl.T * 1e3 / ms_step
    else:
        gbs = wl.weight_bytes() / (ms_step * 1e-3) / 1e9
        out.update({"value": gbs, "unit": "GB/s", "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
                    "calls_per_s": 1e3 / ms_step})
        if isinstance(wl, Dense):
            out["tokens_per_s_equiv"] = 1e3 / (ms_step * args.layers)
            out["tokens_per_s_equiv_layers"] = args.layers
            out["tokens_per_s_equiv_note"] = "assumed layer count (the sources give none for this shape)"
        if isinstance(wl, MoE):
            out["tokens_per_s_equiv"] = 1e3 / (ms_step * 40)
            out["tokens_per_s_equiv_layers"] = 40
        if isinstance(wl, SmallM):
            out["tokens_per_call"] = wl.T

    # roofline of the dominant kernel: the longer of its ideal times decides the bound
    t_hbm = dom["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = dom["flops"] / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    ms_dom = dom["us"] * 1e-3
    if t_mfma > t_hbm:
        ach = dom["flops"] / (ms_dom * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": ach, "peak": BF16_MFMA_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": ach / BF16_MFMA_PEAK_TFLOPS}
    else:
        ach = dom["bytes"] / (ms_dom * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS}
    out["roofline"].update({"traffic": traffic_bytes(wl.name), "kernel": dom["kernel"],
                            "kernel_us": dom["us"], "launches_per_call": dom["launches"],
                            "algorithmic_bytes": dom["bytes"],
                            "algorithmic_flops": dom["flops"] or None})

    # measured ceilings of the same size, same run
    if not args.no_ceiling and args.workload != "copy":
        ceil = stream_ceiling(torch, timer, wl.weight_bytes(), K, W)
        if ceil is not None:
            out["stream_ceiling"] = ceil
            if not gemm_like:
                out["pct_stream_ceiling"] = 100.0 * out["value"] / ceil["GBps"]
            if out["roofline"]["bound"] == "hbm" and dom["bytes"] != wl.weight_bytes():
                cd = stream_ceiling(torch, timer, dom["bytes"], K, W)
                if cd is not None:
                    out["roofline"]["stream_ceiling_GBps"] = cd["GBps"]
            elif out["roofline"]["bound"] == "hbm":
                out["roofline"]["stream_ceiling_GBps"] = ceil["GBps"]
        if isinstance(wl, Prefill):
            gc = gemm_ceiling(torch, timer, wl.T, min(K, 50), min(W, 5))
            out["gemm_ceiling"] = gc
            out["pct_gemm_ceiling"] = 100.0 * out["value"] / gc["TFLOPs"]

    if args.cpu_seconds > 0 and args.workload != "copy":
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds, args.T)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
