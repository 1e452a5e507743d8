"""Host-side mirror of the GEMV launch planner (test infrastructure).

The GEMV kernels come in two forms: a streaming one, whose register ring is
refilled while it is consumed, and one-pass ones (ring depth 1, 2 or 4) used
when no wave of a launch has more steps than that.  Which one a call runs
depends on the plan (lanes per row, rows per task, waves), so the tests that
must reach every form pick their shapes with this mirror of the planner.  It
only chooses shapes: parity is always judged against the oracle.
"""
import math

N_CU = 256
MAX_LDS = 160 * 1024
K_SLOTS = 8  # 128-bit code loads per lane in a wave's ring
XM_OCTETS = {"bf16": 2, "f32": 5, "rms_bf16": 4, "rms_f32": 3}


def lanes_for(chunks: int) -> int:
    lanes = 1
    while lanes < 64 and chunks % (lanes * 2) == 0:
        lanes *= 2
    return lanes


def lds_bytes(xm: str, ncx_pad: int, residual_rows: int, tt: int) -> int:
    xb = 64 if xm == "bf16" else 128
    return tt * (((ncx_pad * 4 + 15) & ~15) + ncx_pad * xb) + residual_rows * 4


def plan(cpr: int, xm: str, tasks_for, residual_rows: int = 0, tt: int = 1):
    """(waves, rt, lanes, spt, n_tasks, grid) as the library plans a launch over rows of cpr
    32-code chunks."""
    best, best_cost = None, math.inf
    cands = [lanes_for(cpr)] + [l for l in (32, 64) if cpr > l and cpr % l and l > lanes_for(cpr)]
    max_w = 8 if tt >= 8 else 12
    for L in cands:
        spt = -(-cpr // L)
        if lds_bytes(xm, spt * L, residual_rows, tt) > MAX_LDS:
            continue
        for rt in (1, 2):
            n_tasks = tasks_for(rt * (64 // L))
            for w in range(1, max_w + 1):
                if residual_rows > w * 64 * 4 * 4:
                    continue
                grid = min(N_CU, -(-n_tasks // w))
                tpw = -(-n_tasks // (grid * w))
                cost = tpw * w * spt * (rt + (0.0 if xm == "bf16" else 1.0))
                if cpr * 4 > XM_OCTETS[xm] * 64 * w:
                    cost *= 1.5
                better = cost < best_cost * (1 - 1e-9) or (
                    cost <= best_cost * (1 + 1e-9) and
                    (rt > best[1] or (rt == best[1] and w > best[0])))
                if better:
                    best_cost, best = cost, (w, rt, L, spt, n_tasks, grid)
    return best


def max_wave_steps(p) -> int:
    w, rt, L, spt, n_tasks, grid = p
    return -(-n_tasks // (grid * w)) * spt


def ring_depth(p, streams: int = 1) -> int:
    """Depth of the ring the launch runs with: 1, 2 or 4 (one pass) or 0 (streaming)."""
    s = max_wave_steps(p)
    rt = p[1]
    if s == 1:
        return 1
    if s == 2 and 2 * rt * streams <= K_SLOTS:
        return 2
    if 3 <= s <= 4 and 4 * rt * streams <= K_SLOTS:
        return 4
    return 0


def gemv_depth(n_out: int, k_in: int, xm: str = "bf16", tt: int = 1) -> int:
    p = plan(k_in // 32, xm, lambda rpt: -(-n_out // rpt), tt=tt)
    return ring_depth(p)


def swiglu_depth(n_out: int, k_in: int, xm: str = "bf16", slots: int = 1) -> int:
    p = plan(k_in // 32, xm, lambda rpt: slots * -(-n_out // rpt))
    return ring_depth(p, streams=2)


def moe_down_depth(hidden: int, inter: int, top_k: int, residual: bool) -> int:
    p = plan(top_k * inter // 32, "f32", lambda rpt: -(-hidden // rpt),
             residual_rows=hidden if residual else 0)
    return ring_depth(p)
