"""The ring-form case tables of test_gpu_gemv_depths, checked on the CPU against the library's
own planner (the host-only plan query of libqint4.so, planning for 256 CUs): a planner change
that moves a case off the form it was chosen for fails here, without a GPU."""
import ctypes

import pytest

import dequant_matmul_int4_amd as q
from tests.test_gpu_gemv_depths import GEMV_CASES, MOE_CASES, SMALLM_CASES, SWIGLU_CASES

N_CU = 256  # MI355X


def _ring(form):
    assert form["kernel"] == "ring"
    return form["ring_depth"], form["busiest_wave_steps"]


def test_case_tables_reach_every_ring_form():
    for n_out, k_in, x_dt, depth, steps in GEMV_CASES:
        assert _ring(q.plan_qgemv([n_out], k_in, x_dtype=x_dt, n_cu=N_CU)) == (depth, steps)
    for T, n_out, k_in, depth, steps in SMALLM_CASES:
        f = q.plan_qgemv([n_out], k_in, T=T, call=q.CALL_SMALLM, n_cu=N_CU)
        assert _ring(f) == (depth, steps) and f["tokens"] == T
    for n_out, k_in, depth, steps in SWIGLU_CASES:
        f = q.plan_qgemv([n_out, n_out], k_in, epilogue=q.EPI_SWIGLU_PAIR, n_cu=N_CU)
        assert _ring(f) == (depth, steps)
    for hidden, inter, top_k, residual, d_gu, d_down in MOE_CASES:
        gu, down = q.plan_moe_gather(hidden, inter, top_k, group_size=64 if inter % 64 == 0 else 32,
                                     residual=residual, n_cu=N_CU)
        assert (gu["ring_depth"], down["ring_depth"]) == (d_gu, d_down)
    # every form is reached: one pass 1, 2, 4 (also with a short wave) and streaming
    assert {c[3] for c in GEMV_CASES} == {0, 1, 2, 4}
    assert {c[4] for c in GEMV_CASES if c[3] == 4} == {3, 4}
    assert {c[3] for c in SMALLM_CASES} == {0, 1, 2, 4}
    assert {c[2] for c in SWIGLU_CASES} == {0, 1, 2, 4}
    assert {c[4] for c in MOE_CASES} == {0, 1, 2} and {c[5] for c in MOE_CASES} == {0, 1, 2, 4}


def test_qkv_projection_is_one_task_pair_per_wave():
    """q/k/v of a 4096 activation (6144 rows): 12 waves per CU, 64 lanes a row, 2 rows per task,
    one task per wave, so a one-pass ring of depth 2."""
    f = q.plan_qgemv([4096, 1024, 1024], 4096, n_cu=N_CU)
    assert (f["kernel"], f["waves"], f["lanes"], f["rows_per_task"], f["steps_per_task"]) == \
        ("ring", 12, 64, 2, 2)
    assert f["grid"] == N_CU and f["ring_depth"] == 2 and f["launches"] == 1


def test_xs_form_for_several_matrices():
    """q/k/v of an 8192 activation (10240 rows, 8 waves of 32 lanes): two workgroups per CU
    shared out by rows, 20 a workgroup (410 + 52 + 52 workgroups)."""
    f = q.plan_qgemv([8192, 1024, 1024], 8192, x_dtype="bf16", n_cu=N_CU)
    assert (f["kernel"], f["waves"], f["lanes"], f["grid"], f["tasks"], f["busiest_wave_steps"],
            f["launches"]) == ("xs", 8, 32, 410 + 52 + 52, 10240, 20, 1)


@pytest.mark.parametrize("n_outs,k_in,x_dt,epi,call,T", [
    ([2000, 2000], 1280, "bf16", q.EPI_SWIGLU_PAIR, q.CALL_QGEMV, 1),
    ([5120], 3584, "f32", q.EPI_NONE, q.CALL_QGEMV, 1),
    ([4096, 1024, 1024], 4096, "bf16", q.EPI_NONE, q.CALL_RMS_NORM, 1),
    ([4096, 1024, 1024], 4096, "f32", q.EPI_NONE, q.CALL_RMS_NORM, 1),
    ([5000], 2304, "bf16", q.EPI_NONE, q.CALL_SMALLM, 13),
    ([3, 9, 100, 31, 2, 7, 1, 64], 192, "bf16", q.EPI_NONE, q.CALL_QGEMV, 1),
])
def test_ring_plans_cover_every_row_and_chunk(n_outs, k_in, x_dt, epi, call, T):
    """Whatever the planner picks: tasks cover every row, lanes x steps cover every 32-code
    chunk of a row, the grid fits the CUs, the waves fit a workgroup, and token blocks cover T."""
    f = q.plan_qgemv(n_outs, k_in, x_dtype=x_dt, T=T, epilogue=epi, call=call, n_cu=N_CU)
    assert f["kernel"] == "ring"
    rows = n_outs[:1] if epi == q.EPI_SWIGLU_PAIR else n_outs
    assert f["tasks"] == sum(-(-n // f["rows_per_task"]) for n in rows)
    assert f["rows_per_task"] * f["lanes"] in (64, 128)
    assert f["lanes"] * f["steps_per_task"] >= k_in // 32 > f["lanes"] * (f["steps_per_task"] - 1)
    assert 1 <= f["grid"] <= N_CU and 1 <= f["waves"] <= 12
    assert f["busiest_wave_steps"] == -(-f["tasks"] // (f["grid"] * f["waves"])) * f["steps_per_task"]
    assert f["launches"] * f["tokens"] >= T > (f["launches"] - 1) * f["tokens"]
    assert f["ring_depth"] in (0, 1, 2, 4)
    if f["ring_depth"]:
        assert f["busiest_wave_steps"] <= f["ring_depth"]


def test_smallm_mfma_form():
    """k_in a multiple of 512 (at most 16 K slices of 512) with bf16 activations: the small-M
    call takes 16-row MFMA tiles, all 16 tokens in one launch where their staged rows fit in LDS,
    else blocks of 8.  Wider rows (the 17408-column down projection) take the GEMV rings in
    token blocks whose staged rows fit."""
    f = q.plan_qgemv([4096, 1024, 1024], 4096, T=16, call=q.CALL_SMALLM, n_cu=N_CU)
    assert (f["kernel"], f["tokens"], f["launches"], f["tasks"]) == ("mfma", 16, 1, 6144 // 16)
    assert f["grid"] == N_CU  # one 145 KB workgroup per CU, each staging its rows once for its tiles
    f = q.plan_qgemv([17408], 5120, T=16, call=q.CALL_SMALLM, n_cu=N_CU)
    assert (f["kernel"], f["tokens"], f["launches"], f["waves"]) == ("mfma", 8, 2, 10)
    f = q.plan_qgemv([17408], 5120, T=1, call=q.CALL_SMALLM, n_cu=N_CU)
    assert (f["kernel"], f["tokens"], f["launches"]) == ("mfma", 1, 1)
    f = q.plan_qgemv([5120], 17408, T=16, call=q.CALL_SMALLM, n_cu=N_CU)
    assert (f["kernel"], f["tokens"], f["launches"]) == ("ring", 4, 4)


def test_xs_form_for_long_rows():
    """One matrix, 4096 <= k_in <= 32768 and at least 5120 x 5120 codes (the dense down
    projection 17408 -> 5120): the activation-stationary kernel, 32 lanes a row (two rows a step)
    while that takes at most 16 waves, else 64; two workgroups per CU while a workgroup has at
    most eight waves, else one."""
    for x_dt in ("f32", "bf16"):
        f = q.plan_qgemv([5120], 17408, x_dtype=x_dt, n_cu=N_CU)
        assert (f["kernel"], f["grid"], f["waves"], f["lanes"], f["tasks"], f["busiest_wave_steps"],
                f["ring_depth"]) == ("xs", N_CU, 9, 64, 5120, 20, 4)
        f = q.plan_qgemv([17408], 5120, x_dtype=x_dt, n_cu=N_CU)
        assert (f["kernel"], f["grid"], f["waves"], f["lanes"], f["busiest_wave_steps"]) == \
            ("xs", 2 * N_CU, 5, 32, 34)
        f = q.plan_qgemv([5120], 5120, x_dtype=x_dt, n_cu=N_CU)
        assert (f["kernel"], f["grid"]) == ("xs", 2 * N_CU)
    f = q.plan_qgemv([5000], 8192, x_dtype="f32", n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["waves"], f["lanes"], f["rows_per_task"], f["busiest_wave_steps"]) == \
        ("xs", 2 * N_CU, 8, 32, 2, 10)
    f = q.plan_qgemv([4100], 8320, group_size=32, x_dtype="f32", n_cu=N_CU)
    assert (f["kernel"], f["waves"], f["lanes"]) == ("xs", 9, 32)
    f = q.plan_qgemv([256 * N_CU], 8320, x_dtype="f32", n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["busiest_wave_steps"]) == ("xs", N_CU, 256)
    f = q.plan_qgemv([512 * N_CU], 4096, x_dtype="bf16", n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["busiest_wave_steps"]) == ("xs", 2 * N_CU, 256)
    f = q.plan_qgemv([2049], 32768, x_dtype="f32", n_cu=N_CU)
    assert (f["kernel"], f["waves"], f["lanes"]) == ("xs", 16, 64)
    # short rows: four workgroups per CU up to three waves (the 128256-row LM head over 2048
    # columns), and more workgroups where one would get over 256 rows
    f = q.plan_qgemv([128256], 2048, x_dtype="bf16", n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["waves"], f["busiest_wave_steps"]) == ("xs", 4 * N_CU, 2, 126)
    f = q.plan_qgemv([152064], 5120, x_dtype="bf16", n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["busiest_wave_steps"]) == ("xs", 594, 256)
    f = q.plan_qgemv([512 * N_CU + 1], 4096, x_dtype="bf16", n_cu=N_CU)
    assert f["kernel"] == "xs" and f["busiest_wave_steps"] <= 256
    # behind the RMSNorm prologue alike (the LM head after the final norm)
    f = q.plan_qgemv([128256], 2048, x_dtype="bf16", call=q.CALL_RMS_NORM, n_cu=N_CU)
    assert (f["kernel"], f["grid"]) == ("xs", 4 * N_CU)
    f = q.plan_qgemv([17408, 17408], 5120, epilogue=q.EPI_SWIGLU_PAIR, call=q.CALL_RMS_NORM, n_cu=N_CU)
    assert (f["kernel"], f["grid"]) == ("xs", 3 * N_CU)


@pytest.mark.parametrize("n_outs,k_in,x_dt,epi,call", [
    ([9000], 1984, "f32", q.EPI_NONE, q.CALL_QGEMV),             # rows shorter than 2048
    ([14000], 1984, "bf16", q.EPI_NONE, q.CALL_QGEMV),           # the same
    ([2000], 32832, "f32", q.EPI_NONE, q.CALL_QGEMV),            # more than 16 waves of 64 lanes
    ([4096], 4096, "f32", q.EPI_NONE, q.CALL_QGEMV),             # fewer than 5120 x 5120 codes
    ([6144], 4096, "bf16", q.EPI_NONE, q.CALL_QGEMV),            # the same
    ([4096, 1024, 1024], 4096, "bf16", q.EPI_NONE, q.CALL_QGEMV),  # q/k/v of 4096: the same
    ([9000, 9000], 1984, "bf16", q.EPI_SWIGLU_PAIR, q.CALL_QGEMV),  # pair, rows under 2048
    ([2000, 2000], 8192, "bf16", q.EPI_SWIGLU_PAIR, q.CALL_QGEMV),  # pair, fewer than 2^25 codes
    ([5120, 5120], 17408, "bf16", q.EPI_SWIGLU_PAIR, q.CALL_SMALLM),  # small-M call
])
def test_xs_form_only_where_it_applies(n_outs, k_in, x_dt, epi, call):
    f = q.plan_qgemv(n_outs, k_in, x_dtype=x_dt, epilogue=epi, call=call, n_cu=N_CU)
    assert f["kernel"] != "xs"


def test_xs_form_for_the_gate_up_pair():
    """The T=1 gate/up pair with 2048 <= k_in <= 32768 (dense FFN 5120 -> 17408): 32 lanes a
    row (two rows a step) up to 16384 columns, 64 beyond; 16 / waves workgroups per CU, one to
    four."""
    f = q.plan_qgemv([17408, 17408], 5120, epilogue=q.EPI_SWIGLU_PAIR, n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["waves"], f["lanes"], f["rows_per_task"], f["tasks"],
            f["busiest_wave_steps"]) == ("xs", 3 * N_CU, 5, 32, 2, 17408, -(-17408 // (3 * N_CU)))
    f = q.plan_qgemv([14336, 14336], 4096, epilogue=q.EPI_SWIGLU_PAIR, n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["waves"]) == ("xs", 4 * N_CU, 4)
    f = q.plan_qgemv([8192, 8192], 8192, epilogue=q.EPI_SWIGLU_PAIR, n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["waves"]) == ("xs", 2 * N_CU, 8)
    f = q.plan_qgemv([2048, 2048], 17408, x_dtype="f32", epilogue=q.EPI_SWIGLU_PAIR, n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["waves"], f["lanes"]) == ("xs", N_CU, 9, 64)
    f = q.plan_qgemv([8192, 8192], 2048, epilogue=q.EPI_SWIGLU_PAIR, n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["waves"], f["lanes"]) == ("xs", 4 * N_CU, 2, 32)
    f = q.plan_qgemv([1000, 1000], 32768, epilogue=q.EPI_SWIGLU_PAIR, n_cu=N_CU)
    assert (f["kernel"], f["grid"], f["waves"], f["lanes"], f["busiest_wave_steps"]) == \
        ("xs", N_CU, 16, 64, 4)
    # fewer rows than workgroups (a part with more CUs): one row each
    f = q.plan_qgemv([1000, 1000], 32768, epilogue=q.EPI_SWIGLU_PAIR, n_cu=2048)
    assert (f["kernel"], f["grid"], f["busiest_wave_steps"]) == ("xs", 1000, 1)


def test_plan_query_rejects_what_the_calls_reject():
    lib = q.load()
    form = q.CGemvForm()
    n1 = (ctypes.c_int64 * 2)(64, 64)
    bad = [
        (q.CALL_QGEMV, 1, n1, 100, 64, 1, 1, 0, 256),     # k_in not a multiple of group_size
        (q.CALL_QGEMV, 1, n1, 128, 48, 1, 1, 0, 256),     # group_size
        (q.CALL_QGEMV, 0, n1, 128, 64, 1, 1, 0, 256),     # n
        (q.CALL_QGEMV, 1, n1, 128, 64, 1, 2, 0, 256),     # T > 1 outside small-M
        (q.CALL_SMALLM, 1, n1, 128, 64, 1, 17, 0, 256),   # T beyond the small-M limit
        (q.CALL_SMALLM, 1, n1, 128, 64, 0, 2, 0, 256),    # T > 1 with float32 activations
        (q.CALL_QGEMV, 1, n1, 128, 64, 1, 1, 1, 256),     # SWIGLU_PAIR with one matrix
        (q.CALL_QGEMV, 1, n1, 128, 64, 2, 1, 0, 256),     # dtype
        (7, 1, n1, 128, 64, 1, 1, 0, 256),                # call
        (q.CALL_QGEMV, 1, n1, 128, 64, 1, 1, 0, -1),      # n_cu
    ]
    for args in bad:
        assert lib.qint4_plan_qgemv(*args, ctypes.byref(form)) != 0, args
    assert lib.qint4_plan_qgemv(q.CALL_QGEMV, 1, n1, 128, 64, 1, 1, 0, 256, None) == 1
    forms = (q.CGemvForm * 2)()
    assert lib.qint4_plan_moe_gather(2048, 768, 9, 64, 1, 0, 1, 256, forms) != 0    # top_k
    assert lib.qint4_plan_moe_gather(2048, 100, 8, 64, 1, 0, 1, 256, forms) != 0    # inter
    assert lib.qint4_plan_moe_gather(2048, 768, 8, 64, 1, 0, 1, 256, forms) == 0
