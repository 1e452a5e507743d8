"""The ring-form case tables of test_gpu_gemv_depths agree with the planner mirror (CPU)."""
from tests import gemv_plan
from tests.test_gpu_gemv_depths import GEMV_CASES, MOE_CASES, SMALLM_CASES, SWIGLU_CASES


def test_case_tables_reach_every_ring_form():
    for n_out, k_in, x_dt, depth, steps in GEMV_CASES:
        p = gemv_plan.plan(k_in // 32, x_dt, lambda rpt: -(-n_out // rpt))
        assert (gemv_plan.ring_depth(p), gemv_plan.max_wave_steps(p)) == (depth, steps)
    for T, n_out, k_in, depth, steps in SMALLM_CASES:
        p = gemv_plan.plan(k_in // 32, "bf16", lambda rpt: -(-n_out // rpt), tt=T)
        assert (gemv_plan.ring_depth(p), gemv_plan.max_wave_steps(p)) == (depth, steps)
    for n_out, k_in, depth, steps in SWIGLU_CASES:
        p = gemv_plan.plan(k_in // 32, "bf16", lambda rpt: -(-n_out // rpt))
        assert (gemv_plan.ring_depth(p, streams=2), gemv_plan.max_wave_steps(p)) == (depth, steps)
    for hidden, inter, top_k, residual, d_gu, d_down in MOE_CASES:
        pg = gemv_plan.plan(hidden // 32, "bf16", lambda rpt: top_k * -(-inter // rpt))
        pd = gemv_plan.plan(top_k * inter // 32, "f32", lambda rpt: -(-hidden // rpt),
                            residual_rows=hidden if residual else 0)
        assert (gemv_plan.ring_depth(pg, streams=2), gemv_plan.ring_depth(pd)) == (d_gu, d_down)
    # every form is reached: one pass 1, 2, 4 (also with a short wave) and streaming
    assert {c[3] for c in GEMV_CASES} == {0, 1, 2, 4}
    assert {c[4] for c in GEMV_CASES if c[3] == 4} == {3, 4}
    assert {c[3] for c in SMALLM_CASES} == {0, 1, 2, 4}
    assert all(c[2] % 512 for c in SMALLM_CASES)  # off the small-M MFMA route
    assert {c[2] for c in SWIGLU_CASES} == {0, 1, 2, 4}
    assert {c[4] for c in MOE_CASES} == {0, 1, 2} and {c[5] for c in MOE_CASES} == {0, 1, 2, 4}


def test_mirror_plans_the_qkv_projection_as_one_task_per_wave():
    """q/k/v of a 4096 activation (6144 rows): 12 waves per CU, 2 rows per task, 2 steps."""
    p = gemv_plan.plan(128, "bf16", lambda rpt: sum(-(-n // rpt) for n in (4096, 1024, 1024)))
    assert p[:4] == (12, 2, 64, 2) and gemv_plan.ring_depth(p) == 2
