// api.cpp -- the extern "C" entry points of libqint4.so: argument validation,
// launch planning and dispatch to the gfx950 kernels.  Semantics, layouts and
// error behaviour are specified in include/qint4.h.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>

#include "kernels.h"
#include "qint4.h"

using namespace qint4;

namespace {

thread_local char g_last_error[768] = "";

qint4_status fail(qint4_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

// Re-raise a status from a helper with the entry point's name in front.
qint4_status prefixed(qint4_status st, const char *fn) {
  char tmp[sizeof(g_last_error)];
  std::memcpy(tmp, g_last_error, sizeof(tmp));
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", fn, tmp);
  return st;
}

qint4_status ok() {
  g_last_error[0] = '\0';
  return QINT4_OK;
}

inline size_t elem_bytes(int32_t dt) { return dt == QINT4_BF16 ? 2 : 4; }
inline bool valid_dtype(int32_t dt) { return dt == QINT4_F32 || dt == QINT4_BF16; }
inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int ilog2(int64_t v) {
  int l = 0;
  while ((int64_t)1 << (l + 1) <= v) ++l;
  return l;
}

// Address range [p, p + n) of one buffer, for overlap checks.
struct Range {
  uintptr_t lo = 0, hi = 0;
  const char *name = "";
};

Range range(const void *p, size_t n, const char *name) {
  Range r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + n;
  r.name = name;
  return r;
}

bool overlap(const Range &a, const Range &b) {
  return a.lo != 0 && b.lo != 0 && a.lo < b.hi && b.lo < a.hi;
}

qint4_status check_no_overlap(const Range *outs, int n_out, const Range *ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j]))
        return fail(QINT4_ERR_ALIAS, "output %s overlaps input %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(QINT4_ERR_ALIAS, "output %s overlaps output %s", outs[i].name, outs[j].name);
  }
  return QINT4_OK;
}

size_t code_bytes(const qint4_matrix *w);
size_t sb_bytes(const qint4_matrix *w);

// Kernels address a matrix (or expert stack) through 32-bit byte offsets.
constexpr size_t kMaxMatrixBytes = (size_t)1 << 31;

qint4_status check_matrix_size(const qint4_matrix *w, const char *name) {
  if (code_bytes(w) >= kMaxMatrixBytes || sb_bytes(w) >= kMaxMatrixBytes)
    return fail(QINT4_ERR_SHAPE, "%s: %zu code bytes / %zu scale bytes exceed the 2 GiB limit", name,
                code_bytes(w), sb_bytes(w));
  return QINT4_OK;
}

constexpr int64_t kMaxK = 1 << 20;
constexpr int64_t kMaxRows = (int64_t)1 << 30;

// Workspace of an expert-gather decode call: the float32 SwiGLU
// intermediates, inter of them per kept expert (0 for sizes it rejects).
size_t moe_ws_bytes(int64_t inter, int32_t top_k) {
  if (inter < 1 || inter > kMaxK || top_k < 1 || top_k > QINT4_TOPK_MAX) return 0;
  return (size_t)top_k * (size_t)inter * sizeof(float);
}

qint4_status check_matrix(const qint4_matrix *w, const char *name, bool experts_ok) {
  if (!w) return fail(QINT4_ERR_NULL, "%s: matrix descriptor is NULL", name);
  if (!w->codes || !w->scales || !w->biases)
    return fail(QINT4_ERR_NULL, "%s: codes/scales/biases pointer is NULL", name);
  if (w->reserved != 0) return fail(QINT4_ERR_SHAPE, "%s: reserved field must be 0", name);
  if (w->group_size != 32 && w->group_size != 64 && w->group_size != 128)
    return fail(QINT4_ERR_SHAPE, "%s: group_size %d not in {32, 64, 128}", name, w->group_size);
  if (w->n_out < 1 || w->n_out > kMaxRows)
    return fail(QINT4_ERR_SHAPE, "%s: n_out %lld out of range [1, 2^30]", name, (long long)w->n_out);
  if (w->k_in < w->group_size || w->k_in > kMaxK || w->k_in % w->group_size != 0)
    return fail(QINT4_ERR_SHAPE, "%s: k_in %lld must be a multiple of group_size %d in [%d, 2^20]",
                name, (long long)w->k_in, w->group_size, w->group_size);
  if (w->n_experts < 1) return fail(QINT4_ERR_SHAPE, "%s: n_experts %d < 1", name, w->n_experts);
  if (!experts_ok && w->n_experts != 1)
    return fail(QINT4_ERR_SHAPE, "%s: n_experts must be 1 here, got %d", name, w->n_experts);
  if (!valid_dtype(w->sb_dtype)) return fail(QINT4_ERR_DTYPE, "%s: sb_dtype %d invalid", name, w->sb_dtype);
  if (!aligned(w->codes, 16)) return fail(QINT4_ERR_ALIGN, "%s: codes not 16-byte aligned", name);
  const size_t sb = elem_bytes(w->sb_dtype);
  if (!aligned(w->scales, sb) || !aligned(w->biases, sb))
    return fail(QINT4_ERR_ALIGN, "%s: scales/biases not aligned to %zu bytes", name, sb);
  return check_matrix_size(w, name);
}

size_t code_bytes(const qint4_matrix *w) {
  return (size_t)w->n_experts * (size_t)w->n_out * (size_t)(w->k_in / 2);
}
size_t sb_bytes(const qint4_matrix *w) {
  return (size_t)w->n_experts * (size_t)w->n_out * (size_t)(w->k_in / w->group_size) *
         elem_bytes(w->sb_dtype);
}

int add_matrix_ranges(const qint4_matrix *w, const char *names[3], Range *out) {
  out[0] = range(w->codes, code_bytes(w), names[0]);
  out[1] = range(w->scales, sb_bytes(w), names[1]);
  out[2] = range(w->biases, sb_bytes(w), names[2]);
  return 3;
}

// Device properties, cached per device ordinal.
struct DevInfo {
  int state = 0;  // 0 unknown, 1 gfx950, 2 other
  int cus = 0;
};
DevInfo g_dev[64];

qint4_status check_device(int *n_cu) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(QINT4_ERR_DEVICE, "no current HIP device");
  }
  if (dev >= 64) return fail(QINT4_ERR_DEVICE, "device ordinal %d not supported", dev);
  DevInfo &d = g_dev[dev];
  if (d.state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(QINT4_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    }
    d.cus = prop.multiProcessorCount;
    d.state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  if (d.state != 1) return fail(QINT4_ERR_DEVICE, "device %d is not gfx950", dev);
  if (n_cu) *n_cu = d.cus;
  return QINT4_OK;
}

// ---------------------------------------------------------------------------
// GEMV planning
// ---------------------------------------------------------------------------

// Lanes per row: the largest power of two <= 64 dividing the chunk count.
int lanes_for(int chunks) {
  int l = 1;
  while (l < 64 && chunks % (l * 2) == 0) l *= 2;
  return l;
}

constexpr int kMaxWaves = 12;  // waves per workgroup (one persistent workgroup per CU)

// Plan a GEMV-family launch over rows of `cpr` (virtual) chunks.
// tasks_for(rows_per_task) returns the task count for a task height.
//
// Candidates: lanes per row L (the exact divisor of the chunk count, or 32/64
// with a partial last step), row groups per task RT (1, 2) and waves per CU W
// (1..8).  Tasks are dealt round-robin to n_cu * W waves, so a CU's critical
// path is ceil(tasks / (n_cu W)) tasks per wave; the cost of a candidate is
// that times W waves times the loads of one task.  Activations staged as
// float32 (128 LDS bytes per chunk, read once per step for the RT row groups
// of a task) add one load's worth per step: taller tasks share those reads.
// The cheapest wins (ties: larger RT, then more waves).  A residual row (MoE down) must fit the
// workgroup's one-pass staging: 4 vectors of 16 bytes per thread.
constexpr double kPlanTie = 0.02;
template <class TasksFor>
GemvPlan plan_gemv(int cpr, int n_cu, int xmode, int64_t residual_rows, TasksFor tasks_for,
                   int tt = 1, int max_rt = 2) {
  GemvPlan best{};
  best.tt = tt;
  double best_cost = 1e300;
  int cand_l[3] = {lanes_for(cpr), 0, 0};
  int nl = 1;
  for (int l : {32, 64})
    if (cpr > l && cpr % l != 0 && l > cand_l[0]) cand_l[nl++] = l;
  const int xq_octets = xm_octets(xmode) * 64;  // octets one wave stages without a stall
  const double x_reads = xmode == XM_BF16 ? 0.0 : 1.0;  // LDS activation reads per step
  for (int li = 0; li < nl; ++li) {
    const int L = cand_l[li];
    const int spt = (cpr + L - 1) / L;
    const size_t lds = gemv_lds_bytes(xmode, spt * L, residual_rows, tt);
    if (lds > (size_t)kMaxLds) continue;
    for (int rt = 1; rt <= max_rt; ++rt) {
      const int64_t n_tasks = tasks_for(rt * (64 / L));
      for (int w = 1; w <= std::min(kMaxWaves, gemv_max_waves(tt)); ++w) {
        if (residual_rows > (int64_t)w * 64 * 4 * 4) continue;
        const int64_t grid = std::min<int64_t>(n_cu, (n_tasks + w - 1) / w);
        const int64_t nw = grid * w;
        const int64_t tpw = (n_tasks + nw - 1) / nw;
        double cost = (double)tpw * w * spt * (rt + x_reads);
        if ((int64_t)cpr * 4 > (int64_t)xq_octets * w) cost *= 1.5;  // staging needs extra rounds
        const bool better = cost < best_cost * (1 - kPlanTie) ||
                            (cost <= best_cost * (1 + kPlanTie) &&
                             (rt > best.rt || (rt == best.rt && w > best.waves)));
        if (better) {
          best_cost = cost;
          best.waves = w;
          best.rt = rt;
          best.log2_lpr = ilog2(L);
          best.spt = spt;
          best.n_tasks = n_tasks;
          best.grid = grid;
          best.lds_bytes = lds;
        }
      }
    }
  }
  return best;
}

// Fill the geometry fields of GemvParams from a plan.
void set_geometry(GemvParams &p, const GemvPlan &plan, int cpr, int ncx, int64_t kwb, int64_t sbrow,
                  int group_size) {
  const int L = 1 << plan.log2_lpr;
  p.log2_lpr = plan.log2_lpr;
  p.log2_group = ilog2(group_size);
  p.spt = plan.spt;
  p.rpt = plan.rt * (64 / L);
  p.last_lanes = cpr - (plan.spt - 1) * L;
  p.ncx = ncx;
  p.ncx_pad = plan.spt * L;
  p.kwb = (int32_t)kwb;
  p.sbrow = (int32_t)sbrow;
  p.n_tasks = (int32_t)plan.n_tasks;
  p.waves_per_wg = plan.waves;
  p.n_waves = (int32_t)(plan.grid * plan.waves);
  p.tasks_q = (int32_t)(plan.n_tasks / p.n_waves);
  p.tasks_r = (int32_t)(plan.n_tasks % p.n_waves);
}

// Token-count template of a launch of nt activation rows.
int tt_for(int64_t nt) { return nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : nt <= 8 ? 8 : 16; }

int multi_xmode(int32_t x_dtype, bool rms) {
  return rms ? (x_dtype == QINT4_BF16 ? XM_RMS_BF16 : XM_RMS_F32)
             : (x_dtype == QINT4_BF16 ? XM_BF16 : XM_F32);
}

// What a qgemv_int4 / _multi / rms_norm_qgemv_int4 / _smallm call launches,
// from its shapes alone: the calls follow it and the plan query reports it.
struct MultiPlan {
  bool mfma = false;  // small-M MFMA tiles of 16 rows
  int blk = 0;        // activation rows per launch
  int64_t tiles = 0;  // MFMA: tiles per launch
  int64_t grid = 0;   // MFMA: workgroups per launch (each takes tiles i, i + grid, ...);
                      // XS: workgroups (each takes rows b, b + grid, ...)
  bool xs = false;    // activation-stationary GEMV (T = 1)
  int32_t wg0[kXsMaxMats + 1] = {};  // XS: each matrix's workgroups
  GemvPlan plan{};    // otherwise: the persistent GEMV plan
};

// n_outs matrices of n_out[i] rows (the gate/up pair: the gate alone) over
// k_in columns; T activation rows of x_dtype; rms: the RMSNorm prologue;
// batched: a qgemv_int4_smallm call.
qint4_status plan_multi(int n_outs, const int64_t *n_out, int64_t k_in, int group_size,
                        int32_t x_dtype, int64_t T, bool swiglu, bool rms, bool batched, int n_cu,
                        MultiPlan *mp) {
  *mp = MultiPlan{};
  const int streams = swiglu ? 2 : 1;
  if (batched && !rms && x_dtype == QINT4_BF16 && gemv_mfma_supported(k_in, group_size, streams)) {
    int64_t tiles = 0;
    for (int i = 0; i < n_outs; ++i) tiles += (n_out[i] + 15) / 16;
    if (tiles > INT32_MAX) return fail(QINT4_ERR_SHAPE, "too many rows");
    mp->mfma = true;
    mp->tiles = tiles;
    // all T rows in one launch (16 tokens fill the MFMA's rows) when their
    // staged activations fit in LDS, else blocks of 8 rows; a row's result is
    // the same either way
    mp->blk = (T > kMaxTokens &&
               gemv_mfma_lds_bytes(QINT4_SMALLM_MAX, group_size, k_in, streams) > (size_t)kMaxLds)
                  ? kMaxTokens
                  : QINT4_SMALLM_MAX;
    // From 8 tokens on, staging the activation slices costs about as much as a
    // tile: as many workgroups as the CUs hold at once (LDS, and 16 waves per
    // CU at the kernel's 128 registers), each staging once for all of its
    // tiles (17408 x 5120 gate/up pair at T = 8: 42 -> 38 us; q/k/v at
    // T = 16: 13.2 -> 10.1 us).  Up to 4 tokens a workgroup per tile is
    // faster (the pair at T = 1..4: 30-32 us against 38 us).
    const int tt = tt_for(std::min<int64_t>(T, mp->blk));
    const size_t lds = gemv_mfma_lds_bytes(tt, group_size, k_in, streams);
    const int ks = gemv_mfma_waves(k_in);
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>((int64_t)(kMaxLds / lds), 16 / ks));
    mp->grid = std::min<int64_t>(tiles, per_cu * n_cu);  // launches of 8 or more tokens
    return QINT4_OK;
  }
  // Matrices with stored outputs, or the gate/up pair, over long rows: each
  // wave holds its slice of x in registers (dense FFN 5120 -> 17408 -> 5120:
  // gate/up 22.6 -> 20.6 us, float32 down 16.3 -> 12.5 us; bf16 activations,
  // one matrix: 5120 x 17408 14.5 -> 11.1 us, 17408 x 5120 14.1 -> 11.3 us,
  // 2048 x 32768 12.3 -> 8.0 us; where it applies: gemv_xs_plan), with or
  // without the RMSNorm prologue.  (Not for small-M calls, whose rows must not
  // depend on T.)
  if (!batched && T == 1 && n_outs <= kXsMaxMats &&
      gemv_xs_plan(n_outs, n_out, k_in, streams, n_cu, mp->wg0)) {
    mp->xs = true;
    mp->blk = 1;
    mp->grid = mp->wg0[n_outs];
    return QINT4_OK;
  }
  const int nc = (int)(k_in / 32);
  const int xmode = multi_xmode(x_dtype, rms);
  auto tasks_for = [&](int rpt) {
    int64_t t = 0;
    for (int i = 0; i < n_outs; ++i) t += (n_out[i] + rpt - 1) / rpt;
    return t;
  };
  // the RMSNorm partial sums take one LDS float per wave; blocks of at most
  // kMaxTokens rows per launch, fewer where that many staged rows do not fit
  // in LDS (each row's result is the same whatever the block)
  int tt = tt_for(std::min<int64_t>(T, kMaxTokens));
  GemvPlan plan = plan_gemv(nc, n_cu, xmode, rms ? kMaxWaves : 0, tasks_for, tt);
  while (plan.waves == 0 && tt > 1) {
    tt /= 2;
    plan = plan_gemv(nc, n_cu, xmode, rms ? kMaxWaves : 0, tasks_for, tt);
  }
  if (plan.waves == 0)
    return fail(QINT4_ERR_SHAPE, "k_in %lld with T = %lld needs more than %d bytes of LDS",
                (long long)k_in, (long long)T, kMaxLds);
  if (plan.n_tasks > INT32_MAX) return fail(QINT4_ERR_SHAPE, "too many rows");
  mp->plan = plan;
  mp->blk = tt;
  return QINT4_OK;
}

// The two launches of an expert-gather decode call: gate/up of every kept
// expert (routed: ranking the logits itself) and the down projection with the
// weighted combine (residual: adding a residual row).
qint4_status plan_moe(int64_t hidden, int64_t inter, int32_t top_k, int32_t act_dtype, bool routed,
                      bool residual, int n_cu, GemvPlan *gate_up, GemvPlan *down) {
  const int xmode_a = act_dtype == QINT4_BF16 ? XM_BF16 : XM_F32;
  auto gu_tasks = [&](int rpt) { return (int64_t)top_k * ((inter + rpt - 1) / rpt); };
  // routing in the gate/up launch: 16 floats of LDS hand the ranked ids to every wave
  *gate_up = plan_gemv((int)(hidden / 32), n_cu, xmode_a, routed ? 16 : 0, gu_tasks);
  if (gate_up->waves == 0) return fail(QINT4_ERR_SHAPE, "hidden %lld needs too much LDS", (long long)hidden);
  // the down projection takes one row group per task: twice the waves of
  // two-row tasks, so two waves per SIMD overlap their dot products and
  // reductions (128 experts, top-8, 2048 x 768: 0.2-0.5 us faster per step,
  // although two-row tasks share their LDS activation reads)
  auto down_tasks = [&](int rpt) { return (hidden + rpt - 1) / rpt; };
  *down = plan_gemv((int)(inter / 32) * top_k, n_cu, XM_F32, residual ? hidden : 0, down_tasks, 1, 1);
  if (down->waves == 0)
    return fail(QINT4_ERR_SHAPE, "top_k * inter = %lld needs too much LDS", (long long)(top_k * inter));
  if (gate_up->n_tasks > INT32_MAX || down->n_tasks > INT32_MAX)
    return fail(QINT4_ERR_SHAPE, "too many rows");
  return QINT4_OK;
}

// The form a planned persistent GEMV launch takes.
void ring_form(const GemvPlan &plan, int xmode, int epi, int64_t launches, qint4_gemv_form *f) {
  std::memset(f, 0, sizeof(*f));
  f->kernel = QINT4_FORM_RING;
  f->tokens = plan.tt;
  f->launches = launches;
  f->waves = plan.waves;
  f->grid = plan.grid;
  f->tasks = plan.n_tasks;
  f->lanes = 1 << plan.log2_lpr;
  f->rows_per_task = plan.rt * (64 >> plan.log2_lpr);
  f->steps_per_task = plan.spt;
  f->busiest_wave_steps = gemv_busiest_steps(plan);
  f->ring_depth = gemv_ring_depth(plan, xmode, epi);
}

}  // namespace

extern "C" {

const char *qint4_status_string(int32_t status) {
  switch (status) {
    case QINT4_OK: return "ok";
    case QINT4_ERR_NULL: return "null pointer";
    case QINT4_ERR_SHAPE: return "invalid shape";
    case QINT4_ERR_DTYPE: return "invalid dtype";
    case QINT4_ERR_ALIGN: return "misaligned pointer";
    case QINT4_ERR_ALIAS: return "output overlaps input";
    case QINT4_ERR_WORKSPACE: return "workspace missing or too small";
    case QINT4_ERR_DEVICE: return "no gfx950 device";
    case QINT4_ERR_LAUNCH: return "kernel launch failed";
    case QINT4_ERR_VALUE: return "scalar argument out of range";
    default: return "unknown status";
  }
}

const char *qint4_last_error(void) { return g_last_error; }

int32_t qint4_abi_version(void) { return QINT4_ABI_VERSION; }

}  // extern "C"

namespace {

// Shared body of qgemv_int4, qgemv_int4_multi and qgemv_int4_smallm: T
// activation rows x + t * ldx (T = 1: the plain GEMV).
// gamma != NULL: RMSNorm prologue (T must be 1).
// batched: a qgemv_int4_smallm call, whose rows must not depend on T (the
// stored-output bf16 form then runs on MFMA for every T, T = 1 included).
qint4_status run_multi(int32_t n, const qint4_matrix *ws, const void *x, int32_t x_dtype,
                       int64_t T, int64_t ldx, void *const *ys, int32_t y_dtype, int32_t epilogue,
                       hipStream_t stream, const char *fn, const void *gamma = nullptr,
                       float eps = 0.f, bool batched = false) {
  if (n < 1 || n > QINT4_MULTI_MAX)
    return fail(QINT4_ERR_SHAPE, "%s: n = %d not in [1, %d]", fn, n, QINT4_MULTI_MAX);
  if (!ws) return fail(QINT4_ERR_NULL, "%s: matrix array is NULL", fn);
  if (!ys) return fail(QINT4_ERR_NULL, "%s: output array is NULL", fn);
  if (!x) return fail(QINT4_ERR_NULL, "%s: x is NULL", fn);
  if (!valid_dtype(x_dtype)) return fail(QINT4_ERR_DTYPE, "%s: x_dtype %d invalid", fn, x_dtype);
  if (!valid_dtype(y_dtype)) return fail(QINT4_ERR_DTYPE, "%s: y_dtype %d invalid", fn, y_dtype);
  if (epilogue != QINT4_EPI_NONE && epilogue != QINT4_EPI_SWIGLU_PAIR)
    return fail(QINT4_ERR_SHAPE, "%s: epilogue %d invalid", fn, epilogue);
  char name[32];
  for (int i = 0; i < n; ++i) {
    snprintf(name, sizeof(name), "ws[%d]", i);
    qint4_status st = check_matrix(&ws[i], name, false);
    if (st != QINT4_OK) return st;
  }
  for (int i = 1; i < n; ++i) {
    if (ws[i].k_in != ws[0].k_in)
      return fail(QINT4_ERR_SHAPE,
                  "%s: packed width mismatch: ws[%d].k_in = %lld (%lld words) but ws[0].k_in = %lld "
                  "(%lld words)",
                  fn, i, (long long)ws[i].k_in, (long long)ws[i].k_in / 8, (long long)ws[0].k_in,
                  (long long)ws[0].k_in / 8);
    if (ws[i].group_size != ws[0].group_size)
      return fail(QINT4_ERR_SHAPE, "%s: ws[%d].group_size %d != ws[0].group_size %d", fn, i,
                  ws[i].group_size, ws[0].group_size);
    if (ws[i].sb_dtype != ws[0].sb_dtype)
      return fail(QINT4_ERR_DTYPE, "%s: ws[%d].sb_dtype differs from ws[0]", fn, i);
  }
  const bool swiglu = epilogue == QINT4_EPI_SWIGLU_PAIR;
  if (swiglu) {
    if (n != 2) return fail(QINT4_ERR_SHAPE, "%s: SWIGLU_PAIR needs n == 2, got %d", fn, n);
    if (ws[0].n_out != ws[1].n_out)
      return fail(QINT4_ERR_SHAPE, "%s: SWIGLU_PAIR gate n_out %lld != up n_out %lld", fn,
                  (long long)ws[0].n_out, (long long)ws[1].n_out);
    if (!ys[0]) return fail(QINT4_ERR_NULL, "%s: ys[0] is NULL", fn);
  } else {
    for (int i = 0; i < n; ++i)
      if (!ys[i]) return fail(QINT4_ERR_NULL, "%s: ys[%d] is NULL", fn, i);
  }
  if (!aligned(x, 16)) return fail(QINT4_ERR_ALIGN, "%s: x not 16-byte aligned", fn);
  const int n_outs = swiglu ? 1 : n;
  for (int i = 0; i < n_outs; ++i)
    if (!aligned(ys[i], elem_bytes(y_dtype)))
      return fail(QINT4_ERR_ALIGN, "%s: ys[%d] not aligned to its element size", fn, i);
  if (T < 1 || T > QINT4_SMALLM_MAX)
    return fail(QINT4_ERR_SHAPE, "%s: T = %lld not in [1, %d]", fn, (long long)T, QINT4_SMALLM_MAX);
  if (T > 1 && x_dtype != QINT4_BF16)
    return fail(QINT4_ERR_DTYPE, "%s: T > 1 needs bfloat16 activations", fn);
  if (T > 1 && (ldx < ws[0].k_in || ldx % 8 != 0))
    return fail(QINT4_ERR_SHAPE, "%s: ldx %lld must be >= k_in %lld and a multiple of 8", fn,
                (long long)ldx, (long long)ws[0].k_in);
  // every kernel of this family addresses the activation rows through 32-bit
  // element strides and byte offsets
  if (((T - 1) * ldx + ws[0].k_in) * (int64_t)elem_bytes(x_dtype) >= ((int64_t)1 << 31))
    return fail(QINT4_ERR_SHAPE, "%s: activation rows span 2 GiB or more (ldx %lld)", fn,
                (long long)ldx);

  if (gamma) {
    if (T != 1) return fail(QINT4_ERR_SHAPE, "%s: the RMSNorm prologue takes one row", fn);
    if (!aligned(gamma, 16)) return fail(QINT4_ERR_ALIGN, "%s: gamma not 16-byte aligned", fn);
    if (!(eps > 0.f) || eps > 3.4e38f)
      return fail(QINT4_ERR_VALUE, "%s: eps %g must be finite and > 0", fn, (double)eps);
  }

  // overlap checks
  Range ins[3 * QINT4_MULTI_MAX + 2], outs[QINT4_MULTI_MAX];
  int ni = 0;
  static const char *mnames[3] = {"codes", "scales", "biases"};
  for (int i = 0; i < n; ++i) ni += add_matrix_ranges(&ws[i], mnames, ins + ni);
  const int64_t k_in = ws[0].k_in;
  ins[ni++] = range(x, (size_t)((T - 1) * ldx + k_in) * elem_bytes(x_dtype), "x");
  if (gamma) ins[ni++] = range(gamma, (size_t)k_in * elem_bytes(x_dtype), "gamma");
  static const char *ynames[QINT4_MULTI_MAX] = {"ys[0]", "ys[1]", "ys[2]", "ys[3]",
                                                  "ys[4]", "ys[5]", "ys[6]", "ys[7]"};
  for (int i = 0; i < n_outs; ++i)
    outs[i] = range(ys[i], (size_t)T * ws[i].n_out * elem_bytes(y_dtype), ynames[i]);
  qint4_status st = check_no_overlap(outs, n_outs, ins, ni);
  if (st != QINT4_OK) return prefixed(st, fn);

  // plan
  const int nc = (int)(k_in / 32);
  const int xmode = multi_xmode(x_dtype, gamma != nullptr);
  const int epi = swiglu ? EPI_SWIGLU : EPI_STORE;
  const int sb_bf16 = ws[0].sb_dtype == QINT4_BF16;
  int n_cu = 256;
  st = check_device(&n_cu);
  if (st != QINT4_OK) return prefixed(st, fn);
  int64_t n_out[QINT4_MULTI_MAX];
  for (int i = 0; i < n_outs; ++i) n_out[i] = ws[i].n_out;
  MultiPlan mp;
  st = plan_multi(n_outs, n_out, k_in, ws[0].group_size, x_dtype, T, swiglu, gamma != nullptr,
                  batched, n_cu, &mp);
  if (st != QINT4_OK) return prefixed(st, fn);
  const size_t yb = elem_bytes(y_dtype);
  const int64_t sbrow_b = (k_in / ws[0].group_size) * (int64_t)elem_bytes(ws[0].sb_dtype);

  // small-M calls with bf16 activations (stored outputs or the gate/up pair):
  // MFMA tiles of 16 rows when the shape allows, for every T alike (so a T-row
  // call equals T one-row calls)
  if (mp.mfma) {
    GemvParams p;
    std::memset(&p, 0, sizeof(p));
    p.n_mats = n;
    int64_t tiles = 0;
    for (int i = 0; i < kMaxMats; ++i) p.task0[i] = INT32_MAX;
    for (int i = 0; i < n; ++i) {
      p.m[i].codes = ws[i].codes;
      p.m[i].scales = ws[i].scales;
      p.m[i].biases = ws[i].biases;
      p.m[i].y = swiglu ? ys[0] : ys[i];
      p.m[i].n_out = ws[i].n_out;
      if (swiglu && i > 0) continue;  // the pair shares the gate's tiles
      p.task0[i] = (int32_t)tiles;
      tiles += (ws[i].n_out + 15) / 16;
    }
    p.n_tasks = (int32_t)tiles;
    p.kwb = (int32_t)(k_in / 2);
    p.sbrow = (int32_t)sbrow_b;
    p.log2_group = ilog2(ws[0].group_size);
    p.ncx = (int32_t)(k_in / 32);
    p.waves_per_wg = gemv_mfma_waves(k_in);
    p.ldx = (int32_t)ldx;
    p.y_bf16 = y_dtype == QINT4_BF16;
    for (int64_t t0 = 0; t0 < T; t0 += mp.blk) {
      const int64_t nt = std::min<int64_t>(mp.blk, T - t0);
      p.n_tok = (int32_t)nt;
      p.x = reinterpret_cast<const unsigned char *>(x) + (size_t)t0 * ldx * 2;
      for (int i = 0; i < n; ++i)
        p.m[i].y = reinterpret_cast<unsigned char *>(swiglu ? ys[0] : ys[i]) +
                   (size_t)t0 * (swiglu ? ws[0].n_out : ws[i].n_out) * yb;
      const int tt = tt_for(nt);
      hipError_t e = launch_gemv_mfma(p, tt, ws[0].group_size, sb_bf16, swiglu ? 1 : 0,
                                      tt <= 4 ? tiles : mp.grid, stream);
      if (e != hipSuccess) return fail(QINT4_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
    }
    return ok();
  }

  if (mp.xs) {
    GemvXsParams p;
    std::memset(&p, 0, sizeof(p));
    for (int i = 0; i < n; ++i) {  // the matrices, or the pair's gate and up
      p.codes[i] = ws[i].codes;
      p.scales[i] = ws[i].scales;
      p.biases[i] = ws[i].biases;
    }
    for (int i = 0; i < n_outs; ++i) {
      p.y[i] = ys[i];
      p.n_out[i] = (int32_t)ws[i].n_out;
    }
    for (int i = 0; i <= n_outs; ++i) p.wg0[i] = mp.wg0[i];
    p.n_mats = n_outs;
    p.x = x;
    p.gamma = gamma;
    p.eps = eps;
    p.ncx = (int32_t)(k_in / 32);
    p.kwb = (int32_t)(k_in / 2);
    p.sbrow = (int32_t)sbrow_b;
    p.log2_group = ilog2(ws[0].group_size);
    p.log2_lpr = gemv_xs_log2_lanes(k_in);
    p.waves = gemv_xs_waves(k_in);
    p.y_bf16 = y_dtype == QINT4_BF16;
    hipError_t e = launch_gemv_xs(p, sb_bf16, x_dtype == QINT4_BF16, swiglu ? 2 : 1, stream);
    if (e != hipSuccess) return fail(QINT4_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
  }

  const GemvPlan &plan = mp.plan;
  const int tt = mp.blk;
  const int rpt = plan.rt * (64 >> plan.log2_lpr);

  GemvParams p;
  std::memset(&p, 0, sizeof(p));
  p.n_mats = swiglu ? 2 : n;
  int64_t t0 = 0;
  for (int i = 0; i < kMaxMats; ++i) p.task0[i] = INT32_MAX;
  for (int i = 0; i < n; ++i) {
    p.m[i].codes = ws[i].codes;
    p.m[i].scales = ws[i].scales;
    p.m[i].biases = ws[i].biases;
    p.m[i].y = swiglu ? ys[0] : ys[i];
    p.m[i].n_out = ws[i].n_out;
    p.task0[i] = (int32_t)t0;
    if (!swiglu) t0 += (ws[i].n_out + rpt - 1) / rpt;
  }
  const int64_t sbrow = (k_in / ws[0].group_size) * (int64_t)elem_bytes(ws[0].sb_dtype);
  set_geometry(p, plan, nc, nc, k_in / 2, sbrow, ws[0].group_size);
  p.y_bf16 = y_dtype == QINT4_BF16;
  p.aux = gamma;
  p.eps = eps;
  p.ldx = (int32_t)ldx;
  p.ids = nullptr;
  p.top_k = 1;
  p.n_experts = 1;
  p.tasks_per_slot = (int32_t)plan.n_tasks;

  for (int64_t t0 = 0; t0 < T; t0 += tt) {
    const int64_t nt = std::min<int64_t>(tt, T - t0);
    p.n_tok = (int32_t)nt;
    p.x = reinterpret_cast<const unsigned char *>(x) + (size_t)t0 * ldx * elem_bytes(x_dtype);
    for (int i = 0; i < n; ++i)
      p.m[i].y = reinterpret_cast<unsigned char *>(swiglu ? ys[0] : ys[i]) +
                 (size_t)t0 * (swiglu ? ws[0].n_out : ws[i].n_out) * yb;
    hipError_t e = launch_gemv(p, plan, xmode, sb_bf16, epi, stream);
    if (e != hipSuccess) return fail(QINT4_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

qint4_status qgemv_int4(const qint4_matrix *w, const void *x, int32_t x_dtype, void *y,
                        int32_t y_dtype, void *stream) {
  if (!w) return fail(QINT4_ERR_NULL, "qgemv_int4: matrix descriptor is NULL");
  void *ys[1] = {y};
  if (!y) return fail(QINT4_ERR_NULL, "qgemv_int4: y is NULL");
  return run_multi(1, w, x, x_dtype, 1, w->k_in, ys, y_dtype, QINT4_EPI_NONE,
                   reinterpret_cast<hipStream_t>(stream), "qgemv_int4");
}

qint4_status qgemv_int4_multi(int32_t n, const qint4_matrix *ws, const void *x, int32_t x_dtype,
                              void *const *ys, int32_t y_dtype, int32_t epilogue, void *stream) {
  return run_multi(n, ws, x, x_dtype, 1, (n >= 1 && ws) ? ws[0].k_in : 0, ys, y_dtype, epilogue,
                   reinterpret_cast<hipStream_t>(stream), "qgemv_int4_multi");
}

qint4_status rms_norm_qgemv_int4(int32_t n, const qint4_matrix *ws, const void *x,
                                 int32_t x_dtype, const void *gamma, float eps,
                                 void *const *ys, int32_t y_dtype, int32_t epilogue,
                                 void *stream) {
  if (!gamma) return fail(QINT4_ERR_NULL, "rms_norm_qgemv_int4: gamma is NULL");
  return run_multi(n, ws, x, x_dtype, 1, (n >= 1 && ws) ? ws[0].k_in : 0, ys, y_dtype, epilogue,
                   reinterpret_cast<hipStream_t>(stream), "rms_norm_qgemv_int4", gamma, eps);
}

qint4_status qgemv_int4_smallm(int32_t n, const qint4_matrix *ws, const void *x, int32_t x_dtype,
                               int64_t T, int64_t ldx, void *const *ys, int32_t y_dtype,
                               int32_t epilogue, void *stream) {
  return run_multi(n, ws, x, x_dtype, T, ldx, ys, y_dtype, epilogue,
                   reinterpret_cast<hipStream_t>(stream), "qgemv_int4_smallm", nullptr, 0.f,
                   true);
}

size_t moe_gather_qgemv_int4_workspace_bytes(const qint4_matrix *down, int32_t top_k) {
  return down ? moe_ws_bytes(down->k_in, top_k) : 0;
}

}  // extern "C"

namespace {

// Shared body of moe_gather_qgemv_int4 and moe_route_gather_qgemv_int4
// (logits != NULL: the gate/up launch ranks the logits itself and writes ids
// and wts, which the down launch then reads).
qint4_status run_moe(const qint4_matrix *gate, const qint4_matrix *up, const qint4_matrix *down,
                     const void *x, const uint32_t *ids, const float *wts, int32_t top_k,
                     const void *residual, void *out, int32_t act_dtype, void *workspace,
                     size_t workspace_bytes, hipStream_t stream, const char *fn,
                     const void *logits, int32_t logits_dtype) {
  qint4_status st;
  if ((st = check_matrix(gate, "gate", true)) != QINT4_OK) return st;
  if ((st = check_matrix(up, "up", true)) != QINT4_OK) return st;
  if ((st = check_matrix(down, "down", true)) != QINT4_OK) return st;
  if (!x || !ids || !wts || !out) return fail(QINT4_ERR_NULL, "%s: x/ids/wts/out is NULL", fn);
  if (!valid_dtype(act_dtype)) return fail(QINT4_ERR_DTYPE, "%s: act_dtype %d invalid", fn, act_dtype);
  if (top_k < 1 || top_k > QINT4_TOPK_MAX)
    return fail(QINT4_ERR_SHAPE, "%s: top_k %d not in [1, %d]", fn, top_k, QINT4_TOPK_MAX);
  if (gate->n_experts != up->n_experts || gate->n_experts != down->n_experts)
    return fail(QINT4_ERR_SHAPE, "%s: n_experts differ (gate %d, up %d, down %d)", fn,
                gate->n_experts, up->n_experts, down->n_experts);
  if (gate->group_size != up->group_size || gate->group_size != down->group_size ||
      gate->sb_dtype != up->sb_dtype || gate->sb_dtype != down->sb_dtype)
    return fail(QINT4_ERR_SHAPE, "%s: gate/up/down must share group_size and sb_dtype", fn);
  const int64_t hidden = gate->k_in, inter = gate->n_out;
  if (up->k_in != hidden || up->n_out != inter)
    return fail(QINT4_ERR_SHAPE, "%s: up is %lldx%lld, gate is %lldx%lld", fn, (long long)up->n_out,
                (long long)up->k_in, (long long)inter, (long long)hidden);
  if (down->k_in != inter || down->n_out != hidden)
    return fail(QINT4_ERR_SHAPE, "%s: down is %lldx%lld, expected %lldx%lld", fn,
                (long long)down->n_out, (long long)down->k_in, (long long)hidden, (long long)inter);
  if (!aligned(x, 16)) return fail(QINT4_ERR_ALIGN, "%s: x not 16-byte aligned", fn);
  if (!aligned(ids, 4) || !aligned(wts, 4)) return fail(QINT4_ERR_ALIGN, "%s: ids/wts misaligned", fn);
  const size_t ab = elem_bytes(act_dtype);
  if (!aligned(out, ab) || (residual && !aligned(residual, ab)))
    return fail(QINT4_ERR_ALIGN, "%s: out/residual not aligned to element size", fn);
  if (logits) {
    if (!valid_dtype(logits_dtype))
      return fail(QINT4_ERR_DTYPE, "%s: logits_dtype %d invalid", fn, logits_dtype);
    if (gate->n_experts > kRouteMaxExperts || gate->n_experts < top_k)
      return fail(QINT4_ERR_SHAPE,
                  "%s: routing in the gate/up launch needs top_k <= n_experts <= %d (got %d); "
                  "use moe_router_topk + moe_gather_qgemv_int4",
                  fn, kRouteMaxExperts, gate->n_experts);
    if (!aligned(logits, elem_bytes(logits_dtype)))
      return fail(QINT4_ERR_ALIGN, "%s: logits not aligned to its element size", fn);
  }
  const size_t need = moe_ws_bytes(inter, top_k);
  if (!workspace || workspace_bytes < need)
    return fail(QINT4_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn,
                workspace ? workspace_bytes : (size_t)0, need);
  if (!aligned(workspace, 16)) return fail(QINT4_ERR_ALIGN, "%s: workspace not 16-byte aligned", fn);

  Range ins[14], outs[4];
  int ni = 0, no = 0;
  static const char *gn[3] = {"gate.codes", "gate.scales", "gate.biases"};
  static const char *un[3] = {"up.codes", "up.scales", "up.biases"};
  static const char *dn[3] = {"down.codes", "down.scales", "down.biases"};
  ni += add_matrix_ranges(gate, gn, ins + ni);
  ni += add_matrix_ranges(up, un, ins + ni);
  ni += add_matrix_ranges(down, dn, ins + ni);
  ins[ni++] = range(x, (size_t)hidden * ab, "x");
  if (logits) {  // ids and wts are outputs
    ins[ni++] = range(logits, (size_t)gate->n_experts * elem_bytes(logits_dtype), "logits");
    outs[no++] = range(ids, (size_t)top_k * 4, "ids");
    outs[no++] = range(wts, (size_t)top_k * 4, "wts");
  } else {
    ins[ni++] = range(ids, (size_t)top_k * 4, "ids");
    ins[ni++] = range(wts, (size_t)top_k * 4, "wts");
  }
  if (residual) ins[ni++] = range(residual, (size_t)hidden * ab, "residual");
  outs[no++] = range(out, (size_t)hidden * ab, "out");
  outs[no++] = range(workspace, need, "workspace");
  if ((st = check_no_overlap(outs, no, ins, ni)) != QINT4_OK) return prefixed(st, fn);

  int n_cu = 256;
  if ((st = check_device(&n_cu)) != QINT4_OK) return prefixed(st, fn);

  const int sb_bf16 = gate->sb_dtype == QINT4_BF16;
  const int xmode_a = act_dtype == QINT4_BF16 ? XM_BF16 : XM_F32;
  float *h = reinterpret_cast<float *>(workspace);
  GemvPlan plan_a, plan_b;
  st = plan_moe(hidden, inter, top_k, act_dtype, logits != nullptr, residual != nullptr, n_cu, &plan_a,
                &plan_b);
  if (st != QINT4_OK) return prefixed(st, fn);

  // ---- launch A: gate/up of every kept expert, SwiGLU -> h[top_k][inter] (f32) ----
  {
    const int nc = (int)(hidden / 32);
    const GemvPlan &plan = plan_a;
    const int rpt = plan.rt * (64 >> plan.log2_lpr);
    GemvParams p;
    std::memset(&p, 0, sizeof(p));
    p.n_mats = 2;
    p.m[0] = {gate->codes, gate->scales, gate->biases, h, inter};
    p.m[1] = {up->codes, up->scales, up->biases, h, inter};
    const int64_t sbrow = (hidden / gate->group_size) * (int64_t)elem_bytes(gate->sb_dtype);
    set_geometry(p, plan, nc, nc, hidden / 2, sbrow, gate->group_size);
    p.y_bf16 = 0;
    p.n_tok = 1;
    p.tasks_per_slot = (int32_t)((inter + rpt - 1) / rpt);
    p.x = x;
    p.ids = const_cast<uint32_t *>(ids);  // written only when routing
    p.wts = const_cast<float *>(wts);
    p.aux = logits;
    p.route = logits ? (logits_dtype == QINT4_BF16 ? 2 : 1) : 0;
    p.top_k = top_k;
    p.n_experts = gate->n_experts;
    p.ecode_bytes = (uint32_t)(inter * (hidden / 2));
    p.esb_bytes = (uint32_t)(inter * sbrow);
    hipError_t e = launch_gemv(p, plan, xmode_a, sb_bf16, EPI_SWIGLU, stream);
    if (e != hipSuccess) return fail(QINT4_ERR_LAUNCH, "%s: gate/up launch failed: %s", fn, hipGetErrorString(e));
  }
  // ---- launch B: down projection of every slot + weighted combine + residual ----
  {
    const int ncl = (int)(inter / 32);
    const int ncv = ncl * top_k;
    const GemvPlan &plan = plan_b;
    GemvParams p;
    std::memset(&p, 0, sizeof(p));
    p.n_mats = 1;
    p.m[0] = {down->codes, down->scales, down->biases, out, hidden};
    const int64_t sbrow = (inter / down->group_size) * (int64_t)elem_bytes(down->sb_dtype);
    set_geometry(p, plan, ncv, ncv, inter / 2, sbrow, down->group_size);
    p.y_bf16 = act_dtype == QINT4_BF16;
    p.n_tok = 1;
    p.x = h;
    p.ids = const_cast<uint32_t *>(ids);  // read only
    p.wts = const_cast<float *>(wts);
    p.aux = residual;
    p.top_k = top_k;
    p.n_experts = down->n_experts;
    p.cpr_e = ncl;
    p.inv_cpr_e = 1.0f / (float)ncl;
    p.ecode_bytes = (uint32_t)(hidden * (inter / 2));
    p.esb_bytes = (uint32_t)(hidden * sbrow);
    p.code_bytes = (uint32_t)code_bytes(down);
    p.sb_bytes = (uint32_t)sb_bytes(down);
    hipError_t e = launch_gemv(p, plan, XM_F32, sb_bf16, EPI_MOE_DOWN, stream);
    if (e != hipSuccess) return fail(QINT4_ERR_LAUNCH, "%s: down launch failed: %s", fn, hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

qint4_status moe_gather_qgemv_int4(const qint4_matrix *gate, const qint4_matrix *up,
                                   const qint4_matrix *down, const void *x, const uint32_t *ids,
                                   const float *wts, int32_t top_k, const void *residual, void *out,
                                   int32_t act_dtype, void *workspace, size_t workspace_bytes,
                                   void *stream) {
  return run_moe(gate, up, down, x, ids, wts, top_k, residual, out, act_dtype, workspace,
                 workspace_bytes, reinterpret_cast<hipStream_t>(stream), "moe_gather_qgemv_int4",
                 nullptr, 0);
}

}  // extern "C"

namespace {

// The scratch of moe_gather_qgemv_int4_noalloc: one copy on every GPU the
// library runs on.  Host code never uses this name as an address (on the host
// it is only a stand-in for the symbol); it looks up each device's copy with
// hipGetSymbolAddress and passes that pointer on.
__device__ __align__(256) unsigned char scratch[QINT4_NOALLOC_SCRATCH_BYTES];

// Device address of the current device's scratch, looked up once per device
// (the current device is the one the lookup resolves for).
qint4_status scratch_address(void **out, const char *fn) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(QINT4_ERR_DEVICE, "%s: no current HIP device", fn);
  }
  if (dev >= 64) return fail(QINT4_ERR_DEVICE, "%s: device ordinal %d not supported", fn, dev);
  static std::mutex mu;
  static void *addr[64] = {};
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(QINT4_ERR_DEVICE, "%s: hipGetSymbolAddress of the scratch array failed: %s", fn,
                  hipGetErrorString(e));
    }
    addr[dev] = p;
  }
  *out = addr[dev];
  return QINT4_OK;
}

}  // namespace

extern "C" {

qint4_status moe_gather_qgemv_int4_noalloc(const qint4_matrix *gate, const qint4_matrix *up,
                                           const qint4_matrix *down, const void *x,
                                           const uint32_t *ids, const float *wts, int32_t top_k,
                                           const void *residual, void *out, int32_t act_dtype,
                                           void *stream) {
  const char *fn = "moe_gather_qgemv_int4_noalloc";
  if (!gate) return fail(QINT4_ERR_NULL, "%s: gate is NULL", fn);
  const size_t need = moe_ws_bytes(gate->n_out, top_k);
  if (need > QINT4_NOALLOC_SCRATCH_BYTES)
    return fail(QINT4_ERR_WORKSPACE,
                "%s: top_k %d x inter %lld needs %zu bytes of scratch, more than the %u the "
                "library holds per device (use moe_gather_qgemv_int4 with a workspace)",
                fn, top_k, (long long)gate->n_out, need, (unsigned)QINT4_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  qint4_status st = scratch_address(&ws, fn);
  if (st != QINT4_OK) return st;
  return run_moe(gate, up, down, x, ids, wts, top_k, residual, out, act_dtype, ws,
                 QINT4_NOALLOC_SCRATCH_BYTES, reinterpret_cast<hipStream_t>(stream), fn, nullptr, 0);
}

qint4_status moe_route_gather_qgemv_int4(const qint4_matrix *gate, const qint4_matrix *up,
                                         const qint4_matrix *down, const void *x,
                                         const void *logits, int32_t logits_dtype, int32_t top_k,
                                         const void *residual, void *out, int32_t act_dtype,
                                         uint32_t *ids, float *wts, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  if (!logits) return fail(QINT4_ERR_NULL, "moe_route_gather_qgemv_int4: logits is NULL");
  return run_moe(gate, up, down, x, ids, wts, top_k, residual, out, act_dtype, workspace,
                 workspace_bytes, reinterpret_cast<hipStream_t>(stream),
                 "moe_route_gather_qgemv_int4", logits, logits_dtype);
}

qint4_status moe_router_topk(const void *logits, int32_t logits_dtype, int64_t n_tokens,
                             int32_t n_experts, int32_t top_k, uint32_t *ids, float *wts,
                             void *stream) {
  const char *fn = "moe_router_topk";
  if (!logits || !ids || !wts) return fail(QINT4_ERR_NULL, "%s: logits/ids/wts is NULL", fn);
  if (!valid_dtype(logits_dtype))
    return fail(QINT4_ERR_DTYPE, "%s: logits_dtype %d invalid", fn, logits_dtype);
  if (top_k < 1 || top_k > QINT4_TOPK_MAX)
    return fail(QINT4_ERR_SHAPE, "%s: top_k %d not in [1, %d]", fn, top_k, QINT4_TOPK_MAX);
  if (n_experts < top_k || n_experts > kRouterMaxExperts)
    return fail(QINT4_ERR_SHAPE, "%s: n_experts %d not in [top_k = %d, %d]", fn, n_experts, top_k,
                kRouterMaxExperts);
  if (n_tokens < 1 || n_tokens > ((int64_t)1 << 31))
    return fail(QINT4_ERR_SHAPE, "%s: n_tokens %lld invalid", fn, (long long)n_tokens);
  const size_t lb = elem_bytes(logits_dtype);
  if (!aligned(logits, lb) || !aligned(ids, 4) || !aligned(wts, 4))
    return fail(QINT4_ERR_ALIGN, "%s: logits/ids/wts not aligned to their element size", fn);
  Range ins[1], outs[2];
  ins[0] = range(logits, (size_t)n_tokens * n_experts * lb, "logits");
  outs[0] = range(ids, (size_t)n_tokens * top_k * 4, "ids");
  outs[1] = range(wts, (size_t)n_tokens * top_k * 4, "wts");
  qint4_status st = check_no_overlap(outs, 2, ins, 1);
  if (st != QINT4_OK) return prefixed(st, fn);
  if ((st = check_device(nullptr)) != QINT4_OK) return prefixed(st, fn);
  hipError_t e = launch_router(logits, logits_dtype == QINT4_BF16, n_tokens, n_experts, top_k, ids,
                               wts, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(QINT4_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Workspace layout of moe_prefill_qgemm_int4 (every region 256-byte aligned).
struct PrefillWs {
  size_t perm, pos, tiles, h_hi, h_lo, d, total;
  int64_t max_tiles;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool prefill_ws(int64_t T, int32_t top_k, int32_t n_experts, int64_t hidden, int64_t inter,
                PrefillWs *w) {
  if (T < 1 || top_k < 1 || top_k > QINT4_TOPK_MAX || n_experts < 1 ||
      n_experts > kMaxExpertsPrefill || hidden < 1 || hidden > kMaxK || inter < 1 || inter > kMaxK)
    return false;
  const int64_t P = T * top_k;
  if (P > ((int64_t)1 << 24)) return false;
  // row tiles of at most 32 rows bound every tile size: ceil(P / 32) + one
  // partial tile per expert that has rows
  w->max_tiles = (P + 31) / 32 + std::min<int64_t>(n_experts, P);
  size_t o = 0;
  w->perm = o;  o = align256(o + (size_t)P * 4);
  w->pos = o;   o = align256(o + (size_t)P * 4);
  w->tiles = o; o = align256(o + (size_t)(1 + 3 * w->max_tiles) * 4);
  w->h_hi = o;  o = align256(o + (size_t)P * inter * 2);
  w->h_lo = o;  o = align256(o + (size_t)P * inter * 2);
  w->d = o;     o = align256(o + (size_t)P * hidden * 4);
  w->total = o;
  return true;
}

}  // namespace

extern "C" {

size_t moe_prefill_qgemm_int4_workspace_bytes(int64_t T, int32_t top_k, int32_t n_experts,
                                              int64_t hidden, int64_t inter) {
  PrefillWs w;
  return prefill_ws(T, top_k, n_experts, hidden, inter, &w) ? w.total : 0;
}

qint4_status moe_prefill_qgemm_int4(const qint4_matrix *gate, const qint4_matrix *up,
                                    const qint4_matrix *down, const void *x, int64_t T, int64_t ldx,
                                    const uint32_t *ids, const float *wts, int32_t top_k,
                                    const void *residual, void *out, int32_t out_dtype,
                                    void *workspace, size_t workspace_bytes, void *stream_) {
  const char *fn = "moe_prefill_qgemm_int4";
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  qint4_status st;
  if ((st = check_matrix(gate, "gate", true)) != QINT4_OK) return st;
  if ((st = check_matrix(up, "up", true)) != QINT4_OK) return st;
  if ((st = check_matrix(down, "down", true)) != QINT4_OK) return st;
  if (!x || !ids || !wts || !out) return fail(QINT4_ERR_NULL, "%s: x/ids/wts/out is NULL", fn);
  if (!valid_dtype(out_dtype)) return fail(QINT4_ERR_DTYPE, "%s: out_dtype %d invalid", fn, out_dtype);
  if (top_k < 1 || top_k > QINT4_TOPK_MAX)
    return fail(QINT4_ERR_SHAPE, "%s: top_k %d not in [1, %d]", fn, top_k, QINT4_TOPK_MAX);
  if (gate->n_experts != up->n_experts || gate->n_experts != down->n_experts)
    return fail(QINT4_ERR_SHAPE, "%s: n_experts differ (gate %d, up %d, down %d)", fn,
                gate->n_experts, up->n_experts, down->n_experts);
  if (gate->n_experts > kMaxExpertsPrefill)
    return fail(QINT4_ERR_SHAPE, "%s: n_experts %d > %d", fn, gate->n_experts, kMaxExpertsPrefill);
  if (gate->group_size != up->group_size || gate->group_size != down->group_size ||
      gate->sb_dtype != up->sb_dtype || gate->sb_dtype != down->sb_dtype)
    return fail(QINT4_ERR_SHAPE, "%s: gate/up/down must share group_size and sb_dtype", fn);
  const int64_t hidden = gate->k_in, inter = gate->n_out;
  if (up->k_in != hidden || up->n_out != inter)
    return fail(QINT4_ERR_SHAPE, "%s: up is %lldx%lld, gate is %lldx%lld", fn, (long long)up->n_out,
                (long long)up->k_in, (long long)inter, (long long)hidden);
  if (down->k_in != inter || down->n_out != hidden)
    return fail(QINT4_ERR_SHAPE, "%s: down is %lldx%lld, expected %lldx%lld", fn,
                (long long)down->n_out, (long long)down->k_in, (long long)hidden, (long long)inter);
  PrefillWs lay;
  if (T < 1 || !prefill_ws(T, top_k, gate->n_experts, hidden, inter, &lay))
    return fail(QINT4_ERR_SHAPE, "%s: T = %lld with top_k %d out of range (T * top_k <= 2^24)", fn,
                (long long)T, top_k);
  if (ldx < hidden || ldx % 8 != 0)
    return fail(QINT4_ERR_SHAPE, "%s: ldx %lld must be >= hidden %lld and a multiple of 8", fn,
                (long long)ldx, (long long)hidden);
  // the GEMMs address x and the h planes through 32-bit byte offsets
  if (T * ldx * 2 >= ((int64_t)1 << 31) || T * top_k * inter * 2 >= ((int64_t)1 << 31))
    return fail(QINT4_ERR_SHAPE, "%s: T = %lld rows too many for this width (x or h over 2 GiB)",
                fn, (long long)T);
  if (!aligned(x, 16) || !aligned(out, 16) || (residual && !aligned(residual, 16)))
    return fail(QINT4_ERR_ALIGN, "%s: x/out/residual not 16-byte aligned", fn);
  if (!aligned(ids, 4) || !aligned(wts, 4)) return fail(QINT4_ERR_ALIGN, "%s: ids/wts misaligned", fn);
  if (!workspace || workspace_bytes < lay.total)
    return fail(QINT4_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn,
                workspace ? workspace_bytes : (size_t)0, lay.total);
  if (!aligned(workspace, 256)) return fail(QINT4_ERR_ALIGN, "%s: workspace not 256-byte aligned", fn);

  const size_t ob = elem_bytes(out_dtype);
  const int64_t P = T * top_k;
  Range ins[14], outs[2];
  int ni = 0;
  static const char *gn[3] = {"gate.codes", "gate.scales", "gate.biases"};
  static const char *un[3] = {"up.codes", "up.scales", "up.biases"};
  static const char *dn[3] = {"down.codes", "down.scales", "down.biases"};
  ni += add_matrix_ranges(gate, gn, ins + ni);
  ni += add_matrix_ranges(up, un, ins + ni);
  ni += add_matrix_ranges(down, dn, ins + ni);
  ins[ni++] = range(x, (size_t)((T - 1) * ldx + hidden) * 2, "x");
  ins[ni++] = range(ids, (size_t)P * 4, "ids");
  ins[ni++] = range(wts, (size_t)P * 4, "wts");
  if (residual) ins[ni++] = range(residual, (size_t)T * hidden * ob, "residual");
  outs[0] = range(out, (size_t)T * hidden * ob, "out");
  outs[1] = range(workspace, lay.total, "workspace");
  if ((st = check_no_overlap(outs, 2, ins, ni)) != QINT4_OK) return prefixed(st, fn);
  if ((st = check_device(nullptr)) != QINT4_OK) return prefixed(st, fn);

  unsigned char *ws = reinterpret_cast<unsigned char *>(workspace);
  uint32_t *perm = reinterpret_cast<uint32_t *>(ws + lay.perm);
  uint32_t *pos = reinterpret_cast<uint32_t *>(ws + lay.pos);
  uint32_t *tiles = reinterpret_cast<uint32_t *>(ws + lay.tiles);
  // row tile height from the mean rows per touched expert (uniform routing)
  const int64_t touched = std::min<int64_t>(gate->n_experts, P);
  const int64_t mean_rows = (P + touched - 1) / touched;
  const int bm = mean_rows <= 32 ? 32 : mean_rows <= 96 ? 64 : 128;
  const int64_t max_mtiles = (P + bm - 1) / bm + touched;
  if (max_mtiles * ((std::max(hidden, inter) + 31) / 32) >= INT32_MAX)
    return fail(QINT4_ERR_SHAPE, "%s: T * top_k too large for one launch at this width", fn);

  hipError_t e = launch_moe_sort(ids, P, gate->n_experts, bm, perm, pos, tiles, (int)lay.max_tiles,
                                 stream);
  MoeGemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.perm = perm;
  p.tiles = tiles;
  p.top_k = top_k;
  p.max_mtiles = (int32_t)max_mtiles;
  p.sb_bf16 = gate->sb_dtype == QINT4_BF16;
  p.log2_group = ilog2(gate->group_size);
  if (e == hipSuccess) {  // gate/up + SwiGLU -> h (hi, lo)
    p.codes0 = gate->codes; p.scales0 = gate->scales; p.biases0 = gate->biases;
    p.codes1 = up->codes;   p.scales1 = up->scales;   p.biases1 = up->biases;
    p.a0 = x;
    p.lda = ldx;
    p.y0 = ws + lay.h_hi;
    p.y1 = ws + lay.h_lo;
    p.n_out = (int32_t)inter;
    p.k_in = (int32_t)hidden;
    e = launch_moe_gemm(p, 0, bm, stream);
  }
  if (e == hipSuccess) {  // down -> d
    p.codes0 = down->codes; p.scales0 = down->scales; p.biases0 = down->biases;
    p.codes1 = nullptr;     p.scales1 = nullptr;      p.biases1 = nullptr;
    p.a0 = ws + lay.h_hi;
    p.a1 = ws + lay.h_lo;
    p.lda = inter;
    p.y0 = ws + lay.d;
    p.y1 = nullptr;
    p.n_out = (int32_t)hidden;
    p.k_in = (int32_t)inter;
    e = launch_moe_gemm(p, 1, bm, stream);
  }
  if (e == hipSuccess)
    e = launch_moe_combine(reinterpret_cast<const float *>(ws + lay.d), pos, wts, top_k, residual, out,
                           out_dtype == QINT4_BF16, T, (int)hidden, stream);
  if (e != hipSuccess) return fail(QINT4_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

qint4_status quantize_int4(const void *w, int32_t w_dtype, int64_t n_rows, int64_t k_in,
                           int32_t group_size, int32_t sb_dtype, uint32_t *codes, void *scales,
                           void *biases, void *stream) {
  const char *fn = "quantize_int4";
  if (!w || !codes || !scales || !biases)
    return fail(QINT4_ERR_NULL, "%s: w/codes/scales/biases is NULL", fn);
  if (!valid_dtype(w_dtype)) return fail(QINT4_ERR_DTYPE, "%s: w_dtype %d invalid", fn, w_dtype);
  if (!valid_dtype(sb_dtype)) return fail(QINT4_ERR_DTYPE, "%s: sb_dtype %d invalid", fn, sb_dtype);
  if (group_size != 32 && group_size != 64 && group_size != 128)
    return fail(QINT4_ERR_SHAPE, "%s: group_size %d not in {32, 64, 128}", fn, group_size);
  if (k_in < group_size || k_in > kMaxK || k_in % group_size != 0)
    return fail(QINT4_ERR_SHAPE, "%s: k_in %lld must be a multiple of group_size %d in [%d, 2^20]",
                fn, (long long)k_in, group_size, group_size);
  if (n_rows < 1 || n_rows > ((int64_t)1 << 34) / k_in)
    return fail(QINT4_ERR_SHAPE, "%s: n_rows %lld out of range", fn, (long long)n_rows);
  const size_t wb = elem_bytes(w_dtype), sbb = elem_bytes(sb_dtype);
  if (!aligned(w, 16) || !aligned(codes, 16))
    return fail(QINT4_ERR_ALIGN, "%s: w and codes must be 16-byte aligned", fn);
  if (!aligned(scales, sbb) || !aligned(biases, sbb))
    return fail(QINT4_ERR_ALIGN, "%s: scales/biases not aligned to %zu bytes", fn, sbb);
  const size_t n_groups = (size_t)n_rows * (size_t)(k_in / group_size);
  Range ins[1], outs[3];
  ins[0] = range(w, (size_t)n_rows * k_in * wb, "w");
  outs[0] = range(codes, (size_t)n_rows * k_in / 2, "codes");
  outs[1] = range(scales, n_groups * sbb, "scales");
  outs[2] = range(biases, n_groups * sbb, "biases");
  qint4_status st = check_no_overlap(outs, 3, ins, 1);
  if (st != QINT4_OK) return prefixed(st, fn);
  if ((st = check_device(nullptr)) != QINT4_OK) return prefixed(st, fn);
  // launches of whole rows spanning < 2 GiB of weights each
  const int64_t row_bytes = k_in * (int64_t)wb;
  const int64_t rows_per = std::max<int64_t>(1, (((int64_t)1 << 31) - 1) / row_bytes);
  const int64_t gpr = k_in / group_size;
  for (int64_t r0 = 0; r0 < n_rows; r0 += rows_per) {
    const int64_t nr = std::min(rows_per, n_rows - r0);
    hipError_t e = launch_quantize(
        reinterpret_cast<const unsigned char *>(w) + r0 * row_bytes, w_dtype == QINT4_BF16,
        nr * k_in / 8, group_size, sb_dtype == QINT4_BF16, codes + r0 * (k_in / 8),
        reinterpret_cast<unsigned char *>(scales) + r0 * gpr * (int64_t)sbb,
        reinterpret_cast<unsigned char *>(biases) + r0 * gpr * (int64_t)sbb,
        reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(QINT4_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
  }
  return ok();
}

// Shared by qgemm_int4_padT (no workspace) and qgemm_int4_padT_ws.
static qint4_status run_gemm(const char *fn, const qint4_matrix *w, const void *x, int64_t T,
                             int64_t ldx, void *y, int64_t ldy, int32_t y_dtype, void *ws,
                             size_t ws_bytes, void *stream) {
  qint4_status st;
  if ((st = check_matrix(w, "w", false)) != QINT4_OK) return st;
  if (!x || !y) return fail(QINT4_ERR_NULL, "%s: x or y is NULL", fn);
  if (!valid_dtype(y_dtype)) return fail(QINT4_ERR_DTYPE, "%s: y_dtype %d invalid", fn, y_dtype);
  if (w->n_out % 32 != 0)
    return fail(QINT4_ERR_SHAPE, "%s: n_out (%lld) must be a multiple of 32 (GEMM tile)", fn,
                (long long)w->n_out);
  if (T < 1 || T > ((int64_t)1 << 31)) return fail(QINT4_ERR_SHAPE, "%s: T = %lld invalid", fn, (long long)T);
  if (ldx < w->k_in || ldx % 8 != 0)
    return fail(QINT4_ERR_SHAPE, "%s: ldx %lld must be >= k_in %lld and a multiple of 8", fn,
                (long long)ldx, (long long)w->k_in);
  if (ldy < w->n_out) return fail(QINT4_ERR_SHAPE, "%s: ldy %lld < n_out %lld", fn, (long long)ldy, (long long)w->n_out);
  if (!aligned(x, 16)) return fail(QINT4_ERR_ALIGN, "%s: x not 16-byte aligned", fn);
  if (!aligned(y, elem_bytes(y_dtype))) return fail(QINT4_ERR_ALIGN, "%s: y misaligned", fn);
  if (w->n_out > INT32_MAX || w->k_in > INT32_MAX) return fail(QINT4_ERR_SHAPE, "%s: too large", fn);

  if (!ws) ws_bytes = 0;
  if (ws && !aligned(ws, 256)) return fail(QINT4_ERR_ALIGN, "%s: workspace not 256-byte aligned", fn);

  Range ins[4], outs[2];
  static const char *mn[3] = {"codes", "scales", "biases"};
  int ni = add_matrix_ranges(w, mn, ins);
  ins[ni++] = range(x, (size_t)((T - 1) * ldx + w->k_in) * 2, "x");
  int no = 0;
  outs[no++] = range(y, (size_t)((T - 1) * ldy + w->n_out) * elem_bytes(y_dtype), "y");
  if ((st = check_no_overlap(outs, no, ins, ni)) != QINT4_OK) return prefixed(st, fn);
  int n_cu = 256;
  if ((st = check_device(&n_cu)) != QINT4_OK) return prefixed(st, fn);

  // T <= 64: weights straight from HBM into MFMA registers, split over K when
  // the workspace allows (qgemm_stream.hip); longer T: LDS-tiled weights
  // (qgemm.hip), which amortise the dequantisation over more rows.  The
  // stream kernel addresses X through 32-bit byte offsets.
  const bool stream_path = T <= kStreamMaxT && (T - 1) * ldx + w->k_in < ((int64_t)1 << 30);
  // the tiled kernel addresses one tile's rows of X through 32-bit offsets
  if (!stream_path && (int64_t)kGemmTileRows * ldx * 2 >= ((int64_t)1 << 31))
    return fail(QINT4_ERR_SHAPE, "%s: ldx %lld too large for T > %d", fn, (long long)ldx, kStreamMaxT);
  StreamPlan plan{};
  size_t ws_used = 0;
  if (stream_path) {
    const bool sb16 = w->sb_dtype == QINT4_BF16;
    const bool sb_dwords = !sb16 || ((w->k_in / w->group_size) % 2 == 0 && aligned(w->scales, 4) &&
                                     aligned(w->biases, 4));
    plan = plan_gemm_stream(T, w->n_out, w->k_in, ilog2(w->group_size), sb16, sb_dwords, n_cu,
                            (int64_t)std::min<size_t>(ws_bytes, (size_t)INT64_MAX));
    ws_used = gemm_stream_ws_bytes(plan, T, w->n_out);
  }
  if (ws_used) {
    outs[no++] = range(ws, ws_used, "workspace");
    if ((st = check_no_overlap(outs, no, ins, ni)) != QINT4_OK) return prefixed(st, fn);
  }

  GemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.codes = w->codes;
  p.scales = w->scales;
  p.biases = w->biases;
  p.x = reinterpret_cast<const uint16_t *>(x);
  p.y = y;
  p.T = T;
  p.ldx = ldx;
  p.ldy = ldy;
  p.n_out = (int32_t)w->n_out;
  p.k_in = (int32_t)w->k_in;
  p.log2_group = ilog2(w->group_size);
  p.y_bf16 = y_dtype == QINT4_BF16;
  p.sb_bf16 = w->sb_dtype == QINT4_BF16;
  p.part = reinterpret_cast<float *>(ws);
  p.ksplit = 1;
  hipError_t e;
  if (stream_path) {
    e = launch_gemm_stream(p, plan, reinterpret_cast<hipStream_t>(stream));
  } else {
    GemmMultiParams mp;
    std::memset(&mp, 0, sizeof(mp));
    mp.m[0] = {w->codes, w->scales, w->biases, y, ldy, (int32_t)w->n_out, 0};
    mp.n_mats = 1;
    mp.x = reinterpret_cast<const uint16_t *>(x);
    mp.T = T;
    mp.ldx = ldx;
    mp.k_in = (int32_t)w->k_in;
    mp.log2_group = ilog2(w->group_size);
    mp.y_bf16 = y_dtype == QINT4_BF16;
    mp.sb_bf16 = w->sb_dtype == QINT4_BF16;
    e = launch_gemm(mp, reinterpret_cast<hipStream_t>(stream));
  }
  if (e != hipSuccess) return fail(QINT4_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

qint4_status qgemm_int4_padT(const qint4_matrix *w, const void *x, int64_t T, int64_t ldx, void *y,
                             int64_t ldy, int32_t y_dtype, void *stream) {
  return run_gemm("qgemm_int4_padT", w, x, T, ldx, y, ldy, y_dtype, nullptr, 0, stream);
}

size_t qgemm_int4_padT_workspace_bytes(int64_t T, int64_t n_out, int64_t k_in) {
  if (T < 1 || T > kStreamMaxT || n_out < 1 || n_out > INT32_MAX || k_in < 32 || k_in > kMaxK)
    return 0;
  int n_cu = 256;
  if (check_device(&n_cu) != QINT4_OK) return 0;
  // the split plan depends on the shape and the device only
  return gemm_stream_ws_bytes(plan_gemm_stream(T, n_out, k_in, 6, 1, true, n_cu, -1), T, n_out);
}

qint4_status qgemm_int4_padT_ws(const qint4_matrix *w, const void *x, int64_t T, int64_t ldx,
                                void *y, int64_t ldy, int32_t y_dtype, void *workspace,
                                size_t workspace_bytes, void *stream) {
  return run_gemm("qgemm_int4_padT_ws", w, x, T, ldx, y, ldy, y_dtype, workspace, workspace_bytes,
                  stream);
}


qint4_status qgemm_int4_padT_multi(int32_t n, const qint4_matrix *ws, const void *x, int64_t T,
                                   int64_t ldx, void *const *ys, const int64_t *ldys,
                                   int32_t y_dtype, void *stream) {
  const char *fn = "qgemm_int4_padT_multi";
  if (n < 1 || n > QINT4_MULTI_MAX)
    return fail(QINT4_ERR_SHAPE, "%s: n = %d not in [1, %d]", fn, n, QINT4_MULTI_MAX);
  if (!ws) return fail(QINT4_ERR_NULL, "%s: matrix array is NULL", fn);
  if (!ys) return fail(QINT4_ERR_NULL, "%s: output array is NULL", fn);
  if (!x) return fail(QINT4_ERR_NULL, "%s: x is NULL", fn);
  if (!valid_dtype(y_dtype)) return fail(QINT4_ERR_DTYPE, "%s: y_dtype %d invalid", fn, y_dtype);
  char name[32];
  qint4_status st;
  for (int i = 0; i < n; ++i) {
    snprintf(name, sizeof(name), "ws[%d]", i);
    if ((st = check_matrix(&ws[i], name, false)) != QINT4_OK) return st;
    if (!ys[i]) return fail(QINT4_ERR_NULL, "%s: ys[%d] is NULL", fn, i);
    if (ws[i].n_out % 32 != 0)
      return fail(QINT4_ERR_SHAPE, "%s: ws[%d].n_out (%lld) must be a multiple of 32 (GEMM tile)", fn,
                  i, (long long)ws[i].n_out);
    if (ws[i].n_out > INT32_MAX / 2) return fail(QINT4_ERR_SHAPE, "%s: ws[%d] too large", fn, i);
    const int64_t ldy = ldys ? ldys[i] : ws[i].n_out;
    if (ldy < ws[i].n_out)
      return fail(QINT4_ERR_SHAPE, "%s: ldys[%d] %lld < n_out %lld", fn, i, (long long)ldy,
                  (long long)ws[i].n_out);
    if (!aligned(ys[i], elem_bytes(y_dtype)))
      return fail(QINT4_ERR_ALIGN, "%s: ys[%d] misaligned", fn, i);
  }
  for (int i = 1; i < n; ++i) {
    if (ws[i].k_in != ws[0].k_in)
      return fail(QINT4_ERR_SHAPE,
                  "%s: packed width mismatch: ws[%d].k_in = %lld (%lld words) but ws[0].k_in = %lld "
                  "(%lld words)",
                  fn, i, (long long)ws[i].k_in, (long long)ws[i].k_in / 8, (long long)ws[0].k_in,
                  (long long)ws[0].k_in / 8);
    if (ws[i].group_size != ws[0].group_size)
      return fail(QINT4_ERR_SHAPE, "%s: ws[%d].group_size %d != ws[0].group_size %d", fn, i,
                  ws[i].group_size, ws[0].group_size);
    if (ws[i].sb_dtype != ws[0].sb_dtype)
      return fail(QINT4_ERR_DTYPE, "%s: ws[%d].sb_dtype differs from ws[0]", fn, i);
  }
  const int64_t k_in = ws[0].k_in;
  if (T < 1 || T > ((int64_t)1 << 31)) return fail(QINT4_ERR_SHAPE, "%s: T = %lld invalid", fn, (long long)T);
  if (ldx < k_in || ldx % 8 != 0)
    return fail(QINT4_ERR_SHAPE, "%s: ldx %lld must be >= k_in %lld and a multiple of 8", fn,
                (long long)ldx, (long long)k_in);
  if (!aligned(x, 16)) return fail(QINT4_ERR_ALIGN, "%s: x not 16-byte aligned", fn);
  if ((int64_t)kGemmTileRows * ldx * 2 >= ((int64_t)1 << 31))
    return fail(QINT4_ERR_SHAPE, "%s: ldx %lld too large", fn, (long long)ldx);

  Range ins[3 * QINT4_MULTI_MAX + 1], outs[QINT4_MULTI_MAX];
  int ni = 0;
  static const char *mnames[3] = {"codes", "scales", "biases"};
  for (int i = 0; i < n; ++i) ni += add_matrix_ranges(&ws[i], mnames, ins + ni);
  ins[ni++] = range(x, (size_t)((T - 1) * ldx + k_in) * 2, "x");
  static const char *ynames[QINT4_MULTI_MAX] = {"ys[0]", "ys[1]", "ys[2]", "ys[3]",
                                                  "ys[4]", "ys[5]", "ys[6]", "ys[7]"};
  for (int i = 0; i < n; ++i) {
    const int64_t ldy = ldys ? ldys[i] : ws[i].n_out;
    outs[i] = range(ys[i], (size_t)((T - 1) * ldy + ws[i].n_out) * elem_bytes(y_dtype), ynames[i]);
  }
  if ((st = check_no_overlap(outs, n, ins, ni)) != QINT4_OK) return prefixed(st, fn);
  if ((st = check_device(nullptr)) != QINT4_OK) return prefixed(st, fn);

  GemmMultiParams mp;
  std::memset(&mp, 0, sizeof(mp));
  for (int i = 0; i < n; ++i)
    mp.m[i] = {ws[i].codes, ws[i].scales, ws[i].biases, ys[i], ldys ? ldys[i] : ws[i].n_out,
               (int32_t)ws[i].n_out, 0};
  mp.n_mats = n;
  mp.x = reinterpret_cast<const uint16_t *>(x);
  mp.T = T;
  mp.ldx = ldx;
  mp.k_in = (int32_t)k_in;
  mp.log2_group = ilog2(ws[0].group_size);
  mp.y_bf16 = y_dtype == QINT4_BF16;
  mp.sb_bf16 = ws[0].sb_dtype == QINT4_BF16;
  hipError_t e = launch_gemm(mp, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(QINT4_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Launch plans (host only)
// ---------------------------------------------------------------------------

namespace {

qint4_status check_plan_shape(int64_t n_out, int64_t k_in, int32_t group_size, const char *name) {
  if (group_size != 32 && group_size != 64 && group_size != 128)
    return fail(QINT4_ERR_SHAPE, "%s: group_size %d not in {32, 64, 128}", name, group_size);
  if (n_out < 1 || n_out > kMaxRows)
    return fail(QINT4_ERR_SHAPE, "%s: n_out %lld out of range [1, 2^30]", name, (long long)n_out);
  if (k_in < group_size || k_in > kMaxK || k_in % group_size != 0)
    return fail(QINT4_ERR_SHAPE, "%s: k_in %lld must be a multiple of group_size %d in [%d, 2^20]",
                name, (long long)k_in, group_size, group_size);
  if ((size_t)n_out * (size_t)(k_in / 2) >= kMaxMatrixBytes)
    return fail(QINT4_ERR_SHAPE, "%s: code bytes exceed the 2 GiB limit", name);
  return QINT4_OK;
}

// CU count to plan for: n_cu itself, or (0) the current device's.
qint4_status plan_cus(int32_t n_cu, int *out) {
  if (n_cu < 0) return fail(QINT4_ERR_VALUE, "n_cu %d < 0", n_cu);
  if (n_cu > 0) {
    *out = n_cu;
    return QINT4_OK;
  }
  return check_device(out);
}

}  // namespace

extern "C" {

qint4_status qint4_plan_qgemv(int32_t call, int32_t n, const int64_t *n_outs, int64_t k_in,
                              int32_t group_size, int32_t x_dtype, int64_t T, int32_t epilogue,
                              int32_t n_cu, qint4_gemv_form *form) {
  const char *fn = "qint4_plan_qgemv";
  if (!form || !n_outs) return fail(QINT4_ERR_NULL, "%s: form or n_outs is NULL", fn);
  if (call != QINT4_CALL_QGEMV && call != QINT4_CALL_RMS_NORM && call != QINT4_CALL_SMALLM)
    return fail(QINT4_ERR_VALUE, "%s: call %d invalid", fn, call);
  if (n < 1 || n > QINT4_MULTI_MAX)
    return fail(QINT4_ERR_SHAPE, "%s: n = %d not in [1, %d]", fn, n, QINT4_MULTI_MAX);
  if (!valid_dtype(x_dtype)) return fail(QINT4_ERR_DTYPE, "%s: x_dtype %d invalid", fn, x_dtype);
  if (epilogue != QINT4_EPI_NONE && epilogue != QINT4_EPI_SWIGLU_PAIR)
    return fail(QINT4_ERR_SHAPE, "%s: epilogue %d invalid", fn, epilogue);
  const bool swiglu = epilogue == QINT4_EPI_SWIGLU_PAIR;
  if (swiglu && (n != 2 || n_outs[0] != n_outs[1]))
    return fail(QINT4_ERR_SHAPE, "%s: SWIGLU_PAIR needs two matrices of equal n_out", fn);
  qint4_status st;
  for (int i = 0; i < n; ++i)
    if ((st = check_plan_shape(n_outs[i], k_in, group_size, fn)) != QINT4_OK) return st;
  const int64_t t_max = call == QINT4_CALL_SMALLM ? QINT4_SMALLM_MAX : 1;
  if (T < 1 || T > t_max)
    return fail(QINT4_ERR_SHAPE, "%s: T = %lld not in [1, %lld]", fn, (long long)T, (long long)t_max);
  if (T > 1 && x_dtype != QINT4_BF16)
    return fail(QINT4_ERR_DTYPE, "%s: T > 1 needs bfloat16 activations", fn);
  int cus = 0;
  if ((st = plan_cus(n_cu, &cus)) != QINT4_OK) return prefixed(st, fn);
  const bool rms = call == QINT4_CALL_RMS_NORM;
  MultiPlan mp;
  st = plan_multi(swiglu ? 1 : n, n_outs, k_in, group_size, x_dtype, T, swiglu, rms,
                  call == QINT4_CALL_SMALLM, cus, &mp);
  if (st != QINT4_OK) return prefixed(st, fn);
  const int64_t launches = (T + mp.blk - 1) / mp.blk;
  if (mp.mfma) {
    std::memset(form, 0, sizeof(*form));
    form->kernel = QINT4_FORM_MFMA;
    form->tokens = tt_for(std::min<int64_t>(T, mp.blk));
    form->launches = launches;
    form->grid = form->tokens <= 4 ? mp.tiles : mp.grid;  // the first launch
    form->tasks = mp.tiles;
    form->waves = gemv_mfma_waves(k_in);
  } else if (mp.xs) {
    std::memset(form, 0, sizeof(*form));
    form->kernel = QINT4_FORM_XS;
    form->tokens = 1;
    form->launches = 1;
    form->grid = mp.grid;
    form->waves = gemv_xs_waves(k_in);
    form->lanes = 1 << gemv_xs_log2_lanes(k_in);
    form->rows_per_task = 64 / form->lanes;
    form->steps_per_task = 1;
    const int nm = swiglu ? 1 : n;
    for (int i = 0; i < nm; ++i) {
      const int64_t gi = mp.wg0[i + 1] - mp.wg0[i];
      form->tasks += n_outs[i];
      form->busiest_wave_steps = std::max<int64_t>(form->busiest_wave_steps, (n_outs[i] + gi - 1) / gi);
    }
    form->ring_depth = gemv_xs_depth();
  } else {
    ring_form(mp.plan, multi_xmode(x_dtype, rms), swiglu ? EPI_SWIGLU : EPI_STORE, launches, form);
  }
  return ok();
}

qint4_status qint4_plan_moe_gather(int64_t hidden, int64_t inter, int32_t top_k,
                                   int32_t group_size, int32_t act_dtype, int32_t routed,
                                   int32_t residual, int32_t n_cu, qint4_gemv_form *forms) {
  const char *fn = "qint4_plan_moe_gather";
  if (!forms) return fail(QINT4_ERR_NULL, "%s: forms is NULL", fn);
  if (!valid_dtype(act_dtype)) return fail(QINT4_ERR_DTYPE, "%s: act_dtype %d invalid", fn, act_dtype);
  if (top_k < 1 || top_k > QINT4_TOPK_MAX)
    return fail(QINT4_ERR_SHAPE, "%s: top_k %d not in [1, %d]", fn, top_k, QINT4_TOPK_MAX);
  qint4_status st;
  if ((st = check_plan_shape(inter, hidden, group_size, fn)) != QINT4_OK) return st;
  if ((st = check_plan_shape(hidden, inter, group_size, fn)) != QINT4_OK) return st;
  int cus = 0;
  if ((st = plan_cus(n_cu, &cus)) != QINT4_OK) return prefixed(st, fn);
  GemvPlan a, b;
  st = plan_moe(hidden, inter, top_k, act_dtype, routed != 0, residual != 0, cus, &a, &b);
  if (st != QINT4_OK) return prefixed(st, fn);
  ring_form(a, act_dtype == QINT4_BF16 ? XM_BF16 : XM_F32, EPI_SWIGLU, 1, &forms[0]);
  ring_form(b, XM_F32, EPI_MOE_DOWN, 1, &forms[1]);
  return ok();
}

}  // extern "C"
