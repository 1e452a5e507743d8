// kernels.h -- internal interface between the C-ABI layer (api.cpp) and the
// gfx950 kernels (qgemv.hip, qgemm.hip).  Not installed; callers use qint4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <unordered_map>

namespace qint4 {

constexpr int kMaxMats = 8;    // projections per multi call
constexpr int kMaxTopK = 8;    // experts combined per MoE call
constexpr int kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

// Lets kernel `kern` use up to `bytes` of dynamic LDS (more than the default
// 64 KB) on the current device.  The attribute is set once per (kernel,
// device) pair: a registry keyed by the kernel's address records the devices
// done (bit d = device d; devices past 63 set the attribute on every call).
// Concurrent first calls both set the same value.
inline hipError_t lds_opt_in(const void *kern, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  static std::mutex mu;
  static std::unordered_map<const void *, uint64_t> done;
  if (bit) {
    std::lock_guard<std::mutex> g(mu);
    auto it = done.find(kern);
    if (it != done.end() && (it->second & bit)) return hipSuccess;
  }
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) {
    std::lock_guard<std::mutex> g(mu);
    done[kern] |= bit;
  }
  return e;
}

// Activation staging / compute modes of the GEMV family.  XM_RMS_*: the
// activation is RMS-normalised on the way in -- x and gamma (both bf16, or
// both float32) are staged as the float32 products x * gamma, the sum of x^2
// is reduced over the workgroup, and results are scaled by
// 1 / sqrt(sum(x^2) / k_in + eps) before the epilogue.
enum XMode { XM_BF16 = 0, XM_F32 = 1, XM_RMS_BF16 = 2, XM_RMS_F32 = 3 };
constexpr bool xm_rms(int xm) { return xm == XM_RMS_BF16 || xm == XM_RMS_F32; }
// Octets (8 activation elements) one thread stages per round.
constexpr int xm_octets(int xm) { return xm == XM_BF16 ? 2 : xm == XM_F32 ? 5 : xm == XM_RMS_BF16 ? 4 : 3; }
enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_MOE_DOWN = 2 };

// One matrix (or expert stack) as the GEMV kernels see it.
struct GemvMat {
  const uint32_t *codes;     // expert 0, row 0
  const void *scales;
  const void *biases;
  void *y;                   // output base (EPI_SWIGLU: [slots][n_out])
  int64_t n_out;
};

// Loads in flight per lane (128-bit code loads) in a GEMV wave's register ring.
constexpr int kSlots = 8;

// Kernel arguments of the GEMV family.  A "task" is rpt rows, all of whose
// chunks (32 codes = 16 bytes) one wave processes; L lanes cover one row, so a
// step (one 16-byte load per lane) covers L chunks of 64 / L rows.  Tasks are
// dealt round-robin: wave w takes tasks w, w + n_waves, ...
struct GemvParams {
  GemvMat m[kMaxMats];
  int32_t task0[kMaxMats];   // first task of each matrix (EPI_STORE), INT32_MAX past n_mats
  int32_t n_mats;
  int32_t log2_lpr;          // L = 1 << log2_lpr lanes per row
  int32_t log2_group;
  int32_t spt;               // steps per task (the last may be partial)
  int32_t rpt;               // rows per task
  int32_t last_lanes;        // lanes of a row holding a chunk in the last step
  int32_t ncx;               // staged activation chunks
  int32_t ncx_pad;           // spt * L: staged chunks including zero padding
  int32_t kwb;               // code bytes of one stored row
  int32_t sbrow;             // scale (= bias) bytes of one stored row
  int32_t n_tasks;
  int32_t tasks_q;           // n_tasks = tasks_q * n_waves + tasks_r
  int32_t tasks_r;
  int32_t n_waves;           // waves of the grid
  int32_t waves_per_wg;
  int32_t y_bf16;
  // MoE
  int32_t top_k;
  int32_t n_experts;
  int32_t tasks_per_slot;    // EPI_SWIGLU: tasks of one expert slot
  int32_t n_tok;             // activation rows (tokens) of a small-M call, 1..TT
  int32_t cpr_e;             // EPI_MOE_DOWN: chunks of one expert row
  float inv_cpr_e;
  uint32_t ecode_bytes;      // code bytes between experts
  uint32_t esb_bytes;        // scale bytes between experts
  uint32_t code_bytes;       // EPI_MOE_DOWN: code bytes of the whole stack (< 2^31)
  uint32_t sb_bytes;         // EPI_MOE_DOWN: scale bytes of the whole stack
  int32_t ldx;               // elements between consecutive activation rows
  float eps;                 // XM_RMS_*: RMSNorm epsilon
  const void *x;             // activation (bf16 bits or float32), 16-byte aligned
  uint32_t *ids;             // device [top_k] or nullptr: read, or (route != 0) written by
                             // the first wave of the grid
  float *wts;                // device [top_k]: read (EPI_MOE_DOWN), or written when routing
  const void *aux;           // EPI_MOE_DOWN: residual [n_out] or nullptr; XM_RMS_*: RMSNorm
                             // weight [k_in] (the activation's dtype); routing: logits [n_experts]
  int32_t route;             // EPI_SWIGLU: 0 = ids given; 1 / 2 = every wave ranks the float32 /
                             // bf16 logits itself (n_experts <= kRouteMaxExperts)
  int32_t stage_last;        // first octet of the activation's last staging round (set by
                             // launch_gemv)
};

// Experts one wave ranks in registers when the gate/up launch routes its token.
constexpr int kRouteMaxExperts = 256;

struct GemvPlan {
  int tt;           // tokens per launch template: 1, 2, 4 or 8
  int waves;        // waves per workgroup
  int rt;           // row groups per task: 1 or 2
  int log2_lpr;
  int spt;
  int64_t n_tasks;
  int64_t grid;     // workgroups (persistent)
  size_t lds_bytes;
};

static_assert(sizeof(GemvParams) <= 512, "GEMV kernel arguments exceed 8 cache lines");

// Launches with one-pass kernels (a ring of depth 1, 2 or 4 filled once, for
// launches where no wave has more steps than that): the stored-output GEMVs
// of up to 4 tokens, the one-token gate/up pair without the RMSNorm prologue
// and the MoE down projection.  Every other launch streams its ring.
constexpr bool gemv_has_one_pass(int epi, int tt, int xmode) {
  return (epi == EPI_STORE && tt <= 4) || (tt == 1 && epi == EPI_SWIGLU && !xm_rms(xmode)) ||
         epi == EPI_MOE_DOWN;
}

// Steps of the busiest wave of a planned launch (tasks are dealt round-robin).
inline int64_t gemv_busiest_steps(const GemvPlan &plan) {
  const int64_t nw = plan.grid * plan.waves;
  return nw > 0 ? (plan.n_tasks + nw - 1) / nw * plan.spt : 0;
}

// Ring depth a planned launch runs with: 1, 2 or 4 (one pass) or 0 (the
// streaming ring).  A one-pass ring holds depth * rt * streams loads per lane,
// within kSlots.
inline int gemv_ring_depth(const GemvPlan &plan, int xmode, int epi) {
  if (!gemv_has_one_pass(epi, plan.tt, xmode)) return 0;
  const int loads = plan.rt * (epi == EPI_SWIGLU ? 2 : 1);
  const int64_t s = gemv_busiest_steps(plan);
  if (s == 1) return 1;
  if (s == 2 && 2 * loads <= kSlots) return 2;
  if (s >= 3 && s <= 4 && 4 * loads <= kSlots) return 4;
  return 0;
}

// Launch one GEMV-family kernel.  `xmode`: an XMode;
// `sb_bf16`: scales/biases element type; `epi`: Epi.
hipError_t launch_gemv(const GemvParams &p, const GemvPlan &plan, int xmode, int sb_bf16,
                       int epi, hipStream_t stream);

// Small-M GEMVs with bf16 activations on MFMA (qgemv_mfma.hip): n_tasks tiles
// of 16 rows (stored outputs: task0[i] = first tile of matrix i; swiglu: the
// gate/up pair m[0], m[1] with h in m[0].y), gemv_mfma_waves(k_in) K slices per
// tile, n_tok rows of x with stride ldx, ncx = k_in / 32.  streams: 1 (stored
// outputs) or 2 (gate/up pair).  `grid` workgroups (1..n_tasks) take tiles
// i, i + grid, ...  Supported shapes take this path for every token count.
bool gemv_mfma_supported(int64_t k_in, int group_size, int streams);
int gemv_mfma_waves(int64_t k_in);  // K slices (waves) per tile
size_t gemv_mfma_lds_bytes(int tt, int group_size, int64_t k_in, int streams);
hipError_t launch_gemv_mfma(const GemvParams &p, int tt, int group_size, int sb_bf16, int swiglu,
                            int64_t grid, hipStream_t stream);

// Activation-stationary T=1 GEMVs (qgemv_xs.hip): up to kXsMaxMats matrices
// sharing x with stored outputs, or the gate/up pair with the SwiGLU
// epilogue.  Lane j of a row group of wave w holds chunk L w + j of x in
// registers (L = 1 << log2_lpr lanes per row, gemv_xs_waves(k_in) waves per
// workgroup cover k_in).  Matrix m owns workgroups wg0[m] .. wg0[m+1]-1, and
// its workgroup b of G = wg0[m+1] - wg0[m] takes rows b, b + G, ... (the
// pair: the block of ceil(n_out / G) rows from b * that)
constexpr int kXsMaxWaves = 16;    // k_in up to 32768
constexpr int kXsMaxRows = 256;    // rows per workgroup
constexpr int kXsMaxMats = 8;      // matrices of one call
struct GemvXsParams {
  // stored outputs: matrix m in codes/scales/biases[m], its outputs in y[m];
  // the pair: gate in [0], up in [1], h in y[0] (n_mats = 1)
  const uint32_t *codes[kXsMaxMats];
  const void *scales[kXsMaxMats];
  const void *biases[kXsMaxMats];
  void *y[kXsMaxMats];
  int32_t n_out[kXsMaxMats];
  int32_t wg0[kXsMaxMats + 1];
  int32_t n_mats;
  const void *x;       // float32 or bf16 bits
  const void *gamma;   // RMSNorm weight (x's dtype), or NULL: no RMSNorm prologue
  float eps;           // RMSNorm epsilon
  int32_t ncx;         // k_in / 32
  int32_t kwb;         // code bytes of one row
  int32_t sbrow;       // scale (= bias) bytes of one row
  int32_t log2_group;
  int32_t log2_lpr;    // gemv_xs_log2_lanes(k_in)
  int32_t waves;       // gemv_xs_waves(k_in)
  int32_t y_bf16;
};
int gemv_xs_log2_lanes(int64_t k_in);
int gemv_xs_waves(int64_t k_in);
// Splits the rows of n_mats matrices (the pair: n_mats = 1, streams = 2) over
// workgroups (wg0[0..n_mats]); returns false where the form does not apply.
bool gemv_xs_plan(int n_mats, const int64_t *n_out, int64_t k_in, int streams, int n_cu, int32_t *wg0);
int gemv_xs_depth();  // rows in flight per wave
hipError_t launch_gemv_xs(const GemvXsParams &p, int sb_bf16, int x_bf16, int streams, hipStream_t stream);
// (p.gamma != NULL: x * gamma is the activation and the row sums are scaled by
// 1 / sqrt(sum(x^2) / k_in + eps), as in the streaming GEMV's RMSNorm form)

// LDS bytes a GEMV launch needs: per token, the staged activation (padded to
// ncx_pad chunks) and its chunk sums; then (MoE down) the float32 residual row
// or (XM_RMS_*) one float per wave.
size_t gemv_lds_bytes(int xmode, int ncx_pad, int64_t residual_rows, int tt = 1);

// Largest token count of one small-M GEMV launch.
constexpr int kMaxTokens = 8;

// Waves per workgroup a GEMV kernel supports: 12, or 8 for the 8-token
// kernels, whose accumulators and decoded weights need up to 256 VGPRs a lane.
constexpr int gemv_max_waves(int tt) { return tt >= 8 ? 8 : 12; }

struct GemmParams {
  const uint32_t *codes;
  const void *scales;
  const void *biases;
  const uint16_t *x;         // bf16 [T][ldx]
  void *y;                   // [T][ldy]
  int64_t T;
  int64_t ldx;
  int64_t ldy;
  int32_t n_out;
  int32_t k_in;
  int32_t log2_group;
  int32_t y_bf16;
  int32_t sb_bf16;
  int32_t m_tiles;
  int32_t n_tiles;
  // split-K (stream kernel): ksplit workgroups share a row block and a token
  // block, each summing split_steps 128-k steps into part[slice][T][n_out]
  // (float32); a reduce kernel adds the slices into y.  ksplit == 1 writes y.
  float *part;
  int32_t ksplit;
  int32_t split_steps;
  int32_t sb_tab_dw;         // dwords of one wave's scale (or bias) table in LDS, 0: none
  int32_t pad_;
};

// LDS-tiled prefill GEMM (qgemm.hip) over the matrix table of GemmMultiParams.
struct GemmMultiParams;
hipError_t launch_gemm(const GemmMultiParams &p, hipStream_t stream);

// Prefill GEMM over the output tiles of up to kMaxMats matrices that share X
// (k_in, group size and scale dtype); n_out % 32 == 0 each.  tile0 / m_tiles /
// n_tiles / tiles / per_xcd are filled in by the launcher.
struct GemmMat {
  const uint32_t *codes;
  const void *scales;
  const void *biases;
  void *y;                   // [T][ldy]
  int64_t ldy;
  int32_t n_out;
  int32_t tile0;             // first weight tile of this matrix
};
struct GemmMultiParams {
  GemmMat m[kMaxMats];
  const uint16_t *x;         // bf16 [T][ldx]
  int64_t T;
  int64_t ldx;
  int32_t k_in;
  int32_t log2_group;
  int32_t y_bf16;
  int32_t sb_bf16;
  int32_t n_mats;
  int32_t m_tiles;
  int32_t n_tiles;           // weight tiles of all matrices
  int32_t tiles;
  int32_t per_xcd;           // tiles each of the eight XCDs takes
  int32_t pad_;
};
static_assert(sizeof(GemmMultiParams) <= 512, "GEMM kernel arguments exceed 8 cache lines");
// Token rows of one tile of the LDS-tiled GEMM (at most); the host keeps that
// many rows of X addressable through 32-bit offsets.
constexpr int kGemmTileRows = 128;

// Register-resident-weight GEMM for T <= 64 (qgemm_stream.hip).
struct StreamPlan {
  int mt;           // 16-token blocks per workgroup (1, 2 or 4)
  int depth;        // weight steps in flight per wave
  int ksplit;       // K slices (1: no workspace needed)
  int split_steps;  // 128-k steps per slice
  int sb_lds;       // scales / biases staged in LDS once per wave
};
constexpr int kStreamMaxT = 64;
// Plan for a T x n_out x k_in product on a device with n_cu compute units;
// ksplit is limited to what ws_bytes holds (ws_bytes < 0: no limit).
// sb_dwords: every row of the scale and bias arrays starts dword-aligned
// (required for the LDS scale tables).
StreamPlan plan_gemm_stream(int64_t T, int64_t n_out, int64_t k_in, int log2_group, int sb_bf16,
                            bool sb_dwords, int n_cu, int64_t ws_bytes);
size_t gemm_stream_ws_bytes(const StreamPlan &plan, int64_t T, int64_t n_out);
hipError_t launch_gemm_stream(const GemmParams &p, const StreamPlan &plan, hipStream_t stream);

// Top-k expert routing of n_rows rows of router logits (float32 or bf16):
// ids/wts are [n_rows][top_k].
constexpr int kRouterMaxExperts = 4096;

// MoE prefill (expert-sorted gather GEMMs).
constexpr int kMaxExpertsPrefill = 4096;

struct MoeGemmParams {
  const uint32_t *codes0, *codes1;  // gate and up stacks, or the down stack (codes0)
  const void *scales0, *scales1;
  const void *biases0, *biases1;
  const void *a0, *a1;    // gate/up: x bf16 [T][lda]; down: h hi / lo planes, bf16 [P][lda]
  void *y0, *y1;          // gate/up: h hi / lo planes, bf16 [P][n_out]; down: d, float32 [P][n_out]
  const uint32_t *perm;   // sorted slot -> pair index t * top_k + k
  const uint32_t *tiles;  // [0] = row tiles, then (expert, first slot, rows) per tile
  int64_t lda;
  int32_t n_out, k_in, log2_group, sb_bf16, top_k, max_mtiles;
  int32_t sb_lds;         // 1: each workgroup stages its rows' scales / biases in LDS once
  int32_t pad_;
};

hipError_t launch_moe_sort(const uint32_t *ids, int64_t n_pairs, int n_experts, int bm, uint32_t *perm,
                           uint32_t *pos, uint32_t *tiles, int max_tiles, hipStream_t stream);
// down = 0: gate/up + SwiGLU; down = 1: down projection.  bm: 32, 64 or 128.
hipError_t launch_moe_gemm(const MoeGemmParams &p, int down, int bm, hipStream_t stream);
hipError_t launch_moe_combine(const float *d, const uint32_t *pos, const float *wts, int top_k,
                              const void *residual, void *out, int out_bf16, int64_t T, int hidden,
                              hipStream_t stream);

// Quantise n_words * 8 row-major weights (bf16 or float32; n_words * 8 * the
// weight size < 2 GiB) into codes / scales / biases with group_size in
// {32, 64, 128}; group g covers words g * group_size / 8 ...
hipError_t launch_quantize(const void *w, int w_bf16, int64_t n_words, int group_size, int sb_bf16,
                           uint32_t *codes, void *scales, void *biases, hipStream_t stream);
hipError_t launch_router(const void *logits, int bf16, int64_t n_rows, int n_experts, int top_k,
                         uint32_t *ids, float *wts, hipStream_t stream);

}  // namespace qint4
