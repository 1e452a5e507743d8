// kernels.h -- internal interface between the C-ABI layer (api.cpp) and the
// gfx950 kernels (qgemv.hip, qgemm.hip).  Not installed; callers use qint4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qint4 {

constexpr int kMaxMats = 8;    // projections per multi call
constexpr int kMaxTopK = 8;    // experts combined per MoE call
constexpr int kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

enum XMode { XM_BF16 = 0, XM_F32 = 1 };
enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_MOE_DOWN = 2 };

// One matrix (or expert stack) as the GEMV kernels see it.
struct GemvMat {
  const uint32_t *codes;     // expert 0, row 0
  const void *scales;
  const void *biases;
  void *y;                   // output base (EPI_STORE: [n_out]; EPI_SWIGLU: [slots][n_out])
  int64_t n_out;
};

// A "task" is one group of rows (rows_per_task = RT * 64 / lanes_per_row)
// processed by one wave; a "step" is one 32-code chunk of each of those rows.
struct GemvParams {
  GemvMat m[kMaxMats];
  int32_t task0[kMaxMats];   // first task of each matrix (EPI_STORE); static offsets,
                             // so the kernel loads them once
  int32_t n_mats;
  int32_t log2_lpr;          // lanes cooperating on one row (row segment)
  int32_t log2_group;        // log2(group_size)
  int32_t chunks_per_row;    // k_in / 32 of one stored row
  int32_t steps_per_task;    // chunk steps per task (virtual row chunks / lanes per row)
  int32_t n_chunks_x;        // chunks of the staged activation
  int32_t y_bf16;            // output element type
  int32_t tasks_per_slot;    // EPI_SWIGLU: tasks per (expert slot)
  int32_t n_tasks;           // total tasks (< 2^31)
  int32_t pad1_;
  const void *x;             // activation (bf16 bits or float32)
  // MoE
  const uint32_t *ids;       // device [top_k] or nullptr
  const float *wts;          // device [top_k] (EPI_MOE_DOWN)
  const void *residual;      // device [n_out] or nullptr (EPI_MOE_DOWN)
  int32_t top_k;
  int32_t n_experts;
  float inv_chunks_per_row;  // 1.0f / chunks_per_row (EPI_MOE_DOWN slot lookup)
  int32_t pad_;
  int64_t expert_code_stride;  // u32 words between experts
  int64_t expert_sb_stride;    // elements between experts in scales/biases
  int64_t code_bytes;          // bytes of codes of one stored matrix / stack (< 2^31)
  int64_t sb_bytes;            // bytes of scales (= biases) of one matrix / stack
};

struct GemvPlan {
  int waves;        // waves per workgroup (1..8)
  int rt;           // rows per lane per task: 1 or 2
  int log2_lpr;
  int64_t n_tasks;
  int64_t grid;     // workgroups (persistent)
  size_t lds_bytes;
};

// Launch one GEMV-family kernel.  `xmode`: XM_BF16 or XM_F32 staging;
// `sb_bf16`: scales/biases element type; `epi`: Epi.
hipError_t launch_gemv(const GemvParams &p, const GemvPlan &plan, int xmode, int sb_bf16,
                       int epi, hipStream_t stream);

// LDS bytes a GEMV launch needs: the staged activation, its chunk sums and
// (MoE down) the float32 residual row.
size_t gemv_lds_bytes(int xmode, int n_chunks_x, int64_t residual_rows);

// Resident workgroups per CU of the kernel a plan selects (0 if unknown).
int gemv_blocks_per_cu(const GemvPlan &plan, int xmode, int sb_bf16, int epi);

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
};

hipError_t launch_gemm(const GemmParams &p, hipStream_t stream);

}  // namespace qint4
