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
  int64_t block0;            // first row block of this matrix (EPI_STORE)
};

struct GemvParams {
  GemvMat m[kMaxMats];
  int32_t n_mats;
  int32_t log2_lpr;          // lanes cooperating on one row inside a wave
  int32_t log2_group;        // log2(group_size)
  int32_t chunks_per_row;    // k_in / 32 of the matrices' rows
  int32_t chunks_per_wave;   // chunk range owned by one wave (multiple of lanes per row)
  int32_t n_chunks_x;        // chunks of the staged activation (k_in/32, or top_k*inter/32)
  int32_t y_bf16;            // output element type
  int32_t blocks_per_slot;   // EPI_SWIGLU: row blocks per (slot, pair)
  int64_t n_blocks;          // total row blocks
  const void *x;             // activation (bf16 bits or float32)
  // MoE
  const uint32_t *ids;       // device [top_k] or nullptr
  const float *wts;          // device [top_k] (EPI_MOE_DOWN)
  const void *residual;      // device [n_out] or nullptr (EPI_MOE_DOWN)
  int32_t top_k;
  int32_t n_experts;
  int64_t expert_code_stride;  // u32 words between experts
  int64_t expert_sb_stride;    // elements between experts in scales/biases
};

struct GemvPlan {
  int waves;        // 1, 2, 4 or 8
  int rt;           // rows per lane: 1, 2 or 4
  int log2_lpr;
  int chunks_per_wave;
  int64_t n_blocks;
  size_t lds_bytes;
};

// Launch one GEMV-family kernel.  `xmode`: XM_BF16 or XM_F32 staging;
// `sb_bf16`: scales/biases element type; `epi`: Epi.
hipError_t launch_gemv(const GemvParams &p, const GemvPlan &plan, int xmode, int sb_bf16,
                       int epi, hipStream_t stream);

// LDS bytes a GEMV launch needs.
size_t gemv_lds_bytes(int xmode, int n_chunks_x, int waves, int rt, int log2_lpr, int epi);

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
