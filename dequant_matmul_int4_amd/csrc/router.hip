// router.hip -- top-K expert routing on the GPU for gfx950.
//
// Source: thewafflehaus/FFAI pull 14, "feat(everything-bagel): clean
// migration of PR #9 + #10 onto updated dev", commit adding the GPU MoE
// router wrappers: one row of router logits [n_experts] becomes [k] u32
// expert indices plus [k] weights, a T-batched form runs one row per program
// in one dispatch, and the index buffer feeds the expert-indexed GEMV with no
// host readback.  Selection order: thewafflehaus/FFAI pull 9, "Everything
// Bagel", top-K partial-sort commit: (value desc, index asc).
//
// Per row: p = softmax(logits); keep the top_k largest p, ties to the smaller
// expert index; weight_k = p_k / sum of the kept p, which equals a softmax over
// the kept logits (the full normaliser cancels), computed here as
// exp(l_k - l_max) / sum_j exp(l_j - l_max) in float32.  Because exp is
// increasing, ranking the logits ranks the probabilities; NaN logits rank
// below every number.
//
// One wave per row: the row's logits sit in registers (a fixed number per
// lane), then top_k rounds each take the best not-yet-chosen (value, index)
// pair of every lane and reduce it across the wave with DPP and lane swaps.

#include "kernels.h"
#include "topk_wave.h"

namespace qint4 {
namespace {

constexpr int kRowsPerBlock = 4;  // waves (rows) per workgroup

// NPL logits per lane in registers (lane l holds experts l, l + 64, ...).
template <int NPL>
__global__ void __launch_bounds__(64 * kRowsPerBlock)
    router_topk_kernel(const void *logits, int bf16, int64_t n_rows, int n_experts,
                       int top_k, uint32_t *__restrict__ ids, float *__restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  if (row >= n_rows) return;  // whole wave; no workgroup barrier below

  float key[NPL];
#pragma unroll
  for (int s = 0; s < NPL; ++s) {
    const int i = lane + 64 * s;
    float x = topk::kNegInf;
    if (i < n_experts) {
      if (bf16)
        x = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(logits)[row * n_experts + i] << 16);
      else
        x = reinterpret_cast<const float *>(logits)[row * n_experts + i];
    }
    key[s] = x;
  }
  int sel_i[8];
  float sel_v[8];
  topk::select<NPL>(key, n_experts, top_k, sel_i, sel_v);
  if (lane < top_k) {
    int id = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (lane == k) id = sel_i[k];
    ids[row * top_k + lane] = (uint32_t)id;
    wts[row * top_k + lane] = topk::slot_weight(sel_v, top_k, lane);
  }
}

template <int NPL>
hipError_t launch_npl(const void *logits, int bf16, int64_t n_rows, int n_experts, int top_k,
                      uint32_t *ids, float *wts, hipStream_t stream) {
  const int64_t grid = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(router_topk_kernel<NPL>, dim3((unsigned)grid), dim3(64 * kRowsPerBlock), 0,
                     stream, logits, bf16, n_rows, n_experts, top_k, ids, wts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const void *logits, int bf16, int64_t n_rows, int n_experts, int top_k,
                         uint32_t *ids, float *wts, hipStream_t stream) {
  const int npl = (n_experts + 63) / 64;
  if (npl <= 1) return launch_npl<1>(logits, bf16, n_rows, n_experts, top_k, ids, wts, stream);
  if (npl <= 2) return launch_npl<2>(logits, bf16, n_rows, n_experts, top_k, ids, wts, stream);
  if (npl <= 4) return launch_npl<4>(logits, bf16, n_rows, n_experts, top_k, ids, wts, stream);
  if (npl <= 8) return launch_npl<8>(logits, bf16, n_rows, n_experts, top_k, ids, wts, stream);
  if (npl <= 16) return launch_npl<16>(logits, bf16, n_rows, n_experts, top_k, ids, wts, stream);
  return launch_npl<64>(logits, bf16, n_rows, n_experts, top_k, ids, wts, stream);
}

}  // namespace qint4
