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
// One wave per row: the row is staged in the wave's slice of LDS, then top_k
// rounds each take the best not-yet-chosen (value, index) pair of every lane
// and reduce it across the wave.

#include "kernels.h"

namespace qint4 {
namespace {

constexpr int kRowsPerBlock = 4;  // waves (rows) per workgroup
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

__global__ void __launch_bounds__(64 * kRowsPerBlock)
    router_topk_kernel(const void *__restrict__ logits, int bf16, int64_t n_rows, int n_experts,
                       int top_k, uint32_t *__restrict__ ids, float *__restrict__ wts) {
  extern __shared__ float rlds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  if (row >= n_rows) return;  // whole wave; no workgroup barrier below
  float *v = rlds + (size_t)wave * n_experts;

  // stage the row as float32 ranking keys (NaN -> -inf)
  for (int i = lane; i < n_experts; i += 64) {
    float x;
    if (bf16)
      x = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(logits)[row * n_experts + i] << 16);
    else
      x = reinterpret_cast<const float *>(logits)[row * n_experts + i];
    v[i] = (x != x) ? kNegInf : x;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

  int sel_i[8];
  float sel_v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sel_i[k] = -1;
    sel_v[k] = kNegInf;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < top_k) {
      // this lane's best element not chosen in an earlier round
      float bv = kNegInf;
      int bi = 0x7fffffff;
      for (int i = lane; i < n_experts; i += 64) {
        bool taken = false;
#pragma unroll
        for (int q = 0; q < k; ++q) taken = taken || (i == sel_i[q]);
        const float x = v[i];
        if (!taken && better(x, i, bv, bi)) {
          bv = x;
          bi = i;
        }
      }
      // reduce (value, index) across the wave: xor-shuffle butterfly
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      sel_i[k] = __builtin_amdgcn_readfirstlane(bi);
      sel_v[k] = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(bv)));
    }
  }

  // weights: softmax over the kept logits (sel_v[0] is their maximum)
  const float m = sel_v[0];
  float e[8], sum = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    e[k] = (k < top_k && m != kNegInf) ? expf(sel_v[k] - m) : 0.f;
    sum += e[k];
  }
  if (lane < top_k) {
    int id = 0;
    float w = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (lane == k) {
        id = sel_i[k];
        w = (m == kNegInf) ? 1.f / (float)top_k : e[k] / sum;
      }
    ids[row * top_k + lane] = (uint32_t)id;
    wts[row * top_k + lane] = w;
  }
}

}  // namespace

hipError_t launch_router(const void *logits, int bf16, int64_t n_rows, int n_experts, int top_k,
                         uint32_t *ids, float *wts, hipStream_t stream) {
  const int64_t grid = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const size_t lds = (size_t)kRowsPerBlock * n_experts * sizeof(float);
  hipLaunchKernelGGL(router_topk_kernel, dim3((unsigned)grid), dim3(64 * kRowsPerBlock), lds, stream,
                     logits, bf16, n_rows, n_experts, top_k, ids, wts);
  return hipGetLastError();
}

}  // namespace qint4
