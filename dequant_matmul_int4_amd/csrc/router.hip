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

namespace qint4 {
namespace {

constexpr int kRowsPerBlock = 4;  // waves (rows) per workgroup
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Keep the better of (v, i) and a partner's (pv, pi).
__device__ __forceinline__ void take(float &v, int &i, float pv, int pi) {
  if (better(pv, pi, v, i)) {
    v = pv;
    i = pi;
  }
}

// Wave-wide best (value desc, index asc); every lane gets the winner.  DPP
// within rows of 16 lanes, then the gfx950 permlane16/32 swaps across rows.
__device__ __forceinline__ void wave_best(float &v, int &i) {
#define QINT4_DPP_STEP(CTRL) \
  take(v, i, __int_as_float(dpp<CTRL>(__float_as_int(v))), dpp<CTRL>(i))
  QINT4_DPP_STEP(0xB1);   // quad_perm [1,0,3,2]
  QINT4_DPP_STEP(0x4E);   // quad_perm [2,3,0,1]
  QINT4_DPP_STEP(0x141);  // row_half_mirror
  QINT4_DPP_STEP(0x140);  // row_mirror
#undef QINT4_DPP_STEP
  {
    auto pv = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    auto pi = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
    take(v, i, __uint_as_float(pv[0]), (int)pi[0]);
    take(v, i, __uint_as_float(pv[1]), (int)pi[1]);
  }
  {
    auto pv = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    auto pi = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
    take(v, i, __uint_as_float(pv[0]), (int)pi[0]);
    take(v, i, __uint_as_float(pv[1]), (int)pi[1]);
  }
}

// NPL logits per lane in registers (lane l holds experts l, l + 64, ...).
template <int NPL>
__global__ void __launch_bounds__(64 * kRowsPerBlock)
    router_topk_kernel(const void *__restrict__ logits, int bf16, int64_t n_rows, int n_experts,
                       int top_k, uint32_t *__restrict__ ids, float *__restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  if (row >= n_rows) return;  // whole wave; no workgroup barrier below

  // ranking keys (NaN -> -inf); experts past n_experts are marked taken
  float key[NPL];
  uint64_t taken = 0;
#pragma unroll
  for (int s = 0; s < NPL; ++s) {
    const int i = lane + 64 * s;
    float x = kNegInf;
    if (i < n_experts) {
      if (bf16)
        x = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(logits)[row * n_experts + i] << 16);
      else
        x = reinterpret_cast<const float *>(logits)[row * n_experts + i];
    } else {
      taken |= (uint64_t)1 << s;
    }
    key[s] = (x != x) ? kNegInf : x;
  }

  int sel_i[8];
  float sel_v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sel_i[k] = 0;
    sel_v[k] = kNegInf;
    if (k < top_k) {
      // this lane's best element not chosen in an earlier round
      float bv = kNegInf;
      int bi = 0x7fffffff;
#pragma unroll
      for (int s = 0; s < NPL; ++s)
        if (!((taken >> s) & 1) && better(key[s], lane + 64 * s, bv, bi)) {
          bv = key[s];
          bi = lane + 64 * s;
        }
      wave_best(bv, bi);
      sel_i[k] = __builtin_amdgcn_readfirstlane(bi);
      sel_v[k] = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(bv)));
      if (lane == (sel_i[k] & 63)) taken |= (uint64_t)1 << (sel_i[k] >> 6);
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
