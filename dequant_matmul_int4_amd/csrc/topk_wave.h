// topk_wave.h -- wave-wide top-K expert selection for gfx950, shared by the
// router kernel and the MoE gate/up GEMV that routes its own token.
//
// Source: thewafflehaus/FFAI pull 9, "Everything Bagel", top-K partial-sort
// commit: selection order (value desc, index asc).  Weights: thewafflehaus/
// FFAI pull 14, GPU MoE router commit (renormalised softmax over the kept k).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qint4 {
namespace topk {
constexpr float kNegInf = -__builtin_inff();

static __device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

template <int CTRL>
static __device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Keep the better of (v, i) and a partner's (pv, pi).
static __device__ __forceinline__ void take(float &v, int &i, float pv, int pi) {
  if (better(pv, pi, v, i)) {
    v = pv;
    i = pi;
  }
}

// Wave-wide best (value desc, index asc); every lane gets the winner.  DPP
// within rows of 16 lanes, then the gfx950 permlane16/32 swaps across rows.
static __device__ __forceinline__ void wave_best(float &v, int &i) {
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


// One row of n_experts logits ranked by one wave: NPL keys per lane (lane l
// holds experts l, l + 64, ...; NaN ranks as -inf, experts >= n_experts are
// excluded), top_k rounds of the wave-wide best (value desc, index asc).
// Returns in every lane: sel_i[k] / sel_v[k] for k < top_k (uniform values).
template <int NPL>
static __device__ __forceinline__ void select(const float (&key_in)[NPL], int n_experts, int top_k,
                                              int (&sel_i)[8], float (&sel_v)[8]) {
  const int lane = threadIdx.x & 63;
  float key[NPL];
  uint64_t taken = 0;
#pragma unroll
  for (int s = 0; s < NPL; ++s) {
    const float x = key_in[s];
    key[s] = (x != x) ? kNegInf : x;
    if (lane + 64 * s >= n_experts) taken |= (uint64_t)1 << s;
  }
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
}

// Weight of kept slot k: softmax over the kept logits (sel_v[0] is their
// maximum); a row whose kept logits are all -inf gets 1 / top_k.
static __device__ __forceinline__ float slot_weight(const float (&sel_v)[8], int top_k, int k) {
  const float m = sel_v[0];
  if (m == kNegInf) return 1.f / (float)top_k;
  float e[8], sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    e[j] = (j < top_k) ? expf(sel_v[j] - m) : 0.f;
    sum += e[j];
  }
  float ek = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j == k) ek = e[j];
  return ek / sum;
}

}  // namespace topk
}  // namespace qint4
