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

template <int CTRL>
static __device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Wave-wide maximum, in every lane: DPP within rows of 16 lanes, then the
// gfx950 permlane16/32 swaps across rows.
static __device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
  {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
}

// One row of n_experts logits ranked by one wave: NPL keys per lane (lane l
// holds experts l, l + 64, ...; NaN ranks as -inf, experts >= n_experts are
// excluded).  Each of the top_k rounds takes the wave-wide maximum m of the
// keys still in play, then the lowest expert index holding m: a ballot of
// the keys equal to m, slot by slot (slot s holds indices 64 s .. 64 s + 63,
// so the first non-empty ballot's lowest lane is the lowest index).  That is
// the order (value desc, index asc).
// Returns in every lane: sel_i[k] / sel_v[k] for k < top_k (uniform values).
template <int NPL>
static __device__ __forceinline__ void select(const float (&key_in)[NPL], int n_experts, int top_k,
                                              int (&sel_i)[8], float (&sel_v)[8]) {
  const int lane = threadIdx.x & 63;
  float key[NPL];
  bool live[NPL];
#pragma unroll
  for (int s = 0; s < NPL; ++s) {
    const float x = key_in[s];
    key[s] = (x != x) ? kNegInf : x;
    live[s] = lane + 64 * s < n_experts;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sel_i[k] = 0;
    sel_v[k] = kNegInf;
    if (k < top_k) {
      float bv = kNegInf;  // this lane's largest key still in play
#pragma unroll
      for (int s = 0; s < NPL; ++s) bv = live[s] ? fmaxf(bv, key[s]) : bv;
      const float m = wave_max(bv);
      int win = 0x7fffffff;  // no key left in play (the hosts reject top_k > n_experts)
#pragma unroll
      for (int s = NPL - 1; s >= 0; --s) {
        const uint64_t b = __builtin_amdgcn_ballot_w64(live[s] && key[s] == m);
        if (b) win = 64 * s + (int)__builtin_ctzll(b);
      }
      sel_i[k] = win;
      sel_v[k] = m;
#pragma unroll
      for (int s = 0; s < NPL; ++s)
        if (win == lane + 64 * s) live[s] = false;
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
