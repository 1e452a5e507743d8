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

// Order-preserving map from logits to int32 keys: for non-NaN a and b,
// a < b as floats iff key(a) < key(b) as signed integers, once -0 is taken
// as +0 (they compare equal as floats).  NaN maps to the key of -inf, so it
// ties with -inf and the lower index goes first.  Every key is above
// kGone, which marks an expert out of play.
constexpr int kGone = (int)0x80000000;
static __device__ __forceinline__ int ordered_key(float x) {
  int i = (x != x) ? __float_as_int(kNegInf) : __float_as_int(x);
  i = (i == kGone) ? 0 : i;  // -0 -> +0
  return i ^ ((i >> 31) & 0x7fffffff);
}
// Inverse of ordered_key (for keys that came from it).
static __device__ __forceinline__ float key_value(int k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7fffffff));
}

// v combined with the value DPP control CTRL moves into each lane of the rows
// in ROWS; lanes of the other rows see kGone (the identity of max) and keep v.
template <int CTRL, int ROWS = 0xF>
static __device__ __forceinline__ int dpp_max(int v) {
  return max(v, __builtin_amdgcn_update_dpp(kGone, v, CTRL, ROWS, 0xF, false));
}

// Wave-wide maximum of integer keys, returned as a uniform value: the row
// reductions by quad permutes and mirrors leave each row of 16 lanes its own
// maximum in every lane, the GFX9 row broadcasts (lane 15 into the next row,
// lane 31 into the upper two rows) fold the four rows into lane 63.
static __device__ __forceinline__ int wave_max(int v) {
  v = dpp_max<0xB1>(v);        // quad_perm [1,0,3,2]
  v = dpp_max<0x4E>(v);        // quad_perm [2,3,0,1]
  v = dpp_max<0x141>(v);       // row_half_mirror
  v = dpp_max<0x140>(v);       // row_mirror
  v = dpp_max<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}

// One row of n_experts logits ranked by one wave: NPL logits per lane (lane l
// holds experts l, l + 64, ...; experts >= n_experts are out of play).  Each
// of the top_k rounds takes the wave-wide maximum m of the keys still in
// play, then the lowest expert index holding m: a ballot of the keys equal to
// m, slot by slot (slot s holds indices 64 s .. 64 s + 63, so the first
// non-empty ballot's lowest lane is the lowest index).  That is the order
// (value desc, index asc); NaN ranks as -inf.
// Returns in every lane: sel_i[k] / sel_v[k] for k < top_k (uniform values;
// a NaN logit comes back as -inf, -0 as +0).
template <int NPL>
static __device__ __forceinline__ void select(const float (&key_in)[NPL], int n_experts, int top_k,
                                              int (&sel_i)[8], float (&sel_v)[8]) {
  const int lane = threadIdx.x & 63;
  int key[NPL];
#pragma unroll
  for (int s = 0; s < NPL; ++s) key[s] = (lane + 64 * s < n_experts) ? ordered_key(key_in[s]) : kGone;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sel_i[k] = 0;
    sel_v[k] = kNegInf;
    if (k < top_k) {
      int bv = key[0];  // this lane's largest key still in play
#pragma unroll
      for (int s = 1; s < NPL; ++s) bv = max(bv, key[s]);
      const int m = wave_max(bv);
      int win = 0x7fffffff;  // no key left in play (the hosts reject top_k > n_experts)
#pragma unroll
      for (int s = NPL - 1; s >= 0; --s) {
        const uint64_t b = __builtin_amdgcn_ballot_w64(key[s] == m);
        if (b) win = 64 * s + (int)__builtin_ctzll(b);
      }
      sel_i[k] = win;
      sel_v[k] = key_value(m);
#pragma unroll
      for (int s = 0; s < NPL; ++s)
        if (win == lane + 64 * s) key[s] = kGone;
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
