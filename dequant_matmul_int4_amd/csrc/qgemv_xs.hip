// qgemv_xs.hip -- T=1 int4 group-affine GEMVs with the activation held in
// registers ("activation-stationary") on gfx950: matrices over long rows
// sharing x (the dense FFN down projection, with float32 activations; LM
// heads; large projections), and the gate/up pair with the SwiGLU epilogue
// (the dense FFN gate/up projection), each optionally behind the RMSNorm
// prologue.
//
// Sources (by page title and passage):
//   [FFAI #14] thewafflehaus/FFAI pull 14, "feat(everything-bagel): clean
//              migration of PR #9 + #10 onto updated dev": int4 GEMV wrapper
//              (weight, scales, biases, in_dim, group_size); the down
//              projection reads the float32 SwiGLU intermediate.
//   [FFAI #9]  thewafflehaus/FFAI pull 9, "Everything Bagel": fused swiglu,
//              h = silu(gate) * up with silu(g) = g / (1 + exp(-g)).
//
// Per row and group the product is the affine form of the GEMV family,
//     sum_k (s q_k + b) x_k = s * sum_k q_k x_k + b * sum_k x_k,
// accumulated in float32: for float32 activations a masked nibble pair is
// the f16 pair (q 2^-24, q' 2^-24) or (16 q 2^-24, 16 q' 2^-24), exact
// subnormals, which v_fma_mix_f32 multiplies by activations stored times 2^24
// or 2^20 (activations of magnitude 2^104 or more overflow there); for bf16
// activations a nibble pair (q_i, q_{i+4}) of a word becomes the exact bf16
// pair (128 + q_i, 128 + q_{i+4}) (bits 0x4300 | q) for v_dot2_f32_bf16, and
// 128 * sum x is removed per chunk, as in the streaming GEMV.
//
// Work decomposition (gfx950 specific, not from the pages):
//   * L lanes (32 or 64) cover one row, so a wave takes 64 / L rows per
//     step.  Lane j of a row group in wave w takes the 32-code chunk
//     c = L w + j of its rows and keeps that chunk's 32 activation values in
//     registers for the whole launch: nothing is staged in LDS and the dot
//     products issue no LDS reads.  A workgroup's ceil(k_in / 32 / L) waves
//     cover k_in; lanes past the last chunk load nothing.
//   * Workgroup b of G takes rows b, b + G, b + 2G, ...: at any moment the
//     grid streams one compact band of each matrix, each row group of a wave
//     reading L * 16 contiguous bytes of a row per stream.  The gate/up pair
//     takes a contiguous block of rows per workgroup instead.
//   * Each wave keeps 4 rows of code, scale and bias loads (per stream) in
//     flight; the loads sit between scheduling barriers, so they are issued
//     where the ring needs them (the compiler otherwise gathers them at the
//     end of the loop body and waits for all of them at its top).
//   * Every 4 rows the per-lane partials are reduced across the wave
//     (permlane32 / permlane16 swaps, then DPP within rows of 16 lanes),
//     leaving row r of the block in the 16 lanes whose bits (5, 4) are
//     (r >> 1, r & 1).  Each wave's row sums go to LDS; after one workgroup
//     barrier they are summed in wave order, and the epilogue (SwiGLU for the
//     pair) runs before the store.
#include <algorithm>

#include "kernels.h"

namespace qint4 {
namespace {

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kXsRowsInFlight = 4;  // per wave (8 measured slower on the down projection)

typedef __bf16 xs_bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 xs_f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t xs_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 xs_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One scale or bias: raw bits (bf16 in the low half, or float32).
template <int SBT>
__device__ __forceinline__ uint32_t xs_load_sb(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (SBT == 1)
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  else
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

template <int SBT>
__device__ __forceinline__ float xs_sb_value(uint32_t bits) {
  return __uint_as_float(SBT == 1 ? bits << 16 : bits);
}

__device__ __forceinline__ float xs_bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float xs_bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int CTRL>
__device__ __forceinline__ float xs_dpp(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum within aligned groups of 16 lanes (every lane gets its group's sum).
__device__ __forceinline__ float xs_sum16(float t) {
  t += xs_dpp<0xB1>(t);   // quad_perm [1,0,3,2]
  t += xs_dpp<0x4E>(t);   // quad_perm [2,3,0,1]
  t += xs_dpp<0x141>(t);  // row_half_mirror
  t += xs_dpp<0x140>(t);  // row_mirror
  return t;
}

// a[m] for a uniform m, by selects (no indexed copy of the kernel arguments)
template <typename T>
__device__ __forceinline__ T xs_pick(const T (&a)[kXsMaxMats], int m) {
  T r = a[0];
#pragma unroll
  for (int i = 1; i < kXsMaxMats; ++i) r = m == i ? a[i] : r;
  return r;
}
__device__ __forceinline__ int32_t xs_pick(const int32_t (&a)[kXsMaxMats + 1], int m) {
  int32_t r = a[0];
#pragma unroll
  for (int i = 1; i <= kXsMaxMats; ++i) r = m == i ? a[i] : r;
  return r;
}

// The activation of one chunk in the form the dot product takes: float32
// values in element order, times 2^24 at even and 2^20 at odd positions
// (XB = false), or the 16 bf16 pairs (x[8 jj + i], x[8 jj + i + 4]) of the
// nibble pairs (XB = true).
template <bool XB>
struct XsChunk {
  uint32_t v[XB ? 16 : 32];
};

// Two code words shifted right by 4 s bits as one 64-bit value: one
// v_lshrrev_b64 instead of two 32-bit shifts (the compiler splits a 64-bit
// shift whose halves are masked).  The high word's low nibbles that move into
// the top of the low word are masked off by the caller.
template <int S>
__device__ __forceinline__ uint64_t xs_shr64(uint64_t w) {
  uint64_t r;
  asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "n"(4 * S), "v"(w));
  return r;
}

// sum over the chunk of q_k x_k (float32 activations).  A word masked with
// 0x000F000F holds nibbles (n, n + 4) as the f16 subnormals q 2^-24, masked
// with 0x00F000F0 nibbles (n + 1, n + 5) as 16 q 2^-24; v_fma_mix_f32 takes
// them exactly, against activations stored times 2^24 and 2^20 respectively
// (XsChunk<false>), so each step is fmaf(q, x, t) with one rounding.  Masks
// on the word and on the word shifted by 8 give all eight nibbles.
__device__ __forceinline__ float xs_dot_f32(const uint4 q, const XsChunk<false> &x) {
  const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
  float a[2];  // one chain per word pair
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint64_t w2 = ((uint64_t)wd[2 * h + 1] << 32) | wd[2 * h];
    const uint64_t w8 = xs_shr64<2>(w2);
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t u0 = (uint32_t)(w2 >> (32 * e)), u8 = (uint32_t)(w8 >> (32 * e));
      const xs_f16x2_t p0 = __builtin_bit_cast(xs_f16x2_t, u0 & 0x000F000Fu);  // nibbles 0, 4
      const xs_f16x2_t p1 = __builtin_bit_cast(xs_f16x2_t, u0 & 0x00F000F0u);  // 1, 5 (times 16)
      const xs_f16x2_t p2 = __builtin_bit_cast(xs_f16x2_t, u8 & 0x000F000Fu);  // 2, 6
      const xs_f16x2_t p3 = __builtin_bit_cast(xs_f16x2_t, u8 & 0x00F000F0u);  // 3, 7 (times 16)
      const uint32_t *xe = x.v + 8 * (2 * h + e);
      t = fmaf((float)p0.x, __uint_as_float(xe[0]), t);
      t = fmaf((float)p1.x, __uint_as_float(xe[1]), t);
      t = fmaf((float)p2.x, __uint_as_float(xe[2]), t);
      t = fmaf((float)p3.x, __uint_as_float(xe[3]), t);
      t = fmaf((float)p0.y, __uint_as_float(xe[4]), t);
      t = fmaf((float)p1.y, __uint_as_float(xe[5]), t);
      t = fmaf((float)p2.y, __uint_as_float(xe[6]), t);
      t = fmaf((float)p3.y, __uint_as_float(xe[7]), t);
    }
    a[h] = t;
  }
  return a[0] + a[1];
}

// sum over the chunk of (128 + q_k) x_k (bf16 activations)
__device__ __forceinline__ float xs_dot_bf16(const uint4 q, const XsChunk<true> &x, uint32_t magic) {
  const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
  float a[4];  // one chain per word
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint64_t w2 = ((uint64_t)wd[2 * h + 1] << 32) | wd[2 * h];
    const uint64_t sh[4] = {w2, xs_shr64<1>(w2), xs_shr64<2>(w2), xs_shr64<3>(w2)};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jj = 2 * h + e;
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // nibbles i and i + 4 of word jj
        const uint32_t pq = ((uint32_t)(sh[i] >> (32 * e)) & 0x000F000Fu) | magic;
        t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(xs_bf16x2_t, pq),
                                            __builtin_bit_cast(xs_bf16x2_t, x.v[4 * jj + i]), t, false);
      }
      a[jj] = t;
    }
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// XB: bf16 activations into the bf16 dot product; NS: code streams (1 stored
// outputs, 2 the gate/up pair); L2: log2 of the lanes per row (5 or 6); RM:
// RMSNorm prologue, 0 none, 1 with bf16 x and gamma, 2 with float32 (the
// float32 dot product on x * gamma).
template <int SBT, bool XB, int NS, int L2, int RM>
__global__ void __launch_bounds__(kXsMaxWaves * 64) qgemv_xs_kernel(const GemvXsParams p) {
  constexpr int L = 1 << L2;
  constexpr int RPS = 64 / L;                  // rows per step
  constexpr int D = kXsRowsInFlight / RPS;     // steps in flight
  constexpr int SPB = 4 / RPS;                 // steps per block of 4 rows
  constexpr uint32_t SBB = SBT == 1 ? 2u : 4u;
  constexpr bool XIN16 = XB || RM == 1;        // activations stored as bf16
  constexpr uint32_t XCB = XIN16 ? 64u : 128u;  // activation bytes of one chunk
  static_assert(L2 == 5 || L2 == 6, "32 or 64 lanes per row");
  static_assert(RM == 0 || !XB, "the RMSNorm form takes the float32 dot product");
  // per-row sums of each wave and stream; row kXsMaxRows takes the lanes that
  // hold no row
  __shared__ float part[NS][kXsMaxRows + 1][kXsMaxWaves + 1];
  __shared__ float ssq_part[kXsMaxWaves];  // RM: each wave's share of sum(x^2)

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = p.waves;
  const int sg = lane >> L2;              // row group of the lane inside a step
  const int c = L * w + (lane & (L - 1));  // this lane's chunk
  const bool active = c < p.ncx;
  // this workgroup's matrix m (uniform) and its place b among matrix m's G
  const int bid = (int)blockIdx.x;
  int m = 0;
#pragma unroll
  for (int i = 1; i < kXsMaxMats; ++i) m = (i < p.n_mats && bid >= p.wg0[i]) ? i : m;
  const int G = xs_pick(p.wg0, m + 1) - xs_pick(p.wg0, m), b = bid - xs_pick(p.wg0, m);
  const int n_out = xs_pick(p.n_out, m);
  // Rows of this workgroup (<= kXsMaxRows): stored outputs take rows b, b + G,
  // ... (the grid streams one compact band of each matrix); the pair takes the
  // contiguous block of rows b * RB .. (measured faster for the pair: 17408 x
  // 5120 21.45 -> 20.86 us, 8192 x 2048 6.73 -> 6.34 us; slower for one
  // matrix: the float32 down projection 12.51 -> 13.03 us, 128256 x 2048
  // 29.9 -> 31.1 us).
  constexpr bool BLOCK = NS == 2;
  const int RB = (n_out + G - 1) / G;
  const int nr = BLOCK ? max(0, min(RB, n_out - b * RB)) : (n_out - b + G - 1) / G;

  const __amdgpu_buffer_rsrc_t rx = xs_rsrc(p.x, (uint32_t)p.ncx * XCB);
  __amdgpu_buffer_rsrc_t rc[NS], rs[NS], rb[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int ms = NS == 2 ? s : m;  // the pair's streams, or this matrix
    rc[s] = xs_rsrc(xs_pick(p.codes, ms), (uint32_t)n_out * (uint32_t)p.kwb);
    rs[s] = xs_rsrc(xs_pick(p.scales, ms), (uint32_t)n_out * (uint32_t)p.sbrow);
    rb[s] = xs_rsrc(xs_pick(p.biases, ms), (uint32_t)n_out * (uint32_t)p.sbrow);
  }

  // the chunk's activation (and RMSNorm weight): loads first, turned into
  // registers after the first code loads are issued
  constexpr int XV = XIN16 ? 4 : 8;
  uint4 xv[XV], gv[RM ? XV : 1];
  {
    const uint32_t xo = active ? (uint32_t)c * XCB : kOutOfRange;
#pragma unroll
    for (int i = 0; i < XV; ++i) xv[i] = xs_load16(rx, xo + 16u * i);
    if constexpr (RM != 0) {
      const __amdgpu_buffer_rsrc_t rg = xs_rsrc(p.gamma, (uint32_t)p.ncx * XCB);
#pragma unroll
      for (int i = 0; i < XV; ++i) gv[i] = xs_load16(rg, xo + 16u * i);
    }
  }

  // byte offsets of this lane's next row: a running sum, advanced by the
  // (uniform) distance between a wave's consecutive steps
  const uint32_t row0 = (uint32_t)(BLOCK ? b * RB + sg : b + G * sg);
  uint32_t run_c = row0 * (uint32_t)p.kwb + (uint32_t)c * 16u;
  uint32_t run_s = row0 * (uint32_t)p.sbrow + (((uint32_t)c * 32u) >> p.log2_group) * SBB;
  const uint32_t row_step = (uint32_t)(BLOCK ? RPS : RPS * G);  // rows between a wave's steps
  const uint32_t step_c = row_step * (uint32_t)p.kwb;
  const uint32_t step_s = row_step * (uint32_t)p.sbrow;
  uint4 q[D][NS];
  uint32_t sv[D][NS], bv[D][NS];
  int issued = 0;  // steps issued by this wave (uniform)
  auto issue = [&](int u) {
    // rows past the workgroup's last are out of range: the loads are still
    // issued, so the number in flight, and every wait, is static (the running
    // offsets may wrap there; they are not used)
    const bool ok = active && RPS * issued + sg < nr;
    const uint32_t oc = ok ? run_c : kOutOfRange;
    const uint32_t os = ok ? run_s : kOutOfRange;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      q[u][s] = xs_load16(rc[s], oc);
      sv[u][s] = xs_load_sb<SBT>(rs[s], os);
      bv[u][s] = xs_load_sb<SBT>(rb[s], os);
    }
    __builtin_amdgcn_sched_barrier(0);
    run_c += step_c;
    run_s += step_s;
    ++issued;
  };
#pragma unroll
  for (int u = 0; u < D; ++u) issue(u);

  XsChunk<XB> xc;
  float xs = 0.f;   // sum of the chunk's activation values
  float ssq = 0.f;  // RM: this lane's sum of x^2 over its chunk
  if constexpr (XB) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t w0 = xv[jj].x, w1 = xv[jj].y, w2 = xv[jj].z, w3 = xv[jj].w;  // x[8jj .. 8jj+7]
      xc.v[4 * jj + 0] = (w0 & 0xFFFFu) | (w2 << 16);
      xc.v[4 * jj + 1] = (w0 >> 16) | (w2 & 0xFFFF0000u);
      xc.v[4 * jj + 2] = (w1 & 0xFFFFu) | (w3 << 16);
      xc.v[4 * jj + 3] = (w1 >> 16) | (w3 & 0xFFFF0000u);
      xs += ((xs_bf16_lo(w0) + xs_bf16_hi(w0)) + (xs_bf16_lo(w1) + xs_bf16_hi(w1))) +
            ((xs_bf16_lo(w2) + xs_bf16_hi(w2)) + (xs_bf16_lo(w3) + xs_bf16_hi(w3)));
    }
  } else {
    // the chunk's values in element order (RM: x * gamma, with this lane's
    // share of sum(x^2))
    float e[32];
    if constexpr (XIN16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          e[8 * i + 2 * j] = xs_bf16_lo(w[j]);
          e[8 * i + 2 * j + 1] = xs_bf16_hi(w[j]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[4 * i] = __uint_as_float(xv[i].x);
        e[4 * i + 1] = __uint_as_float(xv[i].y);
        e[4 * i + 2] = __uint_as_float(xv[i].z);
        e[4 * i + 3] = __uint_as_float(xv[i].w);
      }
    }
    if constexpr (RM != 0) {
      float g[32];
      if constexpr (RM == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            g[8 * i + 2 * j] = xs_bf16_lo(w[j]);
            g[8 * i + 2 * j + 1] = xs_bf16_hi(w[j]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          g[4 * i] = __uint_as_float(gv[i].x);
          g[4 * i + 1] = __uint_as_float(gv[i].y);
          g[4 * i + 2] = __uint_as_float(gv[i].z);
          g[4 * i + 3] = __uint_as_float(gv[i].w);
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        ssq = fmaf(e[i], e[i], ssq);
        e[i] *= g[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) xc.v[i] = __float_as_uint(e[i]);
#pragma unroll
    for (int i = 0; i < 32; ++i) xs += e[i];
    // even nibble positions pair with codes q 2^-24, odd ones with 16 q 2^-24
#pragma unroll
    for (int i = 0; i < 32; ++i) xc.v[i] = __float_as_uint(__uint_as_float(xc.v[i]) * ((i & 1) ? 0x1p20f : 0x1p24f));
  }
  // The chunk has arrived (xs waited for it).  Redefining its registers keeps
  // the compiler from treating the loop below as a consumer of loads issued
  // before it, for which it would wait on every load at the loop top.
#pragma unroll
  for (int i = 0; i < (XB ? 16 : 32); ++i) asm volatile("" : "+v"(xc.v[i]));
  asm volatile("" : "+v"(xs));
  if constexpr (RM != 0) asm volatile("" : "+v"(ssq));
  uint32_t magic = 0x43004300u;
  asm volatile("" : "+v"(magic));  // a VGPR operand, so the AND-OR stays one VOP3
  const float corr = XB ? -128.f * xs : 0.f;

  const int nsteps = (nr + RPS - 1) / RPS;
  for (int base = 0; base < nsteps; base += D) {
#pragma unroll
    for (int blk = 0; blk < D / SPB; ++blk) {
      float v[NS][SPB];
#pragma unroll
      for (int i = 0; i < SPB; ++i) {
        const int u = SPB * blk + i;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          float d;
          if constexpr (XB)
            d = xs_dot_bf16(q[u][s], xc, magic) + corr;
          else
            d = xs_dot_f32(q[u][s], xc);
          v[s][i] = fmaf(xs_sb_value<SBT>(sv[u][s]), d, xs_sb_value<SBT>(bv[u][s]) * xs);
        }
        issue(u);
      }
      // the block's 4 rows across the wave; row r ends in the 16 lanes with
      // (bit 5, bit 4) = (r >> 1, r & 1)
      const int step0 = base + SPB * blk;
      int rr;
      if constexpr (L2 == 6) {
        rr = RPS * step0 + 2 * ((lane >> 5) & 1) + ((lane >> 4) & 1);
      } else {
        // step step0 + (bit 4), row group (bit 5)
        rr = RPS * (step0 + ((lane >> 4) & 1)) + ((lane >> 5) & 1);
      }
      const int slot = ((lane & 15) == 0 && rr < nr) ? rr : kXsMaxRows;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float t;
        if constexpr (L2 == 6) {
          // steps i = 0..3 hold rows i; pair rows (0, 2) and (1, 3) across the halves
          auto r0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[s][0]), __float_as_uint(v[s][2]), false, false);
          auto r1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[s][1]), __float_as_uint(v[s][3]), false, false);
          const float s0 = __uint_as_float(r0[0]) + __uint_as_float(r0[1]);
          const float s1 = __uint_as_float(r1[0]) + __uint_as_float(r1[1]);
          auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(s0), __float_as_uint(s1), false, false);
          t = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
        } else {
          // steps i = 0, 1 hold rows 2 i + (bit 5)
          auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[s][0]), __float_as_uint(v[s][1]), false, false);
          t = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
        }
        part[s][slot][w] = xs_sum16(t);
      }
    }
  }
  if constexpr (RM != 0) {
    // each chunk sits in 64 / L lanes of a wave: count row group 0's
    const float t16 = xs_sum16(sg == 0 ? ssq : 0.f);
    const int tb = __float_as_int(t16);
    const float wsum = (__int_as_float(__builtin_amdgcn_readlane(tb, 0)) +
                        __int_as_float(__builtin_amdgcn_readlane(tb, 16))) +
                       (__int_as_float(__builtin_amdgcn_readlane(tb, 32)) +
                        __int_as_float(__builtin_amdgcn_readlane(tb, 48)));
    if (lane == 0) ssq_part[w] = wsum;
  }
  __syncthreads();
  // RMSNorm: every thread sums the waves' shares in the same order
  float inv_rms = 1.f;
  if constexpr (RM != 0) {
    float tot = 0.f;
    for (int k = 0; k < W; ++k) tot += ssq_part[k];
    inv_rms = 1.f / sqrtf(tot / (float)(p.ncx * 32) + p.eps);
  }
  for (int t = (int)threadIdx.x; t < nr; t += W * 64) {
    float acc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      acc[s] = 0.f;
      for (int k = 0; k < W; ++k) acc[s] += part[s][t][k];
      if constexpr (RM != 0) acc[s] *= inv_rms;
    }
    float out = acc[0];
    if constexpr (NS == 2) out = (acc[0] / (1.f + __expf(-acc[0]))) * acc[1];  // silu(gate) * up
    const int64_t row = BLOCK ? (int64_t)b * RB + t : (int64_t)b + (int64_t)G * t;
    void *y = xs_pick(p.y, m);
    if (p.y_bf16)
      reinterpret_cast<__bf16 *>(y)[row] = (__bf16)out;
    else
      reinterpret_cast<float *>(y)[row] = out;
  }
}

template <int SBT, bool XB, int NS, int RM = 0>
hipError_t xs_launch(const GemvXsParams &p, int64_t grid, hipStream_t stream) {
  auto kern = p.log2_lpr == 5 ? qgemv_xs_kernel<SBT, XB, NS, 5, RM> : qgemv_xs_kernel<SBT, XB, NS, 6, RM>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(p.waves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Lanes per row: 32 while that needs at most kXsMaxWaves waves (k_in up to
// 16384), else 64.
int gemv_xs_log2_lanes(int64_t k_in) { return (k_in / 32 + 31) / 32 <= kXsMaxWaves ? 5 : 6; }

int gemv_xs_waves(int64_t k_in) {
  const int64_t L = (int64_t)1 << gemv_xs_log2_lanes(k_in);
  return (int)((k_in / 32 + L - 1) / L);
}

// Where the form applies, from cold-weight timings (a 1.2 GB pool of copies)
// against the streaming GEMV:
//   * stored outputs (bf16 or float32 activations): k_in >= 2048 and at least
//     26,214,400 codes (5120 x 5120) in all (bf16: 5120 x 5120 7.41 -> 6.38 us,
//     8192 x 8192 11.1 -> 9.6 us, 17408 x 5120 14.6 -> 12.1 us, 2048 x 32768
//     13.4 -> 9.6 us, 12800 x 2048 9.0 -> 6.3 us, 128256 x 2048 86.7 -> 30.0
//     us; 6144 x 4096, q/k/v 4096 -> 4096/1024/1024 and 4096 x 4096 are even
//     or faster on the streaming GEMV: 5.6 against 6.0 us for q/k/v);
//   * the gate/up pair: k_in >= 2048 and 2^25 codes (8192 x 2048 7.67 ->
//     6.72 us, 8192 x 3072 9.00 -> 8.57 us, 14336 x 4096 16.1 -> 14.9 us;
//     5632 x 2048 and smaller pairs are faster on the streaming GEMV).
// Workgroups per CU: for the gate/up pair 16 / waves, one to four (17408 x
// 5120 23.2 -> 20.6 us at three, 8192 x 8192 14.6 us at four -> 14.2 at two,
// 3072 x 16384 13.3 us at four -> 10.4 at one; eight for two-wave pairs is
// 30% slower); for stored outputs four up to three waves, two up to eight,
// else one (cold, bf16: 128256 x 2048 46.8 -> 30.0 us at four instead of
// two; 6144 x 6144 8.0 -> 7.2 us and 5120 x 5120 6.9 -> 6.4 us at two;
// 5120 x 17408 11.9 -> 12.4 us and 4096 x 14336 9.0 -> 9.5 us at two); more
// where a workgroup would get over kXsMaxRows rows.  One matrix takes
// min(that, n_out) workgroups; several matrices take ceil(n_out / r) each,
// r = the rows per workgroup of all their rows over that many workgroups.
bool gemv_xs_plan(int n_mats, const int64_t *n_out, int64_t k_in, int streams, int n_cu, int32_t *wg0) {
  if (n_mats < 1 || n_mats > kXsMaxMats || (streams == 2 && n_mats != 1) || (streams != 1 && streams != 2))
    return false;
  const int64_t min_codes = streams == 2 ? ((int64_t)1 << 25) : (int64_t)5120 * 5120;
  if (k_in < 2048 || k_in > (int64_t)kXsMaxWaves * 2048 || k_in % 32 != 0) return false;
  int64_t rows = 0;
  for (int i = 0; i < n_mats; ++i) {
    if (n_out[i] < 1) return false;
    rows += n_out[i];
  }
  if (rows * k_in * streams < min_codes || rows > INT32_MAX) return false;
  const int w = gemv_xs_waves(k_in);
  const int per_cu = streams == 2 ? std::max(1, std::min(4, 16 / w)) : (w <= 3 ? 4 : w <= 8 ? 2 : 1);
  // more workgroups where that would leave over kXsMaxRows rows to one
  const int64_t target = std::max<int64_t>((int64_t)n_cu * per_cu, (rows + kXsMaxRows - 1) / kXsMaxRows);
  const int64_t r = (rows + target - 1) / target;  // rows per workgroup (several matrices)
  int64_t g = 0;
  wg0[0] = 0;
  for (int i = 0; i < n_mats; ++i) {
    const int64_t gi = n_mats == 1 ? std::min<int64_t>(target, n_out[0]) : (n_out[i] + r - 1) / r;
    if (gi < 1 || (n_out[i] + gi - 1) / gi > kXsMaxRows) return false;
    g += gi;
    if (g > INT32_MAX) return false;
    wg0[i + 1] = (int32_t)g;
  }
  return true;
}

int gemv_xs_depth() { return kXsRowsInFlight; }

hipError_t launch_gemv_xs(const GemvXsParams &p, int sb_bf16, int x_bf16, int streams, hipStream_t stream) {
  const int64_t k_in = (int64_t)p.ncx * 32;
  if (p.log2_lpr != gemv_xs_log2_lanes(k_in) || p.waves != gemv_xs_waves(k_in) || p.waves < 1 ||
      p.waves > kXsMaxWaves || (streams != 1 && streams != 2) || p.n_mats < 1 || p.n_mats > kXsMaxMats ||
      (streams == 2 && p.n_mats != 1) || p.wg0[0] != 0)
    return hipErrorInvalidValue;
  for (int i = 0; i < p.n_mats; ++i) {
    const int64_t gi = (int64_t)p.wg0[i + 1] - p.wg0[i];
    if (gi < 1 || gi > p.n_out[i] || ((int64_t)p.n_out[i] + gi - 1) / gi > kXsMaxRows) return hipErrorInvalidValue;
  }
  const int64_t grid = p.wg0[p.n_mats];
  if (p.gamma) {  // RMSNorm prologue: the float32 dot product on x * gamma
    if (streams == 2)
      return x_bf16 ? (sb_bf16 ? xs_launch<1, false, 2, 1>(p, grid, stream) : xs_launch<0, false, 2, 1>(p, grid, stream))
                    : (sb_bf16 ? xs_launch<1, false, 2, 2>(p, grid, stream) : xs_launch<0, false, 2, 2>(p, grid, stream));
    return x_bf16 ? (sb_bf16 ? xs_launch<1, false, 1, 1>(p, grid, stream) : xs_launch<0, false, 1, 1>(p, grid, stream))
                  : (sb_bf16 ? xs_launch<1, false, 1, 2>(p, grid, stream) : xs_launch<0, false, 1, 2>(p, grid, stream));
  }
  if (streams == 2)
    return x_bf16 ? (sb_bf16 ? xs_launch<1, true, 2>(p, grid, stream) : xs_launch<0, true, 2>(p, grid, stream))
                  : (sb_bf16 ? xs_launch<1, false, 2>(p, grid, stream) : xs_launch<0, false, 2>(p, grid, stream));
  return x_bf16 ? (sb_bf16 ? xs_launch<1, true, 1>(p, grid, stream) : xs_launch<0, true, 1>(p, grid, stream))
                : (sb_bf16 ? xs_launch<1, false, 1>(p, grid, stream) : xs_launch<0, false, 1>(p, grid, stream));
}

}  // namespace qint4
