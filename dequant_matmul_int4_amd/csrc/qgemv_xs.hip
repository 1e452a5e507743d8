// qgemv_xs.hip -- T=1 int4 group-affine GEMV with float32 activations for
// long rows (the dense FFN down projection), "activation-stationary" on gfx950.
//
// Sources (by page title and passage):
//   [FFAI #14] thewafflehaus/FFAI pull 14, "feat(everything-bagel): clean
//              migration of PR #9 + #10 onto updated dev": int4 GEMV wrapper
//              (weight, scales, biases, in_dim, group_size); the down
//              projection reads the float32 SwiGLU intermediate.
//
// Per row and group the product is the affine form of the GEMV family,
//     sum_k (s q_k + b) x_k = s * sum_k q_k x_k + b * sum_k x_k,
// with q_k x_k accumulated in float32 (q from v_cvt_f32_ubyte of the masked
// code bytes, as in the streaming GEMV's float32 path).
//
// Work decomposition (gfx950 specific, not from the pages):
//   * Each wave owns a 2048-wide slice of k_in: lane l of wave w takes the
//     32-code chunk c = 64 w + l of every row and keeps its 32 activation
//     values in registers for the whole launch (nothing is staged in LDS, so
//     the dot products issue no LDS reads).  A workgroup's waves cover k_in
//     (ceil(k_in / 2048) of them; lanes past the last chunk load nothing).
//   * Workgroup b of G takes rows b, b + G, b + 2G, ...: at any moment the
//     grid streams one compact band of the matrix, and every wave reads one
//     1 KB span of each row (64 lanes x 16 contiguous bytes).
//   * Each wave keeps D rows of code, scale and bias loads in flight; the
//     loads sit between scheduling barriers so they are issued where the
//     ring needs them (the compiler otherwise gathers them at the end of the
//     loop body and waits for all of them at its top).
//   * Every 4 rows the 4 per-lane partials are reduced across the wave:
//     one permlane32 swap per pair of rows, one permlane16 swap, then DPP
//     within rows of 16 lanes, leaving row r of the block in the 16 lanes
//     (bit 5, bit 4) = (r >> 1, r & 1).  The wave's row sums go to LDS and,
//     after one workgroup barrier, are summed in wave order and stored.
#include <algorithm>

#include "kernels.h"

namespace qint4 {
namespace {

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kXsDepth = 4;  // rows in flight per wave (8 measured slower)

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

template <int CTRL>
__device__ __forceinline__ float xs_dpp(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int SBT, int D>
__global__ void __launch_bounds__(kXsMaxWaves * 64) qgemv_xs_kernel(const GemvXsParams p) {
  static_assert(D % 4 == 0, "rows are reduced in blocks of 4");
  constexpr uint32_t SBB = SBT == 1 ? 2u : 4u;
  // per-row sums of each wave; row kXsMaxRows takes the lanes that hold no row
  __shared__ float part[kXsMaxRows + 1][kXsMaxWaves + 1];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = p.waves;
  const int c = 64 * w + lane;  // this lane's chunk
  const bool active = c < p.ncx;
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  const int nr = (p.n_out - b + G - 1) / G;  // rows of this workgroup, <= kXsMaxRows

  const __amdgpu_buffer_rsrc_t rx = xs_rsrc(p.x, (uint32_t)p.ncx * 128u);
  const __amdgpu_buffer_rsrc_t rc = xs_rsrc(p.codes, (uint32_t)p.n_out * (uint32_t)p.kwb);
  const __amdgpu_buffer_rsrc_t rs = xs_rsrc(p.scales, (uint32_t)p.n_out * (uint32_t)p.sbrow);
  const __amdgpu_buffer_rsrc_t rb = xs_rsrc(p.biases, (uint32_t)p.n_out * (uint32_t)p.sbrow);

  // the chunk's 32 activation values, element order
  float xr[32];
  {
    const uint32_t xo = active ? (uint32_t)c * 128u : kOutOfRange;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = xs_load16(rx, xo + 16u * i);
      xr[4 * i] = __uint_as_float(v.x);
      xr[4 * i + 1] = __uint_as_float(v.y);
      xr[4 * i + 2] = __uint_as_float(v.z);
      xr[4 * i + 3] = __uint_as_float(v.w);
    }
  }

  const uint32_t lane_c = (uint32_t)c * 16u;
  const uint32_t lane_s = (((uint32_t)c * 32u) >> p.log2_group) * SBB;
  uint4 q[D];
  uint32_t sv[D], bv[D];
  int issued = 0;  // rows issued by this wave (uniform)
  auto issue = [&](int u) {
    // rows past the workgroup's last are out of range: the load is still
    // issued, so the number in flight, and every wait, is static
    const bool ok = active && issued < nr;
    const uint32_t row = (uint32_t)(b + G * issued);
    const uint32_t oc = ok ? row * (uint32_t)p.kwb + lane_c : kOutOfRange;
    const uint32_t os = ok ? row * (uint32_t)p.sbrow + lane_s : kOutOfRange;
    __builtin_amdgcn_sched_barrier(0);
    q[u] = xs_load16(rc, oc);
    sv[u] = xs_load_sb<SBT>(rs, os);
    bv[u] = xs_load_sb<SBT>(rb, os);
    __builtin_amdgcn_sched_barrier(0);
    ++issued;
  };
#pragma unroll
  for (int u = 0; u < D; ++u) issue(u);

  float xs = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) xs += xr[i];
  // The slice has arrived (xs waited for it).  Redefining the registers here
  // keeps the compiler from treating the loop below as a consumer of loads
  // issued before it, for which it would wait on every load at the loop top.
#pragma unroll
  for (int i = 0; i < 32; ++i) asm volatile("" : "+v"(xr[i]));

  for (int base = 0; base < nr; base += D) {
#pragma unroll
    for (int blk = 0; blk < D / 4; ++blk) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int u = 4 * blk + i;
        const uint32_t wd[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
        float a[4];  // one chain per word
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          // bytes of lo: nibbles 0, 2, 4, 6; of hi: nibbles 1, 3, 5, 7
          uint32_t lo = wd[jj] & 0x0F0F0F0Fu, hi = (wd[jj] >> 4) & 0x0F0F0F0Fu;
          asm("" : "+v"(lo), "+v"(hi));  // keep the byte split (v_cvt_f32_ubyte{0..3})
          const float *xe = xr + 8 * jj;
          float t = (float)(lo & 0xFFu) * xe[0];
          t = fmaf((float)(hi & 0xFFu), xe[1], t);
          t = fmaf((float)((lo >> 8) & 0xFFu), xe[2], t);
          t = fmaf((float)((hi >> 8) & 0xFFu), xe[3], t);
          t = fmaf((float)((lo >> 16) & 0xFFu), xe[4], t);
          t = fmaf((float)((hi >> 16) & 0xFFu), xe[5], t);
          t = fmaf((float)(lo >> 24), xe[6], t);
          t = fmaf((float)(hi >> 24), xe[7], t);
          a[jj] = t;
        }
        const float d = (a[0] + a[1]) + (a[2] + a[3]);
        v[i] = fmaf(xs_sb_value<SBT>(sv[u]), d, xs_sb_value<SBT>(bv[u]) * xs);
        issue(u);
      }
      // rows base + 4 blk + r, r = 0..3, across the wave
      auto r0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[2]), false, false);
      auto r1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1]), __float_as_uint(v[3]), false, false);
      const float s0 = __uint_as_float(r0[0]) + __uint_as_float(r0[1]);  // rows 0 | 2
      const float s1 = __uint_as_float(r1[0]) + __uint_as_float(r1[1]);  // rows 1 | 3
      auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(s0), __float_as_uint(s1), false, false);
      float t = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
      t += xs_dpp<0xB1>(t);   // quad_perm [1,0,3,2]
      t += xs_dpp<0x4E>(t);   // quad_perm [2,3,0,1]
      t += xs_dpp<0x141>(t);  // row_half_mirror
      t += xs_dpp<0x140>(t);  // row_mirror
      const int rr = base + 4 * blk + 2 * ((lane >> 5) & 1) + ((lane >> 4) & 1);
      part[((lane & 15) == 0 && rr < nr) ? rr : kXsMaxRows][w] = t;
    }
  }
  __syncthreads();
  for (int t = (int)threadIdx.x; t < nr; t += W * 64) {
    float s = 0.f;
    for (int k = 0; k < W; ++k) s += part[t][k];
    const int64_t row = (int64_t)b + (int64_t)G * t;
    if (p.y_bf16)
      reinterpret_cast<__bf16 *>(p.y)[row] = (__bf16)s;
    else
      reinterpret_cast<float *>(p.y)[row] = s;
  }
}

}  // namespace

bool gemv_xs_supported(int64_t n_out, int64_t k_in, int n_cu) {
  if (k_in < kXsMinK || k_in > (int64_t)kXsMaxWaves * 2048 || k_in % 32 != 0) return false;
  const int64_t grid = std::min<int64_t>(n_cu, n_out);
  return grid >= 1 && (n_out + grid - 1) / grid <= kXsMaxRows;
}

int64_t gemv_xs_grid(int64_t n_out, int n_cu) { return std::min<int64_t>(n_cu, n_out); }

int gemv_xs_waves(int64_t k_in) { return (int)((k_in / 32 + 63) / 64); }

int gemv_xs_depth() { return kXsDepth; }

hipError_t launch_gemv_xs(const GemvXsParams &p, int64_t grid, int sb_bf16, hipStream_t stream) {
  if (p.waves != gemv_xs_waves((int64_t)p.ncx * 32) || p.waves < 1 || p.waves > kXsMaxWaves ||
      grid < 1 || grid > p.n_out || ((int64_t)p.n_out + grid - 1) / grid > kXsMaxRows)
    return hipErrorInvalidValue;
  auto kern = sb_bf16 ? qgemv_xs_kernel<1, kXsDepth> : qgemv_xs_kernel<0, kXsDepth>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(p.waves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace qint4
