// qgemv.hip -- T=1 int4 group-affine GEMV family for gfx950 (CDNA4).
//
// One kernel template covers the single GEMV, the multi-projection GEMV that
// shares one input (q/k/v in one launch), the gate/up pair with a SwiGLU
// epilogue (dense FFN, and the MoE gate/up phase with device-side expert ids),
// and the MoE down projection with the weighted 8-way scalar-FMA combine and
// residual add.
//
// Sources (by page title and passage):
//   [FFAI #14] thewafflehaus/FFAI pull 14, "feat(everything-bagel): clean
//              migration of PR #9 + #10 onto updated dev": int4 GEMV wrappers
//              (weight, scales, biases, in_dim, group_size); batched QKV and
//              4-way qgemv (one launch, input read once); expert-indexed GEMV
//              (expert id read on the device); chain8 down+SwiGLU+accumulate
//              (per-thread accumulator with the slot scalar baked in, reduced
//              across threads at the end); scalarFMAChain8.
//   [FFAI #9]  thewafflehaus/FFAI pull 9, "Everything Bagel": fused swiglu.
//
// Work decomposition (gfx950 specific, not from the pages):
//   * A row is split into 32-code chunks (16 bytes of codes = one 128-bit
//     load, half of a 64-wide group).  A workgroup of W waves owns a block of
//     rows; wave w owns a contiguous chunk range of every row of the block
//     (or, for the MoE down projection, the whole row of expert slot w), and
//     inside a wave LPR lanes cooperate on one row: lane j takes chunks
//     j, j+LPR, ...  Consecutive lanes therefore read consecutive 16 B of a
//     row, and each lane keeps RT rows in flight.
//   * The activation is staged once per workgroup in LDS, permuted so that a
//     lane's 128-bit LDS reads line up with the nibble order of its code
//     words, together with the sum of every 32-element chunk.
//   * bf16 activations: a nibble pair (q_i, q_{i+4}) of a word becomes the
//     bf16 pair (128 + q_i, 128 + q_{i+4}) with one AND-OR (bf16 0x4300 is
//     128.0 and its mantissa step is 1), and v_dot2_f32_bf16 multiplies it
//     with the matching activation pair.  The 128 * sum(x) excess is removed
//     per chunk, and the group affine map is applied per chunk:
//       sum_k (s q_k + b) x_k = s * (sum_k (128+q_k) x_k - 128 sum x) + b sum x.
//   * float32 activations: the low and high nibbles of a word are split into
//     bytes and converted with v_cvt_f32_ubyte{0..3}, then FMA'd in float32.
//   * Row sums are reduced across the LPR lanes with DPP (quad_perm,
//     row_half_mirror, row_mirror) and the gfx950 permlane16/32 swaps, then
//     across waves through LDS in a fixed order (deterministic results).

#include "kernels.h"

namespace qint4 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int SBT>
__device__ __forceinline__ float load_sb(const void *base, int64_t idx) {
  if constexpr (SBT == 1)
    return __uint_as_float((uint32_t)(reinterpret_cast<const uint16_t *>(base)[idx]) << 16);
  else
    return reinterpret_cast<const float *>(base)[idx];
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum across lanes that differ only in bit 4 (rows of 16 swapped in pairs).
__device__ __forceinline__ float swap16_sum(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

// Sum across the two 32-lane halves of the wave.
__device__ __forceinline__ float swap32_sum(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

// Sum over aligned segments of 2^l2 lanes; every lane of a segment gets the
// segment sum.  Must run with the whole wave active.
__device__ __forceinline__ float seg_sum(float v, int l2) {
  if (l2 >= 1) v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  if (l2 >= 2) v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if (l2 >= 3) v += dpp_mov<0x141>(v);  // row_half_mirror: other quad of 8
  if (l2 >= 4) v += dpp_mov<0x140>(v);  // row_mirror: other half of 16
  if (l2 >= 5) v = swap16_sum(v);
  if (l2 >= 6) v = swap32_sum(v);
  return v;
}

// sum over one 32-code chunk of (128 + q_k) * x_k, starting from acc.
// xp: the chunk's 16 bf16 pairs as 4 x uint4 (pair i of word jj is
// (x[8jj+i], x[8jj+i+4])).
__device__ __forceinline__ float dot_chunk_bf16(const uint4 q, const uint4 *xv, uint32_t magic,
                                                float acc) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const uint32_t xs[4] = {xv[jj].x, xv[jj].y, xv[jj].z, xv[jj].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t pq = ((w[jj] >> (4 * i)) & 0x000F000Fu) | magic;
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pq),
                                            __builtin_bit_cast(bf16x2_t, xs[i]), acc, false);
    }
  }
  return acc;
}

// sum over one 32-code chunk of q_k * x_k in float32.  xv: 8 x float4, word jj
// uses xv[2jj] = (x0, x2, x4, x6) and xv[2jj+1] = (x1, x3, x5, x7).
__device__ __forceinline__ float dot_chunk_f32(const uint4 q, const float4 *xv, float acc) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    uint32_t lo = w[jj] & 0x0F0F0F0Fu;
    uint32_t hi = (w[jj] >> 4) & 0x0F0F0F0Fu;
    // keep the byte split: lets the compiler use v_cvt_f32_ubyte{0..3}
    asm("" : "+v"(lo), "+v"(hi));
    const float4 a = xv[2 * jj], b = xv[2 * jj + 1];
    acc = fmaf((float)(lo & 0xFFu), a.x, acc);
    acc = fmaf((float)((lo >> 8) & 0xFFu), a.y, acc);
    acc = fmaf((float)((lo >> 16) & 0xFFu), a.z, acc);
    acc = fmaf((float)(lo >> 24), a.w, acc);
    acc = fmaf((float)(hi & 0xFFu), b.x, acc);
    acc = fmaf((float)((hi >> 8) & 0xFFu), b.y, acc);
    acc = fmaf((float)((hi >> 16) & 0xFFu), b.z, acc);
    acc = fmaf((float)(hi >> 24), b.w, acc);
  }
  return acc;
}

// Stage the activation (n_chunks * 32 elements) into LDS.  Layout is
// plane-major so that lanes reading consecutive chunks hit consecutive 16 B:
//   bf16: plane jj (0..3) of chunk c at uint4 index jj * n_chunks + c
//   f32 : plane pl (0..7) of chunk c at float4 index pl * n_chunks + c
// xsum[c] = sum of the chunk's 32 elements (float32, fixed order).
template <int XM>
__device__ __forceinline__ void stage_x(const void *__restrict__ x, int n_chunks,
                                        unsigned char *xbuf, float *xsum) {
  const int nocts = n_chunks * 4;  // 8-element groups; a multiple of 4
  for (int o = threadIdx.x; o < nocts; o += blockDim.x) {
    const int c = o >> 2, jj = o & 3;
    float s;
    if constexpr (XM == XM_BF16) {
      const uint4 v = reinterpret_cast<const uint4 *>(x)[o];
      uint4 pr;
      pr.x = (v.x & 0xFFFFu) | (v.z << 16);
      pr.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
      pr.z = (v.y & 0xFFFFu) | (v.w << 16);
      pr.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
      reinterpret_cast<uint4 *>(xbuf)[jj * n_chunks + c] = pr;
      s = ((bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y))) +
          ((bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w)));
    } else {
      const float4 a = reinterpret_cast<const float4 *>(x)[2 * o];
      const float4 b = reinterpret_cast<const float4 *>(x)[2 * o + 1];
      reinterpret_cast<float4 *>(xbuf)[(2 * jj) * n_chunks + c] = make_float4(a.x, a.z, b.x, b.z);
      reinterpret_cast<float4 *>(xbuf)[(2 * jj + 1) * n_chunks + c] = make_float4(a.y, a.w, b.y, b.w);
      s = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
    }
    // the four octets of a chunk sit in one quad of lanes
    s += dpp_mov<0xB1>(s);
    s += dpp_mov<0x4E>(s);
    if (jj == 0) xsum[c] = s;
  }
}

__device__ __forceinline__ void store_out(void *y, int64_t i, float v, int bf16) {
  if (bf16)
    reinterpret_cast<__bf16 *>(y)[i] = (__bf16)v;
  else
    reinterpret_cast<float *>(y)[i] = v;
}

__device__ __forceinline__ float load_act(const void *a, int64_t i, int bf16) {
  if (bf16) return __uint_as_float((uint32_t)(reinterpret_cast<const uint16_t *>(a)[i]) << 16);
  return reinterpret_cast<const float *>(a)[i];
}

template <int W, int RT, int XM, int SBT, int EPI>
__global__ void __launch_bounds__(W * 64) qgemv_kernel(const GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int NS = (EPI == EPI_SWIGLU) ? 2 : 1;  // code streams per row
  constexpr int XB = (XM == XM_BF16) ? 64 : 128;   // staged bytes per chunk
  constexpr int SBB = (SBT == 1) ? 2 : 4;          // bytes per scale/bias

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l2 = p.log2_lpr;
  const int lpr = 1 << l2;
  const int j = lane & (lpr - 1);
  const int sg = lane >> l2;
  const int rpi = 64 >> l2;   // rows per wave instruction
  const int rpb = RT * rpi;   // rows per block
  const int nit = p.chunks_per_wave >> l2;
  const int ncx = p.n_chunks_x;

  float *xsum = reinterpret_cast<float *>(smem);
  unsigned char *xbuf = smem + ((ncx * 4 + 15) & ~15);
  float *red = reinterpret_cast<float *>(xbuf + (size_t)ncx * XB);

  stage_x<XM>(p.x, ncx, xbuf, xsum);
  __syncthreads();

  const int64_t kw = (int64_t)p.chunks_per_row * 4;                  // u32 words per row
  const int64_t gpr = ((int64_t)p.chunks_per_row * 32) >> p.log2_group;  // groups per row
  uint32_t magic = 0x43004300u;
  asm volatile("" : "+v"(magic));  // keep in a VGPR so AND-OR stays one VOP3

  for (int64_t blk = blockIdx.x; blk < p.n_blocks; blk += gridDim.x) {
    // ---- what this block computes (wave-uniform) ----
    const uint32_t *codes[NS];
    const unsigned char *scl[NS];
    const unsigned char *bia[NS];
    int64_t n_rows, row0;
    void *yout = nullptr;
    bool live = true;
    int c0 = wave * p.chunks_per_wave;  // first chunk of this wave inside a row
    int xc0 = c0;                       // matching staged chunk
    if constexpr (EPI == EPI_STORE) {
      int m = 0;
      for (int i = 1; i < p.n_mats; ++i)
        if (blk >= p.m[i].block0) m = i;
      codes[0] = p.m[m].codes;
      scl[0] = reinterpret_cast<const unsigned char *>(p.m[m].scales);
      bia[0] = reinterpret_cast<const unsigned char *>(p.m[m].biases);
      n_rows = p.m[m].n_out;
      row0 = (blk - p.m[m].block0) * rpb;
      yout = p.m[m].y;
    } else if constexpr (EPI == EPI_SWIGLU) {
      const int64_t slot = blk / p.blocks_per_slot;
      const int64_t lb = blk - slot * p.blocks_per_slot;
      const uint32_t e = p.ids ? p.ids[slot] : 0u;
      live = e < (uint32_t)p.n_experts;
      const int64_t eo = live ? (int64_t)e : 0;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        codes[s] = p.m[s].codes + eo * p.expert_code_stride;
        scl[s] = reinterpret_cast<const unsigned char *>(p.m[s].scales) + eo * p.expert_sb_stride * SBB;
        bia[s] = reinterpret_cast<const unsigned char *>(p.m[s].biases) + eo * p.expert_sb_stride * SBB;
      }
      n_rows = p.m[0].n_out;
      row0 = lb * rpb;
      yout = reinterpret_cast<unsigned char *>(p.m[0].y) + slot * n_rows * (p.y_bf16 ? 2 : 4);
    } else {  // EPI_MOE_DOWN: wave w handles expert slot w over the whole row
      const int slot = wave;
      const uint32_t e = (slot < p.top_k) ? p.ids[slot] : 0xFFFFFFFFu;
      live = e < (uint32_t)p.n_experts;
      const int64_t eo = live ? (int64_t)e : 0;
      codes[0] = p.m[0].codes + eo * p.expert_code_stride;
      scl[0] = reinterpret_cast<const unsigned char *>(p.m[0].scales) + eo * p.expert_sb_stride * SBB;
      bia[0] = reinterpret_cast<const unsigned char *>(p.m[0].biases) + eo * p.expert_sb_stride * SBB;
      n_rows = p.m[0].n_out;
      row0 = blk * rpb;
      yout = p.m[0].y;
      c0 = 0;
      xc0 = slot * p.chunks_per_row;
    }

    // ---- this lane's rows (clamped for loads; stores are predicated) ----
    int64_t rowc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int64_t row = row0 + r * rpi + sg;
      rowc[r] = row < n_rows ? row : n_rows - 1;
    }

    float acc[NS][RT];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[s][r] = 0.f;

    if (live) {
#pragma unroll 2
      for (int it = 0; it < nit; ++it) {
        const int c = c0 + j + (it << l2);
        const int xc = xc0 + j + (it << l2);
        const int64_t g = ((int64_t)c * 32) >> p.log2_group;
        const float xs = xsum[xc];
        uint4 q[NS][RT];
        float sv[NS][RT], bv[NS][RT];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int r = 0; r < RT; ++r) {
            q[s][r] = *reinterpret_cast<const uint4 *>(codes[s] + rowc[r] * kw + (int64_t)c * 4);
            sv[s][r] = load_sb<SBT>(scl[s], rowc[r] * gpr + g);
            bv[s][r] = load_sb<SBT>(bia[s], rowc[r] * gpr + g);
          }
        if constexpr (XM == XM_BF16) {
          uint4 xv[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) xv[jj] = reinterpret_cast<const uint4 *>(xbuf)[jj * ncx + xc];
          const float d0 = -128.f * xs;
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int r = 0; r < RT; ++r) {
              const float d = dot_chunk_bf16(q[s][r], xv, magic, d0);  // sum q x
              acc[s][r] = fmaf(sv[s][r], d, fmaf(bv[s][r], xs, acc[s][r]));
            }
        } else {
          float4 xv[8];
#pragma unroll
          for (int pl = 0; pl < 8; ++pl) xv[pl] = reinterpret_cast<const float4 *>(xbuf)[pl * ncx + xc];
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int r = 0; r < RT; ++r) {
              const float d = dot_chunk_f32(q[s][r], xv, 0.f);
              acc[s][r] = fmaf(sv[s][r], d, fmaf(bv[s][r], xs, acc[s][r]));
            }
        }
      }
    }

    // ---- reduce: lanes of a row segment, then waves through LDS ----
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[s][r] = seg_sum(acc[s][r], l2);
    if (j == 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int s = 0; s < NS; ++s) red[((wave * rpb) + r * rpi + sg) * NS + s] = acc[s][r];
    }
    __syncthreads();

    for (int rr = tid; rr < rpb; rr += W * 64) {
      const int64_t row = row0 + rr;
      if (row >= n_rows) continue;
      if constexpr (EPI == EPI_STORE) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) v += red[w * rpb + rr];
        store_out(yout, row, v, p.y_bf16);
      } else if constexpr (EPI == EPI_SWIGLU) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
          g += red[(w * rpb + rr) * 2];
          u += red[(w * rpb + rr) * 2 + 1];
        }
        const float h = live ? (g / (1.f + __expf(-g))) * u : 0.f;
        store_out(yout, row, h, p.y_bf16);
      } else {
        // out = residual + sum_k wts[k] * d_k, one scalar FMA per kept slot
        float v = p.residual ? load_act(p.residual, row, p.y_bf16) : 0.f;
        for (int k = 0; k < p.top_k; ++k) {
          if (p.ids[k] < (uint32_t)p.n_experts) v = fmaf(p.wts[k], red[k * rpb + rr], v);
        }
        store_out(yout, row, v, p.y_bf16);
      }
    }
    __syncthreads();  // red is reused by the next block
  }
}

template <int W, int RT, int XM, int SBT, int EPI>
hipError_t launch_one(const GemvParams &p, const GemvPlan &plan, hipStream_t stream) {
  auto kern = qgemv_kernel<W, RT, XM, SBT, EPI>;
  // Opt in to more than 64 KB of dynamic LDS once per process and kernel
  // (a benign race: concurrent first calls set the same value).
  static bool big_lds = false;
  if (plan.lds_bytes > 64 * 1024 && !big_lds) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e != hipSuccess) return e;
    big_lds = true;
  }
  const int64_t grid = plan.n_blocks < (int64_t)1 << 30 ? plan.n_blocks : (int64_t)1 << 30;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(W * 64), plan.lds_bytes, stream, p);
  return hipGetLastError();
}

template <int W, int RT, int EPI>
hipError_t launch_xs(const GemvParams &p, const GemvPlan &plan, int xmode, int sb_bf16,
                     hipStream_t s) {
  if (xmode == XM_BF16) {
    if (sb_bf16) return launch_one<W, RT, XM_BF16, 1, EPI>(p, plan, s);
    return launch_one<W, RT, XM_BF16, 0, EPI>(p, plan, s);
  }
  if (sb_bf16) return launch_one<W, RT, XM_F32, 1, EPI>(p, plan, s);
  return launch_one<W, RT, XM_F32, 0, EPI>(p, plan, s);
}

template <int W, int EPI>
hipError_t launch_rt(const GemvParams &p, const GemvPlan &plan, int xmode, int sb_bf16,
                     hipStream_t s) {
  switch (plan.rt) {
    case 1: return launch_xs<W, 1, EPI>(p, plan, xmode, sb_bf16, s);
    case 2: return launch_xs<W, 2, EPI>(p, plan, xmode, sb_bf16, s);
    default: break;
  }
  if constexpr (EPI == EPI_STORE) {
    if (plan.rt == 4) return launch_xs<W, 4, EPI>(p, plan, xmode, sb_bf16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t gemv_lds_bytes(int xmode, int n_chunks_x, int waves, int rt, int log2_lpr, int epi) {
  const size_t ns = (epi == EPI_SWIGLU) ? 2 : 1;
  const size_t xb = (xmode == XM_BF16) ? 64 : 128;
  const size_t rpb = (size_t)rt * (64u >> log2_lpr);
  return (((size_t)n_chunks_x * 4 + 15) & ~(size_t)15) + (size_t)n_chunks_x * xb +
         (size_t)waves * rpb * ns * 4;
}

hipError_t launch_gemv(const GemvParams &p, const GemvPlan &plan, int xmode, int sb_bf16, int epi,
                       hipStream_t stream) {
  switch (epi) {
    case EPI_STORE:
      if (plan.waves == 4) return launch_rt<4, EPI_STORE>(p, plan, xmode, sb_bf16, stream);
      if (plan.waves == 1) return launch_rt<1, EPI_STORE>(p, plan, xmode, sb_bf16, stream);
      break;
    case EPI_SWIGLU:
      if (plan.waves == 4) return launch_rt<4, EPI_SWIGLU>(p, plan, xmode, sb_bf16, stream);
      if (plan.waves == 1) return launch_rt<1, EPI_SWIGLU>(p, plan, xmode, sb_bf16, stream);
      break;
    case EPI_MOE_DOWN:
      if (plan.waves == 8 && xmode == XM_F32)
        return launch_rt<8, EPI_MOE_DOWN>(p, plan, xmode, sb_bf16, stream);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace qint4
