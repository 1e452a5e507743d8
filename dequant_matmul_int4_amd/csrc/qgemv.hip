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
//     load, half of a 64-wide group).  LPR lanes of a wave cooperate on one
//     row (lane j takes chunks j, j+LPR, ...), so consecutive lanes read
//     consecutive 16 B of a row; a wave task is RT * 64/LPR whole rows.
//   * Waves are persistent and independent: wave w takes tasks w, w + #waves,
//     ...  A register ring keeps the next D chunk steps (D * RT loads of
//     16 B per lane, 8 in total) in flight across task boundaries, and the
//     first D steps are issued before the activation is staged.
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
//   * MoE down projection: the kept experts' rows are one virtual row of
//     top_k * inter codes; each lane looks up the expert slot of its chunk,
//     reads that expert's codes, and folds the slot weight into its
//     accumulator (the scalar FMA of that slot), before the lanes are reduced
//     and the residual added.
//   * Row sums are reduced across the LPR lanes with DPP (quad_perm,
//     row_half_mirror, row_mirror) and the gfx950 permlane16/32 swaps.

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

// Workgroup barrier that orders LDS only.  __syncthreads() also fences
// global memory, which on gfx9 means draining every outstanding vector memory
// operation (vmcnt counts loads and stores alike) -- including prefetched
// code loads that have nothing to do with the LDS hand-off.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Touch every 64-byte line of the kernel-argument block with back-to-back
// scalar loads and wait once.  Argument fields are otherwise read lazily, in
// several dependent rounds, and each round misses all caches when the weight
// stream has evicted the (tiny) argument block -- an HBM round trip apiece.
template <int BYTES>
__device__ __forceinline__ void warm_kernargs() {
  static_assert(BYTES <= 512, "kernel arguments span more than 8 lines");
  typedef const uint32_t __attribute__((address_space(4))) *kptr;
  const kptr ka = (kptr)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (i * 64 < BYTES) ? ka[i * 16] : 0u;
  // one statement consuming every value: all loads issue, then a single wait
  asm volatile("" ::"s"(v[0]), "s"(v[1]), "s"(v[2]), "s"(v[3]), "s"(v[4]), "s"(v[5]), "s"(v[6]),
               "s"(v[7]));
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
//
// Thread t handles the 8-element octets t, t + nthreads, ...  Staging is split
// in two: stage_issue() starts the global loads of the first XQ octets into
// registers, stage_commit() permutes them into LDS.  Code loads issued in
// between overlap the activation's round trip: vmcnt drains in issue order,
// so the commit waits only for the older activation loads.
constexpr int XQ = 8;

template <int XM>
struct XRegs {
  uint4 v[XQ][XM == XM_BF16 ? 1 : 2];
};

template <int XM>
__device__ __forceinline__ void stage_load(const void *x, int o, uint4 *v) {
  if constexpr (XM == XM_BF16) {
    v[0] = reinterpret_cast<const uint4 *>(x)[o];
  } else {
    v[0] = reinterpret_cast<const uint4 *>(x)[2 * o];
    v[1] = reinterpret_cast<const uint4 *>(x)[2 * o + 1];
  }
}

// Writes octet o (already in v) to the LDS planes and its chunk sum.  Must be
// called by whole quads of lanes (the four octets of a chunk are in one quad).
template <int XM>
__device__ __forceinline__ void stage_store(int o, const uint4 *v, int n_chunks,
                                            unsigned char *xbuf, float *xsum) {
  const int c = o >> 2, jj = o & 3;
  float s;
  if constexpr (XM == XM_BF16) {
    const uint4 w = v[0];
    uint4 pr;
    pr.x = (w.x & 0xFFFFu) | (w.z << 16);
    pr.y = (w.x >> 16) | (w.z & 0xFFFF0000u);
    pr.z = (w.y & 0xFFFFu) | (w.w << 16);
    pr.w = (w.y >> 16) | (w.w & 0xFFFF0000u);
    reinterpret_cast<uint4 *>(xbuf)[jj * n_chunks + c] = pr;
    s = ((bf16_lo(w.x) + bf16_hi(w.x)) + (bf16_lo(w.y) + bf16_hi(w.y))) +
        ((bf16_lo(w.z) + bf16_hi(w.z)) + (bf16_lo(w.w) + bf16_hi(w.w)));
  } else {
    const float4 a = __builtin_bit_cast(float4, v[0]);
    const float4 b = __builtin_bit_cast(float4, v[1]);
    reinterpret_cast<float4 *>(xbuf)[(2 * jj) * n_chunks + c] = make_float4(a.x, a.z, b.x, b.z);
    reinterpret_cast<float4 *>(xbuf)[(2 * jj + 1) * n_chunks + c] = make_float4(a.y, a.w, b.y, b.w);
    s = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
  }
  s += dpp_mov<0xB1>(s);
  s += dpp_mov<0x4E>(s);
  if (jj == 0) xsum[c] = s;
}

template <int XM>
__device__ __forceinline__ void stage_issue(const void *__restrict__ x, int n_chunks, XRegs<XM> &r) {
  const int nocts = n_chunks * 4;
#pragma unroll
  for (int i = 0; i < XQ; ++i) {
    // unconditional (clamped) loads: a load inside a branch makes the
    // compiler copy its result at the join, which waits for it right away
    const int o = min((int)(threadIdx.x + i * blockDim.x), nocts - 1);
    stage_load<XM>(x, o, r.v[i]);
  }
}

template <int XM>
__device__ __forceinline__ void stage_commit(const void *__restrict__ x, int n_chunks,
                                             const XRegs<XM> &r, unsigned char *xbuf, float *xsum) {
  const int nocts = n_chunks * 4;
#pragma unroll
  for (int i = 0; i < XQ; ++i) {
    const int o = threadIdx.x + i * blockDim.x;
    if (o < nocts) stage_store<XM>(o, r.v[i], n_chunks, xbuf, xsum);
  }
  // octets beyond the first XQ per thread (very long rows): load and store
  for (int o = threadIdx.x + XQ * blockDim.x; o < nocts; o += blockDim.x) {
    uint4 v[XM == XM_BF16 ? 1 : 2];
    stage_load<XM>(x, o, v);
    stage_store<XM>(o, v, n_chunks, xbuf, xsum);
  }
}

// The MoE residual row, staged as float32 in LDS (loads issued with the
// activation's, before the first code loads; read back at task ends).
constexpr int RQ = 4;

// nvec: 16-byte vectors readable at res (loads are clamped to it)
__device__ __forceinline__ void residual_issue(const void *res, int nvec, uint4 (&v)[RQ]) {
#pragma unroll
  for (int i = 0; i < RQ; ++i) {
    const int o = min((int)(threadIdx.x + i * blockDim.x), nvec - 1);
    v[i] = reinterpret_cast<const uint4 *>(res)[o];
  }
}

__device__ __forceinline__ void residual_store(int o, const uint4 w, int bf16, float *dst) {
  if (bf16) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      dst[8 * o + 2 * k] = bf16_lo(u[k]);
      dst[8 * o + 2 * k + 1] = bf16_hi(u[k]);
    }
  } else {
    reinterpret_cast<float4 *>(dst)[o] = __builtin_bit_cast(float4, w);
  }
}

__device__ __forceinline__ void residual_commit(const void *res, int n, int bf16, const uint4 (&v)[RQ],
                                                float *dst) {
  const int nvec = bf16 ? n / 8 : n / 4;
#pragma unroll
  for (int i = 0; i < RQ; ++i) {
    const int o = threadIdx.x + i * blockDim.x;
    if (o < nvec) residual_store(o, v[i], bf16, dst);
  }
  for (int o = threadIdx.x + RQ * blockDim.x; o < nvec; o += blockDim.x)
    residual_store(o, reinterpret_cast<const uint4 *>(res)[o], bf16, dst);
}

__device__ __forceinline__ void store_out(void *y, int64_t i, float v, int bf16) {
  if (bf16)
    reinterpret_cast<__bf16 *>(y)[i] = (__bf16)v;
  else
    reinterpret_cast<float *>(y)[i] = v;
}


// Registers holding one prefetched step (one 32-code chunk of each of the
// task's rows, with the matching scale and bias).
template <int RT, int NS>
struct StepBuf {
  uint4 q[NS][RT];
  uint32_t s[NS][RT];  // raw scale bits (bf16 zero-extended, or float32)
  uint32_t b[NS][RT];  // raw bias bits; decoded when consumed, so that no
                       // instruction waits on the load where it is issued
  float w;  // EPI_MOE_DOWN: weight of the expert slot this lane's chunk belongs to
};

// Raw buffer resources: a load whose byte offset is >= the resource's
// num_records returns zero without touching memory.  Steps past a wave's end
// and rows past a matrix use such an offset, so every load is unconditional
// (no branch, hence no register copy that would wait on it).
constexpr uint32_t kOutOfRange = 0x80000000u;  // resources are < 2 GiB

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

template <int SBT>
__device__ __forceinline__ uint32_t buf_load_sb(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (SBT == 1)
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  else
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

template <int SBT>
__device__ __forceinline__ float sb_value(uint32_t bits) {
  return __uint_as_float(SBT == 1 ? (bits << 16) : bits);
}

// Persistent GEMV kernel.  Wave gw owns the contiguous task range
// [gw * tpw, (gw + 1) * tpw); a task is rpt = RT * 64/LPR rows, each row
// covered by LPR lanes.  The loads of the next D steps are always in flight
// (a register ring of D * RT * NS 128-bit loads per lane), across task
// boundaries, so a wave streams its rows continuously.  The first D loads are
// issued before the activation is staged, overlapping that L2 traffic with
// the first HBM round trip.  Task bookkeeping is incremental 32-bit scalar
// arithmetic; matrix descriptors and buffer resources are refreshed only when
// a wave crosses into the next matrix (or expert slot).
template <int RT, int XM, int SBT, int EPI>
__global__ void __launch_bounds__(512) qgemv_kernel(const GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  warm_kernargs<sizeof(GemvParams)>();
  constexpr int NS = (EPI == EPI_SWIGLU) ? 2 : 1;  // code streams per row (gate, up)
  constexpr int D = 8 / (RT * NS);                 // steps in flight
  constexpr int XB = (XM == XM_BF16) ? 64 : 128;   // staged bytes per chunk
  constexpr int SBB = (SBT == 1) ? 2 : 4;          // bytes per scale/bias

  const int lane = threadIdx.x & 63;
  const int W = blockDim.x >> 6;
  // wave index made provably uniform: all task bookkeeping stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_waves = gridDim.x * W;
  const int gw = blockIdx.x * W + wave;
  const int l2 = p.log2_lpr;
  const int j = lane & ((1 << l2) - 1);
  const int sg = lane >> l2;
  const int rpi = 64 >> l2;  // rows per wave instruction
  const int rpt = RT * rpi;  // rows per task
  const int spt = p.steps_per_task;
  const int ncx = p.n_chunks_x;
  const uint32_t kwb = (uint32_t)p.chunks_per_row * 16;                   // code bytes per row
  const uint32_t gpr = ((uint32_t)p.chunks_per_row * 32) >> p.log2_group;  // groups per row

  const int tpw = (p.n_tasks + n_waves - 1) / n_waves;
  const int t_begin = min(gw * tpw, p.n_tasks);
  const int t_end = min(t_begin + tpw, p.n_tasks);
  const int S = (t_end - t_begin) * spt;  // steps of this wave

  float *xsum = reinterpret_cast<float *>(smem);
  unsigned char *xbuf = smem + ((ncx * 4 + 15) & ~15);
  float *res_lds = reinterpret_cast<float *>(xbuf + (size_t)ncx * XB);  // EPI_MOE_DOWN

  // expert ids and slot weights: lane k holds slot k's values
  uint32_t v_ids = 0;
  float v_wts = 0.f;
  if constexpr (EPI != EPI_STORE) {
    if (p.ids && lane < p.top_k) v_ids = p.ids[lane];
    if constexpr (EPI == EPI_MOE_DOWN) {
      if (lane < p.top_k) v_wts = p.wts[lane];
    }
  }
  uint32_t magic = 0x43004300u;
  asm volatile("" : "+v"(magic));  // keep in a VGPR so AND-OR stays one VOP3

  // ---- cursors over (task, step) ----
  struct Cur {
    int task, it;
    int m, m_end;  // matrix (EPI_STORE) or expert slot (EPI_SWIGLU); first task past it
    int row0;      // first row of the task inside its matrix
    int n_rows;
    bool live;     // EPI_SWIGLU: the slot's expert id is valid
    const uint32_t *codes[NS];
    const unsigned char *scl[NS];
    const unsigned char *bia[NS];
    void *y;
  };
  auto enter = [&](Cur &c, int m) {  // geometry of matrix / slot m
    c.m = m;
    c.live = true;
    if constexpr (EPI == EPI_STORE) {
      c.codes[0] = p.m[m].codes;
      c.scl[0] = reinterpret_cast<const unsigned char *>(p.m[m].scales);
      c.bia[0] = reinterpret_cast<const unsigned char *>(p.m[m].biases);
      c.n_rows = (int)p.m[m].n_out;
      c.y = p.m[m].y;
      c.m_end = (m + 1 < p.n_mats) ? p.task0[m + 1] : p.n_tasks;
      c.row0 = (c.task - p.task0[m]) * rpt;
    } else if constexpr (EPI == EPI_SWIGLU) {
      const uint32_t e = (uint32_t)__builtin_amdgcn_readlane((int)v_ids, m);
      c.live = e < (uint32_t)p.n_experts;
      const int64_t eo = c.live ? (int64_t)e : 0;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        c.codes[s] = p.m[s].codes + eo * p.expert_code_stride;
        c.scl[s] = reinterpret_cast<const unsigned char *>(p.m[s].scales) + eo * p.expert_sb_stride * SBB;
        c.bia[s] = reinterpret_cast<const unsigned char *>(p.m[s].biases) + eo * p.expert_sb_stride * SBB;
      }
      c.n_rows = (int)p.m[0].n_out;
      c.y = reinterpret_cast<unsigned char *>(p.m[0].y) + (int64_t)m * c.n_rows * (p.y_bf16 ? 2 : 4);
      c.m_end = (m + 1) * p.tasks_per_slot;
      c.row0 = (c.task - m * p.tasks_per_slot) * rpt;
    } else {
      c.codes[0] = p.m[0].codes;
      c.scl[0] = reinterpret_cast<const unsigned char *>(p.m[0].scales);
      c.bia[0] = reinterpret_cast<const unsigned char *>(p.m[0].biases);
      c.n_rows = (int)p.m[0].n_out;
      c.y = p.m[0].y;
      c.m_end = p.n_tasks;
      c.row0 = c.task * rpt;
    }
  };
  auto start = [&](Cur &c) {
    c.task = t_begin;
    c.it = 0;
    int m = 0;
    if constexpr (EPI == EPI_STORE) {
      for (int i = 1; i < p.n_mats; ++i)
        if (t_begin >= p.task0[i]) m = i;
    } else if constexpr (EPI == EPI_SWIGLU) {
      m = min(t_begin / p.tasks_per_slot, p.top_k - 1);
    }
    enter(c, m);
  };
  // next step; returns true when the cursor moved into another matrix / slot
  auto advance = [&](Cur &c) {
    if (++c.it < spt) return false;
    c.it = 0;
    ++c.task;
    c.row0 += rpt;
    if (c.task >= c.m_end && c.task < t_end) {
      enter(c, c.m + 1);
      return true;
    }
    return false;
  };

  // ---- load stream ----
  Cur lc;
  start(lc);
  __amdgpu_buffer_rsrc_t rc[NS], rs[NS], rb[NS];
  auto set_rsrc = [&]() {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t cb = (EPI == EPI_MOE_DOWN) ? (uint32_t)p.code_bytes : (uint32_t)lc.n_rows * kwb;
      const uint32_t sbb = (EPI == EPI_MOE_DOWN) ? (uint32_t)p.sb_bytes : (uint32_t)lc.n_rows * gpr * SBB;
      rc[s] = make_rsrc(lc.codes[s], cb);
      rs[s] = make_rsrc(lc.scl[s], sbb);
      rb[s] = make_rsrc(lc.bia[s], sbb);
    }
  };
  set_rsrc();
  auto load = [&](StepBuf<RT, NS> &bf) {
    const bool ok = lc.task < t_end;  // past the wave's last step: out of range
    int c = j + (lc.it << l2);        // chunk of the (virtual) row
    uint32_t ecode = 0, esb = 0;
    if constexpr (EPI == EPI_MOE_DOWN) {
      // virtual row = the kept experts' rows back to back; this lane's slot
      const int slot = (int)(((float)c + 0.5f) * p.inv_chunks_per_row);
      c -= slot * p.chunks_per_row;
      uint32_t e = (uint32_t)__shfl((int)v_ids, slot);
      float w = __shfl(v_wts, slot);
      if (e >= (uint32_t)p.n_experts) {  // skipped slot: read expert 0, weight 0
        e = 0;
        w = 0.f;
      }
      bf.w = w;
      ecode = e * (uint32_t)(p.expert_code_stride * 4);
      esb = e * (uint32_t)(p.expert_sb_stride * SBB);
    }
    const uint32_t g = ((uint32_t)c * 32) >> p.log2_group;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row = lc.row0 + r * rpi + sg;
      const bool okr = ok && row < lc.n_rows;
      const uint32_t oc = okr ? ecode + (uint32_t)row * kwb + (uint32_t)c * 16 : kOutOfRange;
      const uint32_t os = okr ? esb + ((uint32_t)row * gpr + g) * SBB : kOutOfRange;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        bf.q[s][r] = buf_load_b128(rc[s], oc);
        bf.s[s][r] = buf_load_sb<SBT>(rs[s], os);
        bf.b[s][r] = buf_load_sb<SBT>(rb[s], os);
      }
    }
    if (ok && advance(lc)) set_rsrc();
  };

  XRegs<XM> xr;
  stage_issue<XM>(p.x, ncx, xr);  // activation loads first (L2), ...
  uint4 rr[RQ];
  const bool has_res = (EPI == EPI_MOE_DOWN) && p.residual != nullptr;
  if constexpr (EPI == EPI_MOE_DOWN) {
    // without a residual, harmless clamped loads of the activation's first
    // 16 bytes keep the issue unconditional
    const int nvec = has_res ? (int)(p.y_bf16 ? p.m[0].n_out / 8 : p.m[0].n_out / 4) : 1;
    residual_issue(has_res ? p.residual : p.x, nvec, rr);
  }

  // ... then the first D steps of codes (HBM).
  StepBuf<RT, NS> buf[D];
#pragma unroll
  for (int u = 0; u < D; ++u) load(buf[u]);

  stage_commit<XM>(p.x, ncx, xr, xbuf, xsum);
  if (has_res) residual_commit(p.residual, (int)p.m[0].n_out, p.y_bf16, rr, res_lds);
  lds_barrier();

  // ---- consume stream ----
  float acc[NS][RT];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[s][r] = 0.f;
  Cur cc;
  start(cc);

  auto finish = [&]() {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[s][r] = seg_sum(acc[s][r], l2);
    if (j == 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int row = cc.row0 + r * rpi + sg;
        if (row < cc.n_rows) {
          if constexpr (EPI == EPI_STORE) {
            store_out(cc.y, row, acc[0][r], p.y_bf16);
          } else if constexpr (EPI == EPI_SWIGLU) {
            const float g = acc[0][r], u = acc[1][r];
            const float h = cc.live ? (g / (1.f + __expf(-g))) * u : 0.f;
            store_out(cc.y, row, h, p.y_bf16);
          } else {
            const float res = has_res ? res_lds[row] : 0.f;
            store_out(cc.y, row, res + acc[0][r], p.y_bf16);
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[s][r] = 0.f;
  };

  auto consume = [&](const StepBuf<RT, NS> &bf) {
    const int xc = j + (cc.it << l2);  // staged chunk (virtual row chunk)
    const float xs = xsum[xc];
    if constexpr (XM == XM_BF16) {
      uint4 xv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) xv[jj] = reinterpret_cast<const uint4 *>(xbuf)[jj * ncx + xc];
      const float d0 = -128.f * xs;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const float d = dot_chunk_bf16(bf.q[s][r], xv, magic, d0);  // sum q x
          const float part = fmaf(sb_value<SBT>(bf.s[s][r]), d, sb_value<SBT>(bf.b[s][r]) * xs);
          if constexpr (EPI == EPI_MOE_DOWN)
            acc[s][r] = fmaf(bf.w, part, acc[s][r]);
          else
            acc[s][r] += part;
        }
    } else {
      float4 xv[8];
#pragma unroll
      for (int pl = 0; pl < 8; ++pl) xv[pl] = reinterpret_cast<const float4 *>(xbuf)[pl * ncx + xc];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const float d = dot_chunk_f32(bf.q[s][r], xv, 0.f);
          const float part = fmaf(sb_value<SBT>(bf.s[s][r]), d, sb_value<SBT>(bf.b[s][r]) * xs);
          if constexpr (EPI == EPI_MOE_DOWN)
            acc[s][r] = fmaf(bf.w, part, acc[s][r]);
          else
            acc[s][r] += part;
        }
    }
    if (cc.it == spt - 1) finish();
    advance(cc);
  };

  for (int s0 = 0; s0 < S; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (s0 + u < S) consume(buf[u]);
      load(buf[u]);  // past the wave's last step: out of range, returns zeros
    }
  }
}

template <int RT, int XM, int SBT, int EPI>
const void *kernel_ptr() {
  return reinterpret_cast<const void *>(qgemv_kernel<RT, XM, SBT, EPI>);
}

template <int RT, int XM, int SBT, int EPI>
hipError_t launch_one(const GemvParams &p, const GemvPlan &plan, hipStream_t stream) {
  auto kern = qgemv_kernel<RT, XM, SBT, EPI>;
  // Opt in to more than 64 KB of dynamic LDS once per process and kernel
  // (a benign race: concurrent first calls set the same value).
  static bool big_lds = false;
  if (plan.lds_bytes > 64 * 1024 && !big_lds) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e != hipSuccess) return e;
    big_lds = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)plan.grid), dim3(plan.waves * 64), plan.lds_bytes,
                     stream, p);
  return hipGetLastError();
}

// Kernel selection: (rt, xmode, sb_bf16, epi) -> instantiation.  MoE down
// always stages a float32 activation (the SwiGLU intermediates).
template <int RT, int EPI>
const void *select_ptr(int xmode, int sb_bf16) {
  if (EPI == EPI_MOE_DOWN || xmode == XM_F32)
    return sb_bf16 ? kernel_ptr<RT, XM_F32, 1, EPI>() : kernel_ptr<RT, XM_F32, 0, EPI>();
  return sb_bf16 ? kernel_ptr<RT, XM_BF16, 1, EPI>() : kernel_ptr<RT, XM_BF16, 0, EPI>();
}

template <int RT, int EPI>
hipError_t launch_sel(const GemvParams &p, const GemvPlan &plan, int xmode, int sb_bf16,
                      hipStream_t s) {
  if (EPI == EPI_MOE_DOWN || xmode == XM_F32)
    return sb_bf16 ? launch_one<RT, XM_F32, 1, EPI>(p, plan, s) : launch_one<RT, XM_F32, 0, EPI>(p, plan, s);
  return sb_bf16 ? launch_one<RT, XM_BF16, 1, EPI>(p, plan, s) : launch_one<RT, XM_BF16, 0, EPI>(p, plan, s);
}

}  // namespace

size_t gemv_lds_bytes(int xmode, int n_chunks_x, int64_t residual_rows) {
  const size_t xb = (xmode == XM_BF16) ? 64 : 128;
  return (((size_t)n_chunks_x * 4 + 15) & ~(size_t)15) + (size_t)n_chunks_x * xb +
         (size_t)residual_rows * 4;
}

int gemv_blocks_per_cu(const GemvPlan &plan, int xmode, int sb_bf16, int epi) {
  const void *k = nullptr;
  switch (epi) {
    case EPI_STORE: k = plan.rt == 2 ? select_ptr<2, EPI_STORE>(xmode, sb_bf16) : select_ptr<1, EPI_STORE>(xmode, sb_bf16); break;
    case EPI_SWIGLU: k = plan.rt == 2 ? select_ptr<2, EPI_SWIGLU>(xmode, sb_bf16) : select_ptr<1, EPI_SWIGLU>(xmode, sb_bf16); break;
    case EPI_MOE_DOWN: k = plan.rt == 2 ? select_ptr<2, EPI_MOE_DOWN>(xmode, sb_bf16) : select_ptr<1, EPI_MOE_DOWN>(xmode, sb_bf16); break;
    default: return 0;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, plan.waves * 64, plan.lds_bytes) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

hipError_t launch_gemv(const GemvParams &p, const GemvPlan &plan, int xmode, int sb_bf16, int epi,
                       hipStream_t stream) {
  if (plan.rt != 1 && plan.rt != 2) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE:
      return plan.rt == 2 ? launch_sel<2, EPI_STORE>(p, plan, xmode, sb_bf16, stream)
                          : launch_sel<1, EPI_STORE>(p, plan, xmode, sb_bf16, stream);
    case EPI_SWIGLU:
      return plan.rt == 2 ? launch_sel<2, EPI_SWIGLU>(p, plan, xmode, sb_bf16, stream)
                          : launch_sel<1, EPI_SWIGLU>(p, plan, xmode, sb_bf16, stream);
    case EPI_MOE_DOWN:
      return plan.rt == 2 ? launch_sel<2, EPI_MOE_DOWN>(p, plan, xmode, sb_bf16, stream)
                          : launch_sel<1, EPI_MOE_DOWN>(p, plan, xmode, sb_bf16, stream);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace qint4
