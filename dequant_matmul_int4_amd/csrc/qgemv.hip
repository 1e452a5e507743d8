// qgemv.hip -- T=1 int4 group-affine GEMV family for gfx950 (CDNA4).
//
// One kernel template covers the single GEMV, the multi-projection GEMV that
// shares one input (q/k/v in one launch), the gate/up pair with a SwiGLU
// epilogue (dense FFN, and the MoE gate/up phase with device-side expert ids),
// and the MoE down projection with the weighted scalar-FMA combine of the kept
// experts and the residual add.
//
// Sources (by page title and passage):
//   [FFAI #14] thewafflehaus/FFAI pull 14, "feat(everything-bagel): clean
//              migration of PR #9 + #10 onto updated dev": int4 GEMV wrappers
//              (weight, scales, biases, in_dim, group_size); batched QKV and
//              4-way qgemv (one launch, input read once); expert-indexed GEMV
//              (expert id read on the device); chain8 down+SwiGLU+accumulate
//              (per-thread accumulator with the slot scalar folded in, reduced
//              across threads at the end); scalarFMAChain8.
//   [FFAI #9]  thewafflehaus/FFAI pull 9, "Everything Bagel": fused swiglu.
//   [FFAI #14] also: the RMSNorm-fused qgemv wrappers (the normalised
//              activation goes straight into the dequant GEMV, one launch).
//   [ds4 #844] antirez/ds4 pull 844, "Ornith 1.5 + Qwen 3.8 27B hybrid
//              runtime + DFlash speculative decoding on Metal", commit making
//              both norm kernels use 1 / sqrt(mean + eps) rather than rsqrt.
//
// Work decomposition (gfx950 specific, not from the pages):
//   * A row is split into 32-code chunks (16 bytes of codes = one 128-bit
//     load, inside one group since group_size >= 32).  L lanes of a wave
//     cooperate on one row (lane j takes chunks j, j + L, ...), so consecutive
//     lanes read consecutive 16 bytes; a "step" is one such load per lane and
//     a task is RT * 64/L whole rows.  When L does not divide the chunk count,
//     the last step of a row is partial.
//   * Tasks are dealt round-robin over all waves of a persistent grid (wave w
//     takes tasks w, w + n_waves, ...): at any moment the grid streams one
//     compact region of each matrix, which the memory system serves better
//     than many far-apart streams.  The host picks wave counts that divide
//     the task count where it can, so every wave ends at the same time.
//   * Each wave keeps kSlots 128-bit code loads (plus their scale and bias
//     loads) in flight in a register ring that runs across task boundaries;
//     the first ring fill is issued before the activation is staged.  Few
//     waves per CU with deep rings: vector registers are plentiful at low
//     occupancy, and each wave has fewer prologue instructions to amortise.
//     When no wave of a launch has more than P = 1, 2 or 4 steps, a one-pass
//     instantiation sizes the ring to P and fills it once: the streaming ring
//     would also issue its refills, all out of range at that point, and those
//     instructions compete with the real loads for the memory pipeline.
//   * The activation is staged once per workgroup in LDS, permuted so that a
//     lane's 128-bit LDS reads line up with the nibble order of its code
//     words, together with the sum of every 32-element chunk; it is padded
//     with zero chunks up to whole steps.
//   * bf16 activations: a nibble pair (q_i, q_{i+4}) of a word becomes the
//     bf16 pair (128 + q_i, 128 + q_{i+4}) with one AND-OR (bf16 0x4300 is
//     128.0 and its mantissa step is 1), and v_dot2_f32_bf16 multiplies it
//     with the matching activation pair.  The 128 * sum(x) excess is removed
//     per chunk, and the group affine map is applied per chunk:
//       sum_k (s q_k + b) x_k = s * (sum_k (128+q_k) x_k - 128 sum x) + b sum x.
//   * float32 activations: a word masked with 0x000F000F holds the nibble
//     pair (q_i, q_{i+4}) as the exact f16 subnormals q 2^-24, masked with
//     0x00F000F0 the pair (q_{i+1}, q_{i+5}) as 16 q 2^-24; v_fma_mix_f32
//     multiplies them by activations staged times 2^24 and 2^20, which is
//     fmaf(q, x, t) exactly (activations below 2^104 in magnitude).
//   * MoE down projection: the kept experts' rows are one virtual row of
//     top_k * inter codes; each lane looks up the expert slot of its chunk,
//     reads that expert's codes, and folds the slot weight into its
//     accumulator (the scalar FMA of that slot), before the lanes are reduced
//     and the residual added.
//   * RMSNorm prologue (XM_RMS_*): the staged activation is x * gamma in
//     float32 and every workgroup reduces sum(x^2) over the whole row while
//     staging it; since the norm is one scalar per row,
//       W (x * gamma / rms) = (W (x * gamma)) / rms,
//     the row sums are scaled by 1 / sqrt(sum(x^2) / k_in + eps) at the end.
//   * Row sums are reduced across the L lanes with DPP (quad_perm,
//     row_half_mirror, row_mirror) and the gfx950 permlane16/32 swaps.
//   * Every memory access is a raw buffer load: an offset at or beyond the
//     resource size returns zero without touching memory, which covers rows
//     past a matrix's end, the partial last step and skipped experts without
//     branches.

#include <algorithm>

#include "kernels.h"
#include "topk_wave.h"

namespace qint4 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

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

// Eight 32-bit words from a uniform device address through the scalar cache
// (lgkmcnt, so the wait does not drain outstanding vector loads).  Word k is
// read from base[min(k, n - 1)], so nothing past the n-word array is touched.
__device__ __forceinline__ void scalar_load8(const uint32_t *base, int n, uint32_t (&v)[8]) {
  const uint32_t *a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = base + (k < n ? k : n - 1);
  asm volatile(
      "s_load_dword %0, %8, 0x0\n\t"
      "s_load_dword %1, %9, 0x0\n\t"
      "s_load_dword %2, %10, 0x0\n\t"
      "s_load_dword %3, %11, 0x0\n\t"
      "s_load_dword %4, %12, 0x0\n\t"
      "s_load_dword %5, %13, 0x0\n\t"
      "s_load_dword %6, %14, 0x0\n\t"
      "s_load_dword %7, %15, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      // early-clobber: a result register must not be the address of a later
      // load in this block (the loads complete asynchronously)
      : "=&s"(v[0]), "=&s"(v[1]), "=&s"(v[2]), "=&s"(v[3]), "=&s"(v[4]), "=&s"(v[5]),
        "=&s"(v[6]), "=&s"(v[7])
      : "s"(a[0]), "s"(a[1]), "s"(a[2]), "s"(a[3]), "s"(a[4]), "s"(a[5]), "s"(a[6]), "s"(a[7])
      : "memory");
}

// Two such 8-word reads, va from a and vb from b, with one wait: word k of
// each is read at element min(k, n - 1) (byte offsets in SGPRs).
__device__ __forceinline__ void scalar_load8x2(const uint32_t *a, const uint32_t *b, int n, uint32_t (&va)[8],
                                               uint32_t (&vb)[8]) {
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 4u * (uint32_t)(k < n ? k : n - 1);
  asm volatile(
      "s_load_dword %0, %16, %18\n\t"
      "s_load_dword %1, %16, %19\n\t"
      "s_load_dword %2, %16, %20\n\t"
      "s_load_dword %3, %16, %21\n\t"
      "s_load_dword %4, %16, %22\n\t"
      "s_load_dword %5, %16, %23\n\t"
      "s_load_dword %6, %16, %24\n\t"
      "s_load_dword %7, %16, %25\n\t"
      "s_load_dword %8, %17, %18\n\t"
      "s_load_dword %9, %17, %19\n\t"
      "s_load_dword %10, %17, %20\n\t"
      "s_load_dword %11, %17, %21\n\t"
      "s_load_dword %12, %17, %22\n\t"
      "s_load_dword %13, %17, %23\n\t"
      "s_load_dword %14, %17, %24\n\t"
      "s_load_dword %15, %17, %25\n\t"
      "s_waitcnt lgkmcnt(0)"
      // early-clobber: no result register may alias an address or offset
      // still to be used by a later load of the block
      : "=&s"(va[0]), "=&s"(va[1]), "=&s"(va[2]), "=&s"(va[3]), "=&s"(va[4]), "=&s"(va[5]),
        "=&s"(va[6]), "=&s"(va[7]), "=&s"(vb[0]), "=&s"(vb[1]), "=&s"(vb[2]), "=&s"(vb[3]),
        "=&s"(vb[4]), "=&s"(vb[5]), "=&s"(vb[6]), "=&s"(vb[7])
      : "s"(a), "s"(b), "s"(o[0]), "s"(o[1]), "s"(o[2]), "s"(o[3]), "s"(o[4]), "s"(o[5]), "s"(o[6]),
        "s"(o[7])
      : "memory");
}

// A VGPR whose lane k (k < 8) holds v[k]; other lanes hold 0.
__device__ __forceinline__ uint32_t lanes_from_scalars(const uint32_t (&v)[8]) {
  const int lane = threadIdx.x & 63;
  uint32_t r = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) r = lane == k ? v[k] : r;
  return r;
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

// The 32 codes of a chunk as 16 bf16 pairs (128 + q_i, 128 + q_{i+4}):
// pq[4 jj + i] pairs nibbles i and i+4 of word jj.
// Two words are shifted as one 64-bit value (one v_lshrrev_b64 instead of
// two 32-bit shifts; the compiler splits a 64-bit shift whose halves are
// masked); the high word's nibbles that land in the low word's top bits are
// masked off.
template <int S>
__device__ __forceinline__ uint64_t shr64_nibbles(uint64_t w) {
  uint64_t r;
  asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "n"(4 * S), "v"(w));
  return r;
}

__device__ __forceinline__ void decode_chunk_bf16(const uint4 q, uint32_t magic, uint32_t (&pq)[16]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint64_t w2 = ((uint64_t)w[2 * h + 1] << 32) | w[2 * h];
    const uint64_t sh[4] = {w2, shr64_nibbles<1>(w2), shr64_nibbles<2>(w2), shr64_nibbles<3>(w2)};
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pq[4 * (2 * h + e) + i] = ((uint32_t)(sh[i] >> (32 * e)) & 0x000F000Fu) | magic;
  }
}

// sum over one decoded chunk of (128 + q_k) * x_k, starting from acc.
// xv: the chunk's 16 bf16 pairs as 4 x uint4 (pair i of word jj is
// (x[8jj+i], x[8jj+i+4])).  One accumulator per word: four independent
// dependency chains instead of one.
__device__ __forceinline__ float dot_pq_bf16(const uint32_t (&pq)[16], const uint4 *xv, float acc) {
  float a[4] = {acc, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const uint32_t xs[4] = {xv[jj].x, xv[jj].y, xv[jj].z, xv[jj].w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[jj] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pq[4 * jj + i]),
                                              __builtin_bit_cast(bf16x2_t, xs[i]), a[jj], false);
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// sum over one 32-code chunk of q_k * x_k in float32.  xv: 8 x float4, word jj
// uses xv[2jj] = (x0, x2, x4, x6) * 2^24 and xv[2jj+1] = (x1, x3, x5, x7) *
// 2^20 (the staged planes).  The word masked with 0x000F000F holds codes
// (n, n + 4) as the f16 subnormals q 2^-24, masked with 0x00F000F0 codes
// (n + 1, n + 5) as 16 q 2^-24, so each v_fma_mix_f32 step is fmaf(q, x, t)
// with one rounding.  One accumulator per pair of words.
__device__ __forceinline__ float dot_chunk_f32(const uint4 q, const float4 *xv, float acc) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float c[2] = {acc, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint64_t w2 = ((uint64_t)w[2 * h + 1] << 32) | w[2 * h];
    const uint64_t w8 = shr64_nibbles<2>(w2);
    float t = c[h];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jj = 2 * h + e;
      const uint32_t u0 = (uint32_t)(w2 >> (32 * e)), u8 = (uint32_t)(w8 >> (32 * e));
      const f16x2_t p0 = __builtin_bit_cast(f16x2_t, u0 & 0x000F000Fu);  // codes 0, 4
      const f16x2_t p1 = __builtin_bit_cast(f16x2_t, u0 & 0x00F000F0u);  // 1, 5 (times 16)
      const f16x2_t p2 = __builtin_bit_cast(f16x2_t, u8 & 0x000F000Fu);  // 2, 6
      const f16x2_t p3 = __builtin_bit_cast(f16x2_t, u8 & 0x00F000F0u);  // 3, 7 (times 16)
      const float4 ev = xv[2 * jj], od = xv[2 * jj + 1];
      t = fmaf((float)p0.x, ev.x, t);
      t = fmaf((float)p1.x, od.x, t);
      t = fmaf((float)p2.x, ev.y, t);
      t = fmaf((float)p3.x, od.y, t);
      t = fmaf((float)p0.y, ev.z, t);
      t = fmaf((float)p1.y, od.z, t);
      t = fmaf((float)p2.y, ev.w, t);
      t = fmaf((float)p3.y, od.w, t);
    }
    c[h] = t;
  }
  return c[0] + c[1];
}

// Raw buffer resources: a load whose byte offset is >= the resource's
// num_records returns zero without touching memory.
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

// ---------------------------------------------------------------------------
// Activation staging
// ---------------------------------------------------------------------------
// The activation (ncx chunks of 32 elements) goes to LDS plane-major, so that
// lanes reading consecutive chunks hit consecutive 16 bytes:
//   bf16: plane jj (0..3) of chunk c at uint4 index jj * ncx_pad + c
//   f32 : plane pl (0..7) of chunk c at float4 index pl * ncx_pad + c
// xsum[c] = sum of the chunk's 32 elements (float32, fixed order).  Chunks
// ncx .. ncx_pad-1 are zero.
//
// Staging runs in rounds of xq<XM>() octets (8 elements) per thread: thread t
// of the nthr threads takes octets base + t, base + t + nthr, ...  (nthr comes
// from the kernel arguments rather than the dispatch packet, whose line the
// argument prefetch does not cover.)  The last round is split in
// two: stage_issue() starts its loads, stage_commit() permutes them into LDS,
// and the code loads issued in between overlap the activation's round trip
// (vmcnt drains in issue order, so the commit waits only for the older
// activation loads).  Earlier rounds (very long rows only) complete before
// any code load is issued, so every wait the compiler places after them
// stays exact.
template <int XM>
constexpr int xq() { return xm_octets(XM); }
// Bytes of one octet of the input activation (and of gamma).
template <int XM>
constexpr uint32_t octet_bytes() { return (XM == XM_BF16 || XM == XM_RMS_BF16) ? 16u : 32u; }
// 16-byte vectors loaded per octet: the activation's, then (XM_RMS_*) gamma's.
template <int XM>
constexpr int octet_vecs() { return XM == XM_BF16 ? 1 : XM == XM_F32 || XM == XM_RMS_BF16 ? 2 : 4; }

template <int XM>
struct XRegs {
  uint4 v[xq<XM>()][octet_vecs<XM>()];
};

// Writes octet o (values in v) to the LDS planes and its chunk sum; XM_RMS_*
// add the octet's sum of x^2 to ssq.  Must be called by whole quads of lanes
// (the four octets of a chunk are in one quad).
template <int XM>
__device__ __forceinline__ void stage_store(int o, const uint4 *v, int ncx_pad, unsigned char *xbuf,
                                            float *xsum, float &ssq) {
  const int c = o >> 2, jj = o & 3;
  float s;
  if constexpr (XM == XM_BF16) {
    const uint4 w = v[0];
    uint4 pr;
    pr.x = (w.x & 0xFFFFu) | (w.z << 16);
    pr.y = (w.x >> 16) | (w.z & 0xFFFF0000u);
    pr.z = (w.y & 0xFFFFu) | (w.w << 16);
    pr.w = (w.y >> 16) | (w.w & 0xFFFF0000u);
    reinterpret_cast<uint4 *>(xbuf)[jj * ncx_pad + c] = pr;
    s = ((bf16_lo(w.x) + bf16_hi(w.x)) + (bf16_lo(w.y) + bf16_hi(w.y))) +
        ((bf16_lo(w.z) + bf16_hi(w.z)) + (bf16_lo(w.w) + bf16_hi(w.w)));
  } else {
    float e[8];  // the octet's staged values, element order
    if constexpr (XM == XM_F32) {
      const float4 a = __builtin_bit_cast(float4, v[0]);
      const float4 b = __builtin_bit_cast(float4, v[1]);
      e[0] = a.x; e[1] = a.y; e[2] = a.z; e[3] = a.w;
      e[4] = b.x; e[5] = b.y; e[6] = b.z; e[7] = b.w;
    } else {
      float xe[8], ge[8];
      if constexpr (XM == XM_RMS_F32) {
        const float4 xa = __builtin_bit_cast(float4, v[0]), xb = __builtin_bit_cast(float4, v[1]);
        const float4 ga = __builtin_bit_cast(float4, v[2]), gb = __builtin_bit_cast(float4, v[3]);
        xe[0] = xa.x; xe[1] = xa.y; xe[2] = xa.z; xe[3] = xa.w;
        xe[4] = xb.x; xe[5] = xb.y; xe[6] = xb.z; xe[7] = xb.w;
        ge[0] = ga.x; ge[1] = ga.y; ge[2] = ga.z; ge[3] = ga.w;
        ge[4] = gb.x; ge[5] = gb.y; ge[6] = gb.z; ge[7] = gb.w;
      } else {  // XM_RMS_BF16: bf16 products and squares are exact in float32
        const uint32_t xw[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
        const uint32_t gw[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xe[2 * i] = bf16_lo(xw[i]);
          xe[2 * i + 1] = bf16_hi(xw[i]);
          ge[2 * i] = bf16_lo(gw[i]);
          ge[2 * i + 1] = bf16_hi(gw[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ssq = fmaf(xe[i], xe[i], ssq);
        e[i] = xe[i] * ge[i];
      }
    }
    // even elements times 2^24, odd ones times 2^20 (the scales dot_chunk_f32
    // takes with its f16-subnormal codes); the chunk sum is of the values
    constexpr float kE = 0x1p24f, kO = 0x1p20f;
    reinterpret_cast<float4 *>(xbuf)[(2 * jj) * ncx_pad + c] =
        make_float4(e[0] * kE, e[2] * kE, e[4] * kE, e[6] * kE);
    reinterpret_cast<float4 *>(xbuf)[(2 * jj + 1) * ncx_pad + c] =
        make_float4(e[1] * kO, e[3] * kO, e[5] * kO, e[7] * kO);
    s = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  }
  s += dpp_mov<0xB1>(s);
  s += dpp_mov<0x4E>(s);
  if (jj == 0) xsum[c] = s;
}

// gamma: XM_RMS_* only (the RMSNorm weight, same layout as x).
template <int XM>
__device__ __forceinline__ void stage_issue(const void *__restrict__ x, const void *__restrict__ gamma,
                                            int ncx, int base, int nthr, XRegs<XM> &r) {
  const uint32_t nocts = (uint32_t)ncx * 4;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, nocts * octet_bytes<XM>());
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(xm_rms(XM) ? gamma : x, nocts * octet_bytes<XM>());
#pragma unroll
  for (int i = 0; i < xq<XM>(); ++i) {
    // unconditional loads (a load inside a branch makes the compiler copy its
    // result at the join, which waits for it right away); slots past the end
    // are out of range
    const uint32_t o = base + threadIdx.x + i * nthr;
    const uint32_t off = o < nocts ? o * octet_bytes<XM>() : kOutOfRange;
    constexpr int XV = xm_rms(XM) ? octet_vecs<XM>() / 2 : octet_vecs<XM>();  // vectors of x
#pragma unroll
    for (int k = 0; k < XV; ++k) r.v[i][k] = buf_load_b128(rx, off + 16 * k);
    if constexpr (xm_rms(XM)) {
#pragma unroll
      for (int k = 0; k < XV; ++k) r.v[i][XV + k] = buf_load_b128(rg, off + 16 * k);
    }
  }
}

template <int XM>
__device__ __forceinline__ void stage_commit(int ncx, int ncx_pad, int base, int nthr, const XRegs<XM> &r,
                                             unsigned char *xbuf, float *xsum, float &ssq) {
  const int nocts = ncx * 4;
#pragma unroll
  for (int i = 0; i < xq<XM>(); ++i) {
    const int o = base + threadIdx.x + i * nthr;
    if (o < nocts) stage_store<XM>(o, r.v[i], ncx_pad, xbuf, xsum, ssq);
  }
}

// All staging rounds but the last (the one starting at octet `last`), each
// loaded and stored before the next.
template <int XM>
__device__ __forceinline__ void stage_early_rounds(const void *__restrict__ x, const void *__restrict__ gamma,
                                                   int ncx, int ncx_pad, int last, int nthr,
                                                   unsigned char *xbuf, float *xsum, float &ssq) {
  for (int base = 0; base < last; base += xq<XM>() * nthr) {
    XRegs<XM> r;
    stage_issue<XM>(x, gamma, ncx, base, nthr, r);
    stage_commit<XM>(ncx, ncx_pad, base, nthr, r, xbuf, xsum, ssq);
  }
}

// Zero chunks ncx .. ncx_pad-1 (whole quads: the padding is whole chunks).
template <int XM>
__device__ __forceinline__ void stage_padding(int ncx, int ncx_pad, int nthr, unsigned char *xbuf,
                                              float *xsum, float &ssq) {
  for (int o = ncx * 4 + threadIdx.x; o < ncx_pad * 4; o += nthr) {
    uint4 z[octet_vecs<XM>()];
#pragma unroll
    for (int k = 0; k < octet_vecs<XM>(); ++k) z[k] = make_uint4(0, 0, 0, 0);
    stage_store<XM>(o, z, ncx_pad, xbuf, xsum, ssq);
  }
}

// The MoE residual row, staged as float32 in LDS (loads issued with the
// activation's, before the first code loads; read back at task ends).  The
// host guarantees RQ 16-byte vectors per thread cover it.
constexpr int RQ = 4;

// nvec: 16-byte vectors readable at res (0: no residual; every slot is out
// of range)
__device__ __forceinline__ void residual_issue(const void *res, uint32_t nvec, int nthr, uint4 (&v)[RQ]) {
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(res, nvec * 16);
#pragma unroll
  for (int i = 0; i < RQ; ++i) {
    const uint32_t o = threadIdx.x + i * nthr;
    v[i] = buf_load_b128(rr, o < nvec ? o * 16 : kOutOfRange);
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

__device__ __forceinline__ void residual_commit(int n, int bf16, int nthr, const uint4 (&v)[RQ], float *dst) {
  const int nvec = bf16 ? n / 8 : n / 4;
#pragma unroll
  for (int i = 0; i < RQ; ++i) {
    const int o = threadIdx.x + i * nthr;
    if (o < nvec) residual_store(o, v[i], bf16, dst);
  }
}

__device__ __forceinline__ void store_out(void *y, int64_t i, float v, int bf16) {
  if (bf16)
    reinterpret_cast<__bf16 *>(y)[i] = (__bf16)v;
  else
    reinterpret_cast<float *>(y)[i] = v;
}

// Registers holding one prefetched step (one 32-code chunk of each of the
// task's row groups, with the matching scale and bias).
template <int RT, int NS>
struct StepBuf {
  uint4 q[NS][RT];
  uint32_t s[NS][RT];  // raw scale bits (bf16 zero-extended, or float32)
  uint32_t b[NS][RT];  // raw bias bits; decoded when consumed, so that no
                       // instruction waits on the load where it is issued
  float w;  // EPI_MOE_DOWN: weight of the expert slot this lane's chunk belongs to
};

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
// Wave gw processes tasks gw, gw + n_waves, ... (tasks_q or tasks_q + 1 of
// them).  A load cursor runs D steps ahead of the consume cursor through the
// same (task, step) sequence; both are uniform (scalar) state.  Matrix
// descriptors and buffer resources are refreshed only when the load cursor
// crosses into another matrix (or expert slot).
//
// TT > 1 (small-M products): p.n_tok <= TT activation rows share every code
// load and its decode; each token has its own staged activation, accumulator
// and output row.
//
// P > 0 (one pass): no wave has more than P steps.  The ring is P steps deep
// and is filled once; nothing is loaded after the prologue, so no load is
// issued for a step past the wave's end except when the wave has fewer than
// P steps.
template <int RT, int XM, int SBT, int EPI, int TT, int P>
__global__ void __launch_bounds__(TT >= 8 ? 512 : 768) qgemv_kernel(const GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  warm_kernargs<sizeof(GemvParams)>();
  constexpr int NS = (EPI == EPI_SWIGLU) ? 2 : 1;  // code streams per row (gate, up)
  constexpr int D = P > 0 ? P : kSlots / (RT * NS);  // steps in flight
  static_assert(D * RT * NS <= kSlots, "ring deeper than the register budget");
  constexpr int XB = (XM == XM_BF16) ? 64 : 128;   // staged bytes per chunk
  static_assert(!xm_rms(XM) || (TT == 1 && EPI != EPI_MOE_DOWN), "RMSNorm prologue: one token");
  constexpr uint32_t SBB = (SBT == 1) ? 2 : 4;     // bytes per scale/bias

  const int lane = threadIdx.x & 63;
  // wave index made provably uniform: all task bookkeeping stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * p.waves_per_wg + wave;
  const int nthr = p.waves_per_wg * 64;  // threads of the workgroup
  const int NW = p.n_waves;
  const int l2 = p.log2_lpr;
  const int L = 1 << l2;
  const int j = lane & (L - 1);
  const int sg = lane >> l2;
  const int rpi = 64 >> l2;  // rows per wave instruction
  const int rpt = p.rpt;     // rows per task (RT * rpi)
  const int spt = p.spt;
  const int ncx_pad = p.ncx_pad;
  const uint32_t kwb = (uint32_t)p.kwb;
  const uint32_t sbrow = (uint32_t)p.sbrow;
  const int lg = p.log2_group;
  const int S = (p.tasks_q + (gw < p.tasks_r ? 1 : 0)) * spt;  // steps of this wave

  // LDS: per token, chunk sums then the staged activation; then (MoE down)
  // the float32 residual row, or (XM_RMS_*) one partial sum of x^2 per wave
  const int xs_bytes = (ncx_pad * 4 + 15) & ~15;
  const int tok_bytes = xs_bytes + ncx_pad * XB;
  float *xsum = reinterpret_cast<float *>(smem);
  unsigned char *xbuf = smem + xs_bytes;
  float *res_lds = reinterpret_cast<float *>(smem + (size_t)TT * tok_bytes);  // EPI_MOE_DOWN

  // expert ids and slot weights, through the scalar cache: lane k of v_ids /
  // v_wts holds slot k's values
  // (given ids are read once the activation loads are in flight, below)
  uint32_t v_ids = 0, v_wts = 0;
  // Routing (EPI_SWIGLU, p.route != 0): this token's router logits are loaded
  // here (lane l: experts l, l + 64, ...; indices past n_experts clamped, so
  // every load is unconditional) and ranked after the activation loads are
  // issued, so the two round trips overlap.
  constexpr int RK = kRouteMaxExperts / 64;
  float key[RK];
  if constexpr (EPI == EPI_SWIGLU) {
    if (p.route) {
#pragma unroll
      for (int s = 0; s < RK; ++s) {
        const int i = min(lane + 64 * s, p.n_experts - 1);
        key[s] = p.route == 2 ? bf16_lo(reinterpret_cast<const uint16_t *>(p.aux)[i])
                              : reinterpret_cast<const float *>(p.aux)[i];
      }
    }
  }
  uint32_t magic = 0x43004300u;
  asm volatile("" : "+v"(magic));  // keep in a VGPR so AND-OR stays one VOP3

  // per-lane constant parts of the load offsets
  const uint32_t lo_c = (uint32_t)sg * kwb + (uint32_t)j * 16;
  const uint32_t lo_s = (uint32_t)sg * sbrow + (((uint32_t)j * 32) >> lg) * SBB;
  const uint32_t step_c = (uint32_t)L * 16;
  const uint32_t step_s = (((uint32_t)L * 32) >> lg) * SBB;
  const bool lane_in_last = j < p.last_lanes;  // lane holds a chunk in a row's last step

  // ---- cursors over (task, step) ----
  // A cursor walks this wave's tasks t = gw, gw + NW, ...  Moving to the next
  // task is an add and a compare against the first task of the next matrix
  // (or expert slot); crossing it, which is rare, re-reads that matrix's
  // descriptor.
  struct Cur {
    int t;       // task
    int m;       // matrix (EPI_STORE) or expert slot (EPI_SWIGLU)
    int bound;   // first task past matrix / slot m
    int row0;    // first row of the task inside its matrix
    int n_rows;
    bool live;   // EPI_SWIGLU: the slot's expert id is valid
    unsigned char *y;  // output of matrix / slot m
  };
  const int row_step = NW * rpt;  // rows between a wave's consecutive tasks
  auto seek = [&](Cur &c) {  // matrix / slot of task c.t, its geometry and row0
    int m = c.m;
    if constexpr (EPI == EPI_STORE) {
      // task0 is ascending with INT32_MAX past n_mats: the matrix is the count
      // of later starts at or below t, its start the largest of them and the
      // bound the smallest start above t (all read at once, no dependent loads)
      m = 0;
      int first = 0, bound = p.n_tasks;
#pragma unroll
      for (int i = 1; i < kMaxMats; ++i) {
        const int t0 = p.task0[i];
        const bool in = c.t >= t0;
        m += in ? 1 : 0;
        first = in ? t0 : first;
        bound = (!in && t0 < bound) ? t0 : bound;
      }
      c.bound = bound;
      c.n_rows = (int)p.m[m].n_out;
      c.row0 = (c.t - first) * rpt;
      c.y = reinterpret_cast<unsigned char *>(p.m[m].y);
    } else if constexpr (EPI == EPI_SWIGLU) {
      m = min(c.t / p.tasks_per_slot, p.top_k - 1);
      c.bound = (m + 1 < p.top_k) ? (m + 1) * p.tasks_per_slot : p.n_tasks;
      const uint32_t e = p.ids ? (uint32_t)__builtin_amdgcn_readlane((int)v_ids, m) : 0u;
      c.live = e < (uint32_t)p.n_experts;
      c.n_rows = (int)p.m[0].n_out;
      c.row0 = (c.t - m * p.tasks_per_slot) * rpt;
      c.y = reinterpret_cast<unsigned char *>(p.m[0].y) + (int64_t)m * c.n_rows * (p.y_bf16 ? 2 : 4);
    } else {
      c.bound = p.n_tasks;
      c.n_rows = (int)p.m[0].n_out;
      c.row0 = c.t * rpt;
      c.y = reinterpret_cast<unsigned char *>(p.m[0].y);
    }
    c.m = m;
  };
  auto start = [&](Cur &c) {
    c.t = gw;
    c.m = 0;
    c.live = true;
    seek(c);
  };
  // next task; true when the cursor moved into another matrix / slot
  auto next_task = [&](Cur &c) {
    c.t += NW;
    if (c.t < c.bound) {
      c.row0 += row_step;
      return false;
    }
    if (c.t < p.n_tasks) seek(c);
    return true;
  };

  // ---- load stream ----
  Cur lc;  // started once the expert ids are known
  __amdgpu_buffer_rsrc_t rc[NS], rs[NS], rb[NS];
  auto set_rsrc = [&]() {
    if constexpr (EPI == EPI_STORE) {
      const GemvMat &d = p.m[lc.m];
      rc[0] = make_rsrc(d.codes, (uint32_t)lc.n_rows * kwb);
      rs[0] = make_rsrc(d.scales, (uint32_t)lc.n_rows * sbrow);
      rb[0] = make_rsrc(d.biases, (uint32_t)lc.n_rows * sbrow);
    } else if constexpr (EPI == EPI_SWIGLU) {
      // a skipped slot (invalid id) reads nothing: zero-size resources
      const uint32_t e = p.ids ? (uint32_t)__builtin_amdgcn_readlane((int)v_ids, lc.m) : 0u;
      const uint32_t ee = lc.live ? e : 0u;
      const uint32_t cb = lc.live ? (uint32_t)lc.n_rows * kwb : 0u;
      const uint32_t sb = lc.live ? (uint32_t)lc.n_rows * sbrow : 0u;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        rc[s] = make_rsrc(reinterpret_cast<const unsigned char *>(p.m[s].codes) + (uint64_t)ee * p.ecode_bytes, cb);
        rs[s] = make_rsrc(reinterpret_cast<const unsigned char *>(p.m[s].scales) + (uint64_t)ee * p.esb_bytes, sb);
        rb[s] = make_rsrc(reinterpret_cast<const unsigned char *>(p.m[s].biases) + (uint64_t)ee * p.esb_bytes, sb);
      }
    } else {
      rc[0] = make_rsrc(p.m[0].codes, p.code_bytes);
      rs[0] = make_rsrc(p.m[0].scales, p.sb_bytes);
      rb[0] = make_rsrc(p.m[0].biases, p.sb_bytes);
    }
  };
  int lstep = 0;   // steps issued by the load cursor
  int lit = 0;     // step inside the task
  uint32_t lstep_c = 0, lstep_s = 0;  // byte offsets of step lit inside a row
  // advance = false: the last load of a one-pass ring (the cursor is not needed again)
  auto load = [&](StepBuf<RT, NS> &bf, bool advance) {
    // past the wave's last step: out of range (the load is still issued, so
    // the number of loads in flight, and with it every wait, is static)
    const bool past = lstep++ >= S;
    uint32_t oc, os;
    if constexpr (EPI == EPI_MOE_DOWN) {
      // virtual row = the kept experts' rows back to back; this lane's slot
      const int c = j + lit * L;
      const int slot = (int)(((float)c + 0.5f) * p.inv_cpr_e);
      const int cl = c - slot * p.cpr_e;
      const uint32_t e = (uint32_t)__shfl((int)v_ids, slot);
      const float w = __uint_as_float((uint32_t)__shfl((int)v_wts, slot));
      const bool ok = slot < p.top_k && e < (uint32_t)p.n_experts;  // else: skipped, weight 0
      bf.w = ok ? w : 0.f;
      const uint32_t rowc = (uint32_t)(lc.row0 + sg) * kwb, rows = (uint32_t)(lc.row0 + sg) * sbrow;
      oc = ok && !past ? e * p.ecode_bytes + rowc + (uint32_t)cl * 16 : kOutOfRange;
      os = ok && !past ? e * p.esb_bytes + rows + (((uint32_t)cl * 32) >> lg) * SBB : kOutOfRange;
    } else {
      // partial last step: lanes past the row's chunks have nothing to load
      const bool off = past || (lit == spt - 1 && !lane_in_last);
      oc = off ? kOutOfRange : lo_c + ((uint32_t)lc.row0 * kwb + lstep_c);
      os = off ? kOutOfRange : lo_s + ((uint32_t)lc.row0 * sbrow + lstep_s);
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      // rows past the matrix (or stack) end fall outside the resource: zeros
      const uint32_t rc_off = (uint32_t)(r * rpi) * kwb;
      const uint32_t rs_off = (uint32_t)(r * rpi) * sbrow;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        bf.q[s][r] = buf_load_b128(rc[s], oc + rc_off);
        bf.s[s][r] = buf_load_sb<SBT>(rs[s], os + rs_off);
        bf.b[s][r] = buf_load_sb<SBT>(rb[s], os + rs_off);
      }
    }
    // advance the load cursor
    if (!advance) return;
    lstep_c += step_c;
    lstep_s += step_s;
    if (++lit == spt) {
      lit = 0;
      lstep_c = 0;
      lstep_s = 0;
      if (next_task(lc) && lc.t < p.n_tasks) set_rsrc();
    }
  };

  // token t's activation is x + t * ldx elements; tokens past n_tok stage zeros
  auto x_tok = [&](int t) {
    return reinterpret_cast<const unsigned char *>(p.x) + (size_t)t * p.ldx * (XM == XM_BF16 ? 2 : 4);
  };
  float ssq = 0.f;  // XM_RMS_*: this thread's share of sum(x^2)
  const int xbase = p.stage_last;
#pragma unroll
  for (int t = 0; t < TT; ++t)
    stage_early_rounds<XM>(x_tok(t), p.aux, t < p.n_tok ? p.ncx : 0, ncx_pad, t < p.n_tok ? xbase : 0,
                           nthr, xbuf + t * tok_bytes,
                           reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(xsum) + t * tok_bytes),
                           ssq);
  XRegs<XM> xr[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t)  // activation loads first (L2), ...
    stage_issue<XM>(x_tok(t), p.aux, t < p.n_tok ? p.ncx : 0, xbase, nthr, xr[t]);
  uint4 rr[RQ];
  const bool has_res = (EPI == EPI_MOE_DOWN) && p.aux != nullptr;
  if constexpr (EPI == EPI_MOE_DOWN) {
    const uint32_t nvec = has_res ? (uint32_t)(p.y_bf16 ? p.m[0].n_out / 8 : p.m[0].n_out / 4) : 0u;
    residual_issue(has_res ? p.aux : p.x, nvec, nthr, rr);
  }

  if constexpr (EPI == EPI_SWIGLU) {
    if (p.route) {
      // the first wave of each workgroup ranks the logits (every workgroup
      // the same way) and hands the ids to the others through LDS, so the
      // ranking does not take every wave's SIMD time while the code loads
      // wait for it; lane k < top_k takes slot k.  The first wave of the grid
      // also writes the ids and weights out for the down launch and the caller.
      uint32_t *rid = reinterpret_cast<uint32_t *>(res_lds);  // 8 ids (64 B reserved by the host)
      if (wave == 0) {
        int sel_i[8];
        float sel_v[8];
        if (p.n_experts <= 128) {
          const float k2[2] = {key[0], key[1]};
          topk::select<2>(k2, p.n_experts, p.top_k, sel_i, sel_v);
        } else {
          topk::select<RK>(key, p.n_experts, p.top_k, sel_i, sel_v);
        }
        int id = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (lane == k) id = sel_i[k];
        if (lane < 8) rid[lane] = (uint32_t)id;
        if (blockIdx.x == 0 && lane < p.top_k) {
          p.ids[lane] = (uint32_t)id;
          p.wts[lane] = topk::slot_weight(sel_v, p.top_k, lane);
        }
      }
      lds_barrier();
      v_ids = lane < 8 ? rid[lane] : 0u;
    }
  }
  // Given expert ids (and, for the down projection, the slot weights), read
  // through the scalar cache while the activation loads are in flight; the
  // wait for them does not drain those vector loads.
  if constexpr (EPI == EPI_SWIGLU) {
    if (!p.route && p.ids) {
      uint32_t s_ids[8];
      scalar_load8(p.ids, p.top_k, s_ids);
      v_ids = lanes_from_scalars(s_ids);
    }
  } else if constexpr (EPI == EPI_MOE_DOWN) {
    if (p.ids) {
      uint32_t s_ids[8], s_wts[8];
      scalar_load8x2(p.ids, reinterpret_cast<const uint32_t *>(p.wts), p.top_k, s_ids, s_wts);
      v_ids = lanes_from_scalars(s_ids);
      v_wts = lanes_from_scalars(s_wts);
    }
  }
  start(lc);
  set_rsrc();

  // ... then the first D steps of codes (HBM).
  StepBuf<RT, NS> buf[D];
#pragma unroll
  for (int u = 0; u < D; ++u) load(buf[u], P == 0 || u + 1 < D);

#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float *xs_t = reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(xsum) + t * tok_bytes);
    stage_commit<XM>(p.ncx, ncx_pad, xbase, nthr, xr[t], xbuf + t * tok_bytes, xs_t, ssq);
    stage_padding<XM>(p.ncx, ncx_pad, nthr, xbuf + t * tok_bytes, xs_t, ssq);
  }
  if (has_res) residual_commit((int)p.m[0].n_out, p.y_bf16, nthr, rr, res_lds);
  if constexpr (xm_rms(XM)) {
    const float wave_ssq = seg_sum(ssq, 6);
    if (lane == 0) res_lds[wave] = wave_ssq;
  }
  lds_barrier();

  // RMSNorm: every wave sums the per-wave partials in the same order
  float inv_rms = 1.f;
  if constexpr (xm_rms(XM)) {
    float tot = 0.f;
    for (int wv = 0; wv < p.waves_per_wg; ++wv) tot += res_lds[wv];
    inv_rms = 1.f / sqrtf(tot / (float)(p.ncx * 32) + p.eps);
  }

  // ---- consume stream ----
  float acc[TT][NS][RT];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int r = 0; r < RT; ++r) acc[t][s][r] = 0.f;
  Cur cc;
  start(cc);
  int cit = 0;  // step inside the task

  auto finish = [&]() {
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t >= p.n_tok) break;  // uniform
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          acc[t][s][r] = seg_sum(acc[t][s][r], l2);
          if constexpr (xm_rms(XM)) acc[t][s][r] *= inv_rms;
        }
      if (j == 0) {
        // token t's output row: y + t * n_rows elements
        void *yt = cc.y + (size_t)t * cc.n_rows * (p.y_bf16 ? 2 : 4);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const int row = cc.row0 + r * rpi + sg;
          if (row < cc.n_rows) {
            if constexpr (EPI == EPI_STORE) {
              store_out(yt, row, acc[t][0][r], p.y_bf16);
            } else if constexpr (EPI == EPI_SWIGLU) {
              const float g = acc[t][0][r], u = acc[t][1][r];
              const float h = cc.live ? (g / (1.f + __expf(-g))) * u : 0.f;
              store_out(yt, row, h, p.y_bf16);
            } else {
              const float res = has_res ? res_lds[row] : 0.f;
              store_out(yt, row, res + acc[t][0][r], p.y_bf16);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[t][s][r] = 0.f;
  };

  auto consume = [&](const StepBuf<RT, NS> &bf) {
    const int xc = j + cit * L;  // staged chunk (virtual row chunk); < ncx_pad
    if constexpr (XM == XM_BF16) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          uint32_t pq[16];
          decode_chunk_bf16(bf.q[s][r], magic, pq);  // once for every token
          const float sc = sb_value<SBT>(bf.s[s][r]), bi = sb_value<SBT>(bf.b[s][r]);
#pragma unroll
          for (int t = 0; t < TT; ++t) {
            const unsigned char *xb = xbuf + t * tok_bytes;
            const float xs = *reinterpret_cast<const float *>(xb - xs_bytes + 4 * xc);
            uint4 xv[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) xv[jj] = reinterpret_cast<const uint4 *>(xb)[jj * ncx_pad + xc];
            const float d = dot_pq_bf16(pq, xv, -128.f * xs);  // sum q x
            const float part = fmaf(sc, d, bi * xs);
            if constexpr (EPI == EPI_MOE_DOWN)
              acc[t][s][r] = fmaf(bf.w, part, acc[t][s][r]);
            else
              acc[t][s][r] += part;
          }
        }
    } else {
      static_assert(XM == XM_BF16 || TT == 1, "float32 activations: one token");
      const float xs = xsum[xc];
      float4 xv[8];
#pragma unroll
      for (int pl = 0; pl < 8; ++pl) xv[pl] = reinterpret_cast<const float4 *>(xbuf)[pl * ncx_pad + xc];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const float d = dot_chunk_f32(bf.q[s][r], xv, 0.f);
          const float part = fmaf(sb_value<SBT>(bf.s[s][r]), d, sb_value<SBT>(bf.b[s][r]) * xs);
          if constexpr (EPI == EPI_MOE_DOWN)
            acc[0][s][r] = fmaf(bf.w, part, acc[0][s][r]);
          else
            acc[0][s][r] += part;
        }
    }
    if (++cit == spt) {
      finish();
      cit = 0;
      next_task(cc);
    }
  };

  if constexpr (P > 0) {
#pragma unroll
    for (int u = 0; u < D; ++u)
      if (u < S) consume(buf[u]);
  } else {
    for (int s0 = 0; s0 < S; s0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        if (s0 + u < S) consume(buf[u]);
        load(buf[u], true);
      }
    }
  }
}

template <int RT, int XM, int SBT, int EPI, int TT = 1>
hipError_t launch_one(const GemvParams &p, const GemvPlan &plan, hipStream_t stream) {
  auto kern = qgemv_kernel<RT, XM, SBT, EPI, TT, 0>;
  // the ring form the plan calls for (gemv_ring_depth is also what the
  // library's plan query reports)
  constexpr int NS = (EPI == EPI_SWIGLU) ? 2 : 1;
  if (plan.rt != RT || plan.tt != TT || plan.grid * plan.waves != p.n_waves)
    return hipErrorInvalidValue;
  if constexpr (gemv_has_one_pass(EPI, TT, XM)) {
    switch (gemv_ring_depth(plan, XM, EPI)) {
      case 1: kern = qgemv_kernel<RT, XM, SBT, EPI, TT, 1>; break;
      case 2:
        if constexpr (2 * RT * NS <= kSlots) kern = qgemv_kernel<RT, XM, SBT, EPI, TT, 2>;
        break;
      case 4:
        if constexpr (4 * RT * NS <= kSlots) kern = qgemv_kernel<RT, XM, SBT, EPI, TT, 4>;
        break;
      default: break;
    }
  }
  // opt in to more than 64 KB of dynamic LDS (once per device)
  if (plan.lds_bytes > 64 * 1024) {
    hipError_t e = lds_opt_in(reinterpret_cast<const void *>(kern), kMaxLds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)plan.grid), dim3(plan.waves * 64), plan.lds_bytes,
                     stream, p);
  return hipGetLastError();
}

// Kernel selection: (rt, xmode, sb_bf16, epi) -> instantiation.  MoE down
// always stages a float32 activation (the SwiGLU intermediates).
template <int RT, int EPI>
hipError_t launch_sel(const GemvParams &p, const GemvPlan &plan, int xmode, int sb_bf16,
                      hipStream_t s) {
  if constexpr (EPI != EPI_MOE_DOWN) {
    if (xmode == XM_RMS_BF16)
      return sb_bf16 ? launch_one<RT, XM_RMS_BF16, 1, EPI>(p, plan, s)
                     : launch_one<RT, XM_RMS_BF16, 0, EPI>(p, plan, s);
    if (xmode == XM_RMS_F32)
      return sb_bf16 ? launch_one<RT, XM_RMS_F32, 1, EPI>(p, plan, s)
                     : launch_one<RT, XM_RMS_F32, 0, EPI>(p, plan, s);
  } else if (xm_rms(xmode)) {
    return hipErrorInvalidValue;
  }
  if (EPI == EPI_MOE_DOWN || xmode == XM_F32)
    return sb_bf16 ? launch_one<RT, XM_F32, 1, EPI>(p, plan, s) : launch_one<RT, XM_F32, 0, EPI>(p, plan, s);
  return sb_bf16 ? launch_one<RT, XM_BF16, 1, EPI>(p, plan, s) : launch_one<RT, XM_BF16, 0, EPI>(p, plan, s);
}

}  // namespace

size_t gemv_lds_bytes(int xmode, int ncx_pad, int64_t residual_rows, int tt) {
  const size_t xb = (xmode == XM_BF16) ? 64 : 128;
  return (size_t)tt * ((((size_t)ncx_pad * 4 + 15) & ~(size_t)15) + (size_t)ncx_pad * xb) +
         (size_t)residual_rows * 4;
}

// Small-M launches: bf16 activations, store or SwiGLU-pair epilogue.
template <int TT>
hipError_t launch_tokens(const GemvParams &p, const GemvPlan &plan, int sb_bf16, int epi,
                         hipStream_t s) {
  if (epi == EPI_STORE)
    return plan.rt == 2 ? (sb_bf16 ? launch_one<2, XM_BF16, 1, EPI_STORE, TT>(p, plan, s)
                                   : launch_one<2, XM_BF16, 0, EPI_STORE, TT>(p, plan, s))
                        : (sb_bf16 ? launch_one<1, XM_BF16, 1, EPI_STORE, TT>(p, plan, s)
                                   : launch_one<1, XM_BF16, 0, EPI_STORE, TT>(p, plan, s));
  if (epi == EPI_SWIGLU)
    return plan.rt == 2 ? (sb_bf16 ? launch_one<2, XM_BF16, 1, EPI_SWIGLU, TT>(p, plan, s)
                                   : launch_one<2, XM_BF16, 0, EPI_SWIGLU, TT>(p, plan, s))
                        : (sb_bf16 ? launch_one<1, XM_BF16, 1, EPI_SWIGLU, TT>(p, plan, s)
                                   : launch_one<1, XM_BF16, 0, EPI_SWIGLU, TT>(p, plan, s));
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(const GemvParams &p_in, const GemvPlan &plan, int xmode, int sb_bf16, int epi,
                       hipStream_t stream) {
  if (plan.rt != 1 && plan.rt != 2) return hipErrorInvalidValue;
  // activation staging rounds of xm_octets(xmode) octets per thread
  GemvParams p = p_in;
  const int64_t per_round = (int64_t)xm_octets(xmode) * plan.waves * 64;
  const int64_t rounds = ((int64_t)p.ncx * 4 + per_round - 1) / per_round;
  p.stage_last = (int32_t)(std::max<int64_t>(rounds, 1) - 1) * (int32_t)per_round;
  if (plan.tt != 1) {
    if (xmode != XM_BF16) return hipErrorInvalidValue;
    switch (plan.tt) {
      case 2: return launch_tokens<2>(p, plan, sb_bf16, epi, stream);
      case 4: return launch_tokens<4>(p, plan, sb_bf16, epi, stream);
      case 8: return launch_tokens<8>(p, plan, sb_bf16, epi, stream);
      default: return hipErrorInvalidValue;
    }
  }
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
