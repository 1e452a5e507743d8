// qgemm_stream.hip -- prefill int4 dequant GEMM with register-resident weights
// on gfx950 bf16 MFMA (v_mfma_f32_16x16x32_bf16).
//
//   Y[t][o] = sum_k bf16(s[o][k/g] * q[o][k] + b[o][k/g]) * X[t][k],  t < T
//
// Source: thewafflehaus/FFAI pull 9, "Everything Bagel", commit adding the
// dequantGemmDynamicM T-padding driver (rows past T are zero and sliced
// away) -- here rows >= T are predicated, never read or written.
//
// Work decomposition (gfx950 specific):
//   * A wave owns NTW tiles of 16 output rows and a block of 16 * MT tokens
//     and walks the whole K range in steps of 128.  In a step, lane
//     (r = l % 16, q = l / 16) loads the 32 codes k0 + 32q .. k0 + 32q + 31 of
//     row r with one 128-bit load and dequantises them in registers
//     (float32 s * q + b, rounded to bf16): word s of that chunk is the B
//     operand of MFMA sub-step s.  Sub-step s therefore covers the k set
//     {k0 + 32q + 8s + j : q < 4, j < 8}; the matching A operand (the
//     activations) is read from LDS with the same k set, so the sum over k
//     is unchanged.
//   * Weights never pass through LDS.  Each wave keeps D steps of code,
//     scale and bias loads in flight in a register ring (raw buffer loads:
//     rows past n_out and chunks past k_in read as zero without touching
//     memory, so every load is unconditional).
//   * The 16 * MT x 128 activation tile of each step is staged in an
//     NBUF-deep LDS ring (one barrier per step) by one extra producer wave
//     with direct buffer-to-LDS loads, and shared by the W compute waves,
//     which cover different rows.  Loads complete in issue
//     order as far as the wait counters go, so an activation load issued by a
//     compute wave behind its weight ring would drain that ring; the producer
//     wave keeps the two streams apart.
//   * Output: accumulator element i of lane l is token 4 (l / 16) + i,
//     output row l % 16 of the 16 x 16 tile, so 16 lanes store 16
//     consecutive outputs of one token row.

#include "kernels.h"

namespace qint4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int KS = 128;           // k per step
constexpr uint32_t kOOR = 0x80000000u;

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

template <int SBT>
__device__ __forceinline__ uint32_t ldsb(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (SBT == 1)
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  else
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

template <int SBT>
__device__ __forceinline__ float sbval(uint32_t bits) {
  return __uint_as_float(SBT == 1 ? (bits << 16) : bits);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// 8 codes of one word -> the 8 bf16 weights s * q + b (code order).
__device__ __forceinline__ bf16x8_t dequant8(uint32_t w, float s, float b) {
  uint32_t lo = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6 in bytes 0..3
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
  asm("" : "+v"(lo), "+v"(hi));
  uint4 r;
  r.x = pack2(fmaf(s, (float)(lo & 0xFFu), b), fmaf(s, (float)(hi & 0xFFu), b));
  r.y = pack2(fmaf(s, (float)((lo >> 8) & 0xFFu), b), fmaf(s, (float)((hi >> 8) & 0xFFu), b));
  r.z = pack2(fmaf(s, (float)((lo >> 16) & 0xFFu), b), fmaf(s, (float)((hi >> 16) & 0xFFu), b));
  r.w = pack2(fmaf(s, (float)(lo >> 24), b), fmaf(s, (float)(hi >> 24), b));
  return __builtin_bit_cast(bf16x8_t, r);
}

template <int NTW>
struct WStep {
  uint4 q[NTW];
  uint32_t s[NTW], b[NTW];
};

// vmcnt <= n (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima, i.e. not waited for)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Activation tile layout in LDS (per buffer and K slice): TOK token rows of
// 16 vectors of 16 bytes (8 bf16), no padding; vector g of token t is stored
// at position g ^ (t & 15) of its row, so the 16 rows a 16-lane group reads
// at one g fall in 16 different bank groups.
__device__ __forceinline__ int xs_index(int t, int g) { return t * KS + 8 * (g ^ (t & 15)); }

template <int MT, int NTW, int W, int D, int SBT, int NBUF>
__global__ void __launch_bounds__((W + 1) * 64) qgemm_stream_kernel(const GemmParams p) {
  constexpr int TOK = 16 * MT;                       // tokens per workgroup
  constexpr int NBLK = TOK / 4;                      // producer load instructions per step (4 rows each)
  constexpr uint32_t SBB = SBT == 1 ? 2 : 4;
  constexpr int TILE = TOK * KS;                     // bf16 elements of one activation tile
  constexpr int NT = (W + 1) * 64;
  static_assert(NBUF >= 2, "activation ring");
  static_assert(NT <= 1024, "workgroup too large");

  // activation tile ring (dynamic LDS, NBUF * TILE bf16)
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // token block fastest: workgroups launched together share weight rows
  const int tb = blockIdx.x % p.m_tiles;
  const int nb = blockIdx.x / p.m_tiles;
  const int64_t t0 = (int64_t)tb * TOK;
  const int nsteps = (p.k_in + KS - 1) / KS;
  // The K loop runs a whole number of D-step rounds, so no branch sits inside
  // a round (a branch around a step makes the compiler wait for every load in
  // flight); steps past the end load out-of-range zeros and add nothing.
  const int spw = (nsteps + D - 1) / D * D;

  // Zero the activation ring once: lanes of a tile that fall past T or k_in
  // then hold finite values whatever the out-of-range loads leave, and those
  // only meet zero weights (k past k_in) or outputs that are never stored.
  for (int i = threadIdx.x; i < NBUF * TILE / 8; i += NT)
    reinterpret_cast<uint4 *>(xs)[i] = make_uint4(0, 0, 0, 0);
  lds_barrier();

  if (wave == W) {
    // ---- producer wave: the activation tile of each step goes straight
    // from memory into LDS (buffer loads with an LDS destination: no
    // registers), NBUF - 1 steps ahead.  Its loads are the only ones it waits
    // for, so the compute waves' weight rings are never drained by them.
    const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, 0x7FFFFFF0u);
    auto issue = [&](int j) {  // step j -> buffer j % NBUF
      uint16_t *base = xs + (j % NBUF) * TILE;
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int t = b * 4 + (lane >> 4);
        const int g = (lane & 15) ^ (t & 15);       // lane i writes position i of the block
        const int64_t tok = t0 + t;
        const int k = j * KS + 8 * g;
        const bool ok = tok < p.T && k < p.k_in && j < spw;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (__attribute__((address_space(3))) void *)(base + b * 4 * KS), 16,
            ok ? (uint32_t)((tok * p.ldx + k) * 2) : kOOR, 0, 0, 0);
      }
    };
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j) issue(j);
    wait_vmcnt<(NBUF - 2) * NBLK>();  // step 0's tiles are in LDS
    lds_barrier();
    for (int j = 0; j < spw; ++j) {
      issue(j + NBUF - 1);              // into the buffer step j - 1 used
      wait_vmcnt<(NBUF - 2) * NBLK>();  // step j + 1's tiles are in LDS
      lds_barrier();
    }
    return;
  }

  // ---- compute waves ----
  const int r = lane & 15, q = lane >> 4;
  const int row0 = (nb * W + wave) * (16 * NTW);     // first row of this wave
  const uint32_t kwb = (uint32_t)p.k_in / 2;         // code bytes per row
  const uint32_t gpr = (uint32_t)p.k_in >> p.log2_group;
  const uint32_t sbrow = gpr * SBB;

  const __amdgpu_buffer_rsrc_t rc = rsrc(p.codes, (uint32_t)p.n_out * kwb);
  const __amdgpu_buffer_rsrc_t rs = rsrc(p.scales, (uint32_t)p.n_out * sbrow);
  const __amdgpu_buffer_rsrc_t rb = rsrc(p.biases, (uint32_t)p.n_out * sbrow);

  // per-lane byte offsets of the code / scale loads of row tile 0
  // (rows past n_out fall outside the resources and read as zero)
  const uint32_t c_lane = (uint32_t)(row0 + r) * kwb + (uint32_t)q * 16;
  const uint32_t s_lane = (uint32_t)(row0 + r) * sbrow;
  const int cpr = p.k_in / 32;

  auto load_w = [&](int kt, WStep<NTW> &st) {
    const int c = kt * 4 + q;                        // this lane's 32-code chunk
    const bool ok = kt < spw && c < cpr;
    const uint32_t gofs = (((uint32_t)c * 32) >> p.log2_group) * SBB;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const uint32_t oc = ok ? c_lane + (uint32_t)nt * 16 * kwb + (uint32_t)kt * 64 : kOOR;
      const uint32_t os = ok ? s_lane + (uint32_t)nt * 16 * sbrow + gofs : kOOR;
      st.q[nt] = ld128(rc, oc);
      st.s[nt] = ldsb<SBT>(rs, os);
      st.b[nt] = ldsb<SBT>(rb, os);
    }
  };

  f32x4_t acc[MT][NTW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[m][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  WStep<NTW> ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u) load_w(u, ring[u]);
  lds_barrier();  // the first activation tiles are in LDS

  for (int j0 = 0; j0 < spw; j0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int j = j0 + u;
      // dequantise this step's weights: B operands of the four sub-steps
      bf16x8_t bw[NTW][4];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const float sc = sbval<SBT>(ring[u].s[nt]), bi = sbval<SBT>(ring[u].b[nt]);
        const uint32_t wd[4] = {ring[u].q[nt].x, ring[u].q[nt].y, ring[u].q[nt].z, ring[u].q[nt].w};
#pragma unroll
        for (int s = 0; s < 4; ++s) bw[nt][s] = dequant8(wd[s], sc, bi);
      }
      load_w(j + D, ring[u]);  // refill the slot just consumed
      const uint16_t *xt = xs + (j % NBUF) * TILE;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(xt + xs_index(m * 16 + r, 4 * q + s));
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
            acc[m][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw[nt][s], acc[m][nt], 0, 0, 0);
        }
      lds_barrier();
    }
  }

  // epilogue
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int o = row0 + nt * 16 + r;
      if (o >= p.n_out) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + m * 16 + 4 * q + i;
        if (t < p.T) {
          if (p.y_bf16)
            reinterpret_cast<__bf16 *>(p.y)[t * p.ldy + o] = (__bf16)acc[m][nt][i];
          else
            reinterpret_cast<float *>(p.y)[t * p.ldy + o] = acc[m][nt][i];
        }
      }
    }
}

template <int MT, int NTW, int W, int D, int NBUF>
hipError_t launch_cfg(GemmParams p, hipStream_t stream) {
  constexpr int TOK = 16 * MT;
  p.m_tiles = (int)((p.T + TOK - 1) / TOK);
  p.n_tiles = (p.n_out + W * 16 * NTW - 1) / (W * 16 * NTW);
  const int64_t grid = (int64_t)p.m_tiles * p.n_tiles;
  auto kern = p.sb_bf16 ? qgemm_stream_kernel<MT, NTW, W, D, 1, NBUF>
                        : qgemm_stream_kernel<MT, NTW, W, D, 0, NBUF>;
  constexpr size_t lds = (size_t)NBUF * TOK * KS * 2;
  static_assert(lds <= kMaxLds, "activation ring exceeds LDS");
  // Opt in to more than 64 KB of dynamic LDS once per process and kernel (a
  // benign race: concurrent first calls set the same value).
  static bool big_lds[2] = {false, false};
  if (lds > 64 * 1024 && !big_lds[p.sb_bf16 ? 1 : 0]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    big_lds[p.sb_bf16 ? 1 : 0] = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3((W + 1) * 64), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_stream(const GemmParams &p, int cfg, hipStream_t stream) {
  switch (cfg) {
    case 0: return launch_cfg<2, 1, 2, 8, 3>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qint4
