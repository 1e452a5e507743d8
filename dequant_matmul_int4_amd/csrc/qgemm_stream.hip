// qgemm_stream.hip -- prefill int4 dequant GEMM for T <= 64 with
// register-resident weights on gfx950 bf16 MFMA (v_mfma_f32_16x16x32_bf16).
//
//   Y[t][o] = sum_k bf16(s[o][k/g] * q[o][k] + b[o][k/g]) * X[t][k],  t < T
//
// Source: thewafflehaus/FFAI pull 9, "Everything Bagel", commit adding the
// dequantGemmDynamicM T-padding driver (rows past T are zero and sliced
// away) -- here rows >= T are predicated, never read or written.
//
// Work decomposition (gfx950 specific):
//   * A workgroup is kW compute waves plus one producer wave.  Compute wave w
//     owns 16 output rows and a block of 16 * MT tokens and walks one K slice
//     in steps of 128.  In a step, lane (r = l % 16, q = l / 16) loads the 32
//     codes k0 + 32q .. k0 + 32q + 31 of row r with one 128-bit load and
//     dequantises them in registers (float32 s * q + b, rounded to bf16):
//     word s of that chunk is the B operand of MFMA sub-step s.  Sub-step s
//     therefore covers the k set {k0 + 32q + 8s + j : q < 4, j < 8}; the
//     matching A operand (the activations) is read from LDS with the same k
//     set, so the sum over k is unchanged.
//   * Weights never pass through LDS.  Each wave keeps D steps of code loads
//     in flight in a register ring (raw buffer loads: rows past n_out and
//     chunks past k_in read as zero without touching memory, so every load is
//     unconditional).
//   * The scales and biases of a wave's 16 rows over its K slice are copied
//     into LDS once, by direct buffer-to-LDS loads issued behind the first
//     ring fill, and read from there in every step: per-step 2-byte loads
//     from 16 scattered rows cost more memory-pipeline work than the code
//     loads themselves.  Those loads move whole dwords, so the table needs
//     dword-aligned rows (float32 scales, or bf16 with an even number of
//     groups per row and 4-byte aligned arrays); otherwise every step loads
//     its scales and biases directly.
//   * The 16 * MT x 128 activation tile of each step is staged in an
//     NBUF-deep LDS ring (one barrier per step) by the producer wave with
//     direct buffer-to-LDS loads, and shared by the compute waves, which
//     cover different rows.  Loads complete in issue order as far as the
//     wait counters go, so an activation load issued by a compute wave behind
//     its weight ring would drain that ring; the producer keeps the two
//     streams apart.
//   * Split K: with 16-row tiles a 17408-row matrix gives only 1088 waves,
//     about one per SIMD, which can neither hide memory latency nor spread
//     evenly over 1024 SIMDs.  ksplit workgroups therefore share a row block,
//     each summing one K slice into a float32 partial plane; a second kernel
//     adds the planes into Y.  With ksplit == 1 the GEMM writes Y directly.
//   * Output: accumulator element i of lane l is token 4 (l / 16) + i,
//     output row l % 16 of the 16 x 16 tile, so 16 lanes store 16
//     consecutive outputs of one token row.

#include <algorithm>
#include <climits>

#include "kernels.h"

namespace qint4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int KS = 128;           // k per step
constexpr int kW = 4;             // compute waves per workgroup
constexpr uint32_t kOOR = 0x80000000u;
constexpr int64_t kMaxTableBytes = 32 * 1024;  // scale + bias tables of one workgroup

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
// The word masked with 0x000F000F holds codes (n, n + 4) as the f16
// subnormals q 2^-24, masked with 0x00F000F0 codes (n + 1, n + 5) as
// 16 q 2^-24; v_fma_mix_f32 against the scale times 2^24 (s24) or 2^20 (s20)
// gives fmaf(s, q, b) exactly (scales below 2^104 in magnitude).
__device__ __forceinline__ bf16x8_t dequant8(uint32_t w, float s24, float s20, float b) {
  const uint32_t w8 = w >> 8;
  const f16x2_t p0 = __builtin_bit_cast(f16x2_t, w & 0x000F000Fu);   // codes 0, 4
  const f16x2_t p1 = __builtin_bit_cast(f16x2_t, w & 0x00F000F0u);   // 1, 5 (times 16)
  const f16x2_t p2 = __builtin_bit_cast(f16x2_t, w8 & 0x000F000Fu);  // 2, 6
  const f16x2_t p3 = __builtin_bit_cast(f16x2_t, w8 & 0x00F000F0u);  // 3, 7 (times 16)
  uint4 r;
  r.x = pack2(fmaf((float)p0.x, s24, b), fmaf((float)p1.x, s20, b));
  r.y = pack2(fmaf((float)p2.x, s24, b), fmaf((float)p3.x, s20, b));
  r.z = pack2(fmaf((float)p0.y, s24, b), fmaf((float)p1.y, s20, b));
  r.w = pack2(fmaf((float)p2.y, s24, b), fmaf((float)p3.y, s20, b));
  return __builtin_bit_cast(bf16x8_t, r);
}

struct WStep {
  uint4 q;
  uint32_t s, b;  // unused when the scales and biases come from LDS
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

// The groups of a K slice as its LDS table holds them: upr dwords per row
// starting at group g0e; bf16 tables start at an even group so that every
// row is whole dwords.
struct SliceGroups {
  int g0e;
  int upr;
};

template <int SBT>
__device__ __forceinline__ SliceGroups slice_groups(int k_begin, int k_end, int log2_group) {
  const int g0 = k_begin >> log2_group;
  const int g1 = ((k_end - 1) >> log2_group) + 1;
  SliceGroups r;
  if constexpr (SBT == 1) {
    r.g0e = g0 & ~1;
    r.upr = (((g1 + 1) & ~1) - r.g0e) / 2;
  } else {
    r.g0e = g0;
    r.upr = g1 - g0;
  }
  return r;
}

template <int MT, int D, int NBUF, int SBT, bool SBL>
__global__ void __launch_bounds__((kW + 1) * 64) qgemm_stream_kernel(const GemmParams p) {
  constexpr int TOK = 16 * MT;                       // tokens per workgroup
  constexpr int NBLK = TOK / 4;                      // producer load instructions per step (4 rows each)
  constexpr uint32_t SBB = SBT == 1 ? 2 : 4;
  constexpr int TILE = TOK * KS;                     // bf16 elements of one activation tile
  constexpr int NT = (kW + 1) * 64;
  static_assert(NBUF >= 2, "activation ring");

  // activation tile ring (NBUF * TILE bf16), then per compute wave a scale
  // table and a bias table of p.sb_tab_dw dwords each
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // token block fastest, then K slice, then row block: workgroups launched
  // together read neighbouring slices of the same weight rows
  const int tb = blockIdx.x % p.m_tiles;
  const int rest = blockIdx.x / p.m_tiles;
  const int ksl = rest % p.ksplit;
  const int nb = rest / p.ksplit;
  const int64_t t0 = (int64_t)tb * TOK;
  const int nsteps = (p.k_in + KS - 1) / KS;
  const int jb = ksl * p.split_steps;                // first step of this slice
  const int nst = min(p.split_steps, nsteps - jb);   // its steps (>= 1: the host sizes ksplit)
  // The K loop runs a whole number of D-step rounds, so no branch sits inside
  // a round (a branch around a step makes the compiler wait for every load in
  // flight); steps past the slice load out-of-range zeros and add nothing.
  const int spw = (nst + D - 1) / D * D;

  // Zero the activation ring once: lanes of a tile that fall past T or k_in
  // then hold finite values whatever the out-of-range loads leave, and those
  // only meet zero weights (k past k_in) or outputs that are never stored.
  for (int i = threadIdx.x; i < NBUF * TILE / 8; i += NT)
    reinterpret_cast<uint4 *>(xs)[i] = make_uint4(0, 0, 0, 0);
  lds_barrier();

  if (wave == kW) {
    // ---- producer wave: the activation tile of each step goes straight
    // from memory into LDS (buffer loads with an LDS destination: no
    // registers), NBUF - 1 steps ahead.  Its loads are the only ones it waits
    // for, so the compute waves' weight rings are never drained by them.
    const __amdgpu_buffer_rsrc_t rx = rsrc(p.x, 0x7FFFFFF0u);
    auto issue = [&](int j) {  // step j of the slice -> buffer j % NBUF
      uint16_t *base = xs + (j % NBUF) * TILE;
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int t = b * 4 + (lane >> 4);
        const int g = (lane & 15) ^ (t & 15);       // lane i writes position i of the block
        const int64_t tok = t0 + t;
        const int k = (jb + j) * KS + 8 * g;
        const bool ok = tok < p.T && k < p.k_in && j < nst;
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
  const int row0 = (nb * kW + wave) * 16;            // first row of this wave
  const uint32_t kwb = (uint32_t)p.k_in / 2;         // code bytes per row
  const uint32_t gpr = (uint32_t)p.k_in >> p.log2_group;
  const uint32_t sbrow = gpr * SBB;
  const __amdgpu_buffer_rsrc_t rc = rsrc(p.codes, (uint32_t)p.n_out * kwb);
  const __amdgpu_buffer_rsrc_t rs = rsrc(p.scales, (uint32_t)p.n_out * sbrow);
  const __amdgpu_buffer_rsrc_t rb = rsrc(p.biases, (uint32_t)p.n_out * sbrow);

  // per-lane byte offsets of the code / scale loads (rows past n_out fall
  // outside the resources and read as zero)
  const uint32_t c_lane = (uint32_t)(row0 + r) * kwb + (uint32_t)q * 16 + (uint32_t)jb * 64;
  const uint32_t s_lane = (uint32_t)(row0 + r) * sbrow;
  const int cpr = p.k_in / 32;

  auto load_w = [&](int j, WStep &st) {  // step j of the slice
    const int c = (jb + j) * 4 + q;       // this lane's 32-code chunk
    const bool ok = j < nst && c < cpr;
    st.q = ld128(rc, ok ? c_lane + (uint32_t)j * 64 : kOOR);
    if constexpr (!SBL) {
      const uint32_t os = ok ? s_lane + ((((uint32_t)c * 32) >> p.log2_group) * SBB) : kOOR;
      st.s = ldsb<SBT>(rs, os);
      st.b = ldsb<SBT>(rb, os);
    }
  };

  f32x4_t acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  WStep ring[D];
#pragma unroll
  for (int u = 0; u < D; ++u) load_w(u, ring[u]);

  const SliceGroups sg = slice_groups<SBT>(jb * KS, min(p.k_in, (jb + nst) * KS), p.log2_group);
  unsigned char *tab = reinterpret_cast<unsigned char *>(xs + NBUF * TILE) + (size_t)wave * 2 * p.sb_tab_dw * 4;
  if constexpr (SBL) {
    // Scale and bias tables of this wave: 16 rows x upr dwords each, dense,
    // so dword e of a table is lane e % 64 of load instruction e / 64 (the
    // region holds whole instructions: p.sb_tab_dw is a multiple of 64 and at
    // least 16 * upr).  Issued behind the ring fill, whose first step waits
    // for them anyway.
    const int total = 16 * sg.upr;
    for (int i = 0; i * 64 < total; ++i) {
      const int e = i * 64 + lane;
      const int row = e / sg.upr, u = e - row * sg.upr;
      const uint32_t off =
          e < total ? (uint32_t)(row0 + row) * sbrow + (uint32_t)sg.g0e * SBB + (uint32_t)u * 4 : kOOR;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void *)(tab + i * 256), 4, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void *)(tab + p.sb_tab_dw * 4 + i * 256), 4, off, 0, 0, 0);
    }
    wait_vmcnt<0>();  // tables (and the ring fill ahead of them) have landed
  }
  lds_barrier();  // the first activation tiles are in LDS

  const unsigned char *tab_s = tab + r * sg.upr * 4;
  const unsigned char *tab_b = tab_s + p.sb_tab_dw * 4;

  for (int j0 = 0; j0 < spw; j0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int j = j0 + u;
      float sc, bi;
      if constexpr (SBL) {
        // table entry of this lane's chunk; zero past the slice and k_in
        const int c = (jb + j) * 4 + q;
        const bool ok = j < nst && c < cpr;
        const int gi = ok ? (((c * 32) >> p.log2_group) - sg.g0e) * (int)SBB : 0;
        uint32_t sbits, bbits;
        if constexpr (SBT == 1) {
          sbits = *reinterpret_cast<const uint16_t *>(tab_s + gi);
          bbits = *reinterpret_cast<const uint16_t *>(tab_b + gi);
        } else {
          sbits = *reinterpret_cast<const uint32_t *>(tab_s + gi);
          bbits = *reinterpret_cast<const uint32_t *>(tab_b + gi);
        }
        sc = ok ? sbval<SBT>(sbits) : 0.f;
        bi = ok ? sbval<SBT>(bbits) : 0.f;
      } else {
        sc = sbval<SBT>(ring[u].s);
        bi = sbval<SBT>(ring[u].b);
      }
      // dequantise this step's weights: B operands of the four sub-steps
      bf16x8_t bw[4];
      const uint32_t wd[4] = {ring[u].q.x, ring[u].q.y, ring[u].q.z, ring[u].q.w};
      const float s24 = sc * 0x1p24f, s20 = sc * 0x1p20f;
#pragma unroll
      for (int s = 0; s < 4; ++s) bw[s] = dequant8(wd[s], s24, s20, bi);
      load_w(j + D, ring[u]);  // refill the slot just consumed
      const uint16_t *xt = xs + (j % NBUF) * TILE;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(xt + xs_index(m * 16 + r, 4 * q + s));
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw[s], acc[m], 0, 0, 0);
        }
      lds_barrier();
    }
  }

  // epilogue: Y (one slice) or this slice's float32 partial plane
  const int o = row0 + r;
  if (o >= p.n_out) return;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + m * 16 + 4 * q + i;
      if (t >= p.T) continue;
      if (p.ksplit > 1)
        p.part[((int64_t)ksl * p.T + t) * p.n_out + o] = acc[m][i];
      else if (p.y_bf16)
        reinterpret_cast<__bf16 *>(p.y)[t * p.ldy + o] = (__bf16)acc[m][i];
      else
        reinterpret_cast<float *>(p.y)[t * p.ldy + o] = acc[m][i];
    }
}

// Y[t][o] = sum over slices of part[slice][t][o]; one thread per 8 outputs.
// The planes are read eight at a time with every load issued before the
// first add, so a thread waits for memory once per eight planes.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float *__restrict__ part, int ksplit,
                                                            int64_t T, int n_out, void *y, int64_t ldy,
                                                            int y_bf16) {
  const int64_t n8 = (int64_t)n_out / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * n8) return;
  const int64_t t = i / n8;
  const int o = (int)(i - t * n8) * 8;
  const int64_t plane = T * (int64_t)n_out;
  const float *src = part + t * n_out + o;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int k0 = 0; k0 < ksplit; k0 += 8) {
    float4 v[8][2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 *q = reinterpret_cast<const float4 *>(src + (int64_t)min(k0 + k, ksplit - 1) * plane);
      v[k][0] = q[0];
      v[k][1] = q[1];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k0 + k >= ksplit) break;
      acc[0] += v[k][0].x;
      acc[1] += v[k][0].y;
      acc[2] += v[k][0].z;
      acc[3] += v[k][0].w;
      acc[4] += v[k][1].x;
      acc[5] += v[k][1].y;
      acc[6] += v[k][1].z;
      acc[7] += v[k][1].w;
    }
  }
  if (y_bf16) {
    __bf16 *d = reinterpret_cast<__bf16 *>(y) + t * ldy + o;
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = (__bf16)acc[j];
  } else {
    float *d = reinterpret_cast<float *>(y) + t * ldy + o;
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = acc[j];
  }
}

constexpr int nbuf_for(int mt) { return mt == 4 ? 2 : 3; }

template <int MT, int D, int SBT, bool SBL>
hipError_t launch_cfg(const GemmParams &p, size_t lds, size_t grid, hipStream_t stream) {
  auto kern = qgemm_stream_kernel<MT, D, nbuf_for(MT), SBT, SBL>;
  // opt in to the LDS limit (once per device)
  if (lds > 64 * 1024) {
    hipError_t e = lds_opt_in(reinterpret_cast<const void *>(kern), kMaxLds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3((kW + 1) * 64), lds, stream, p);
  return hipGetLastError();
}

template <int MT, int SBT>
hipError_t launch_d(const GemmParams &p, int depth, size_t lds, size_t grid, hipStream_t stream) {
  switch (depth) {
    case 4: return launch_cfg<MT, 4, SBT, true>(p, lds, grid, stream);
    case 5: return launch_cfg<MT, 5, SBT, true>(p, lds, grid, stream);
    case 8: return launch_cfg<MT, 8, SBT, true>(p, lds, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int MT>
hipError_t launch_mt(const GemmParams &p, const StreamPlan &plan, size_t lds, size_t grid,
                     hipStream_t stream) {
  if (plan.sb_lds)
    return p.sb_bf16 ? launch_d<MT, 1>(p, plan.depth, lds, grid, stream)
                     : launch_d<MT, 0>(p, plan.depth, lds, grid, stream);
  if (plan.depth != 8) return hipErrorInvalidValue;  // the direct scale path is built for D = 8 only
  return p.sb_bf16 ? launch_cfg<MT, 8, 1, false>(p, lds, grid, stream)
                   : launch_cfg<MT, 8, 0, false>(p, lds, grid, stream);
}

// Table dwords per wave and array for a slice of split_steps steps: the
// groups a slice touches plus one at each end (the even-group start of bf16
// tables), rounded up to whole 64-lane load instructions.
int64_t table_dw(int64_t split_steps, int log2_group, int sbb) {
  const int64_t groups = ((split_steps * KS) >> log2_group) + 2;
  const int64_t upr = (groups * sbb + 3) / 4;
  return (16 * upr + 63) / 64 * 64;
}

}  // namespace

StreamPlan plan_gemm_stream(int64_t T, int64_t n_out, int64_t k_in, int log2_group, int sb_bf16,
                            bool sb_dwords, int n_cu, int64_t ws_bytes) {
  StreamPlan pl{};
  pl.mt = T <= 16 ? 1 : T <= 32 ? 2 : 4;
  const int64_t nsteps = (k_in + KS - 1) / KS;
  const int64_t blocks = (n_out + kW * 16 - 1) / (kW * 16);
  const int64_t m_tiles = (T + 16 * pl.mt - 1) / (16 * pl.mt);
  // As many slices as keep every workgroup resident in one round: a CU holds
  // 4 workgroups of kW + 1 waves at up to 96 VGPRs (5 waves per SIMD), i.e.
  // 16 compute waves, while LDS allows; a second, partial round of
  // workgroups would double the time of the CUs that run it.  At least 4
  // steps per slice, and no more slices than the workspace holds.
  const int64_t x_lds = (int64_t)nbuf_for(pl.mt) * 16 * pl.mt * KS * 2;
  const int64_t units = blocks * m_tiles;
  int64_t S = 1;
  for (int64_t s = 2; s <= nsteps / 4; ++s) {
    const int64_t per = (nsteps + s - 1) / s;
    const int64_t lds = x_lds + (int64_t)kW * 2 * table_dw(per + 7, log2_group, sb_bf16 ? 2 : 4) * 4;
    const int64_t cap = std::min<int64_t>(4, (int64_t)kMaxLds / lds);
    if (units * s > cap * n_cu) break;
    S = s;
  }
  if (ws_bytes >= 0) S = std::min<int64_t>(S, std::max<int64_t>(1, ws_bytes / (T * n_out * 4)));
  // prefetch depth: the shortest padded slice, then the deepest ring
  const int64_t per = (nsteps + S - 1) / S;
  int64_t best = INT64_MAX;
  for (int d : {8, 5, 4}) {
    const int64_t ss = (per + d - 1) / d * d;
    if (ss < best) {
      best = ss;
      pl.depth = d;
    }
  }
  pl.split_steps = (int)best;
  pl.ksplit = (int)((nsteps + best - 1) / best);
  pl.sb_lds = sb_dwords && (int64_t)kW * 2 * table_dw(best, log2_group, sb_bf16 ? 2 : 4) * 4 <= kMaxTableBytes;
  if (!pl.sb_lds) pl.depth = 8;  // the direct scale path is built for D = 8
  return pl;
}

size_t gemm_stream_ws_bytes(const StreamPlan &plan, int64_t T, int64_t n_out) {
  return plan.ksplit > 1 ? (size_t)plan.ksplit * (size_t)T * (size_t)n_out * 4 : 0;
}

hipError_t launch_gemm_stream(const GemmParams &p_in, const StreamPlan &plan, hipStream_t stream) {
  GemmParams p = p_in;
  const int TOK = 16 * plan.mt;
  p.m_tiles = (int)((p.T + TOK - 1) / TOK);
  p.n_tiles = (p.n_out + kW * 16 - 1) / (kW * 16);
  p.ksplit = plan.ksplit;
  p.split_steps = plan.split_steps;
  p.sb_tab_dw = plan.sb_lds ? (int32_t)table_dw(plan.split_steps, p.log2_group, p.sb_bf16 ? 2 : 4) : 0;
  if (p.ksplit > 1 && !p.part) return hipErrorInvalidValue;
  const size_t grid = (size_t)p.m_tiles * p.ksplit * p.n_tiles;
  const size_t lds = (size_t)nbuf_for(plan.mt) * TOK * KS * 2 + (size_t)kW * 2 * p.sb_tab_dw * 4;
  if (lds > (size_t)kMaxLds) return hipErrorInvalidValue;
  hipError_t e;
  switch (plan.mt) {
    case 1: e = launch_mt<1>(p, plan, lds, grid, stream); break;
    case 2: e = launch_mt<2>(p, plan, lds, grid, stream); break;
    case 4: e = launch_mt<4>(p, plan, lds, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || p.ksplit == 1) return e;
  const int64_t n = p.T * (p.n_out / 8);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     (const float *)p.part, p.ksplit, p.T, p.n_out, p.y, p.ldy, p.y_bf16);
  return hipGetLastError();
}

}  // namespace qint4
