// qgemm.hip -- prefill int4 dequant GEMM on gfx950 bf16 MFMA.
//
//   Y[t][o] = sum_k bf16(s[o][k/g] * q[o][k] + b[o][k/g]) * X[t][k],  t < T
//
// Source: thewafflehaus/FFAI pull 9, "Everything Bagel", commit adding the
// dequantGemmDynamicM T-padding driver (T rounded up to a multiple of 32 with
// zero rows, first T rows kept), and pull 14, commit adding the outDim % 32
// guard for that GEMM.  Here the padding is virtual: X rows >= T load as zero
// and Y rows >= T are never stored, so neither buffer is copied or padded.
//
// Tiling (gfx950): a workgroup owns a BM x BN tile of Y and walks K in steps
// of 64 (one 64-group, or two 32-groups).  Per step every thread loads 32
// codes of one W row (a 128-bit load) with that group's scale and bias,
// dequantises them in float32, rounds to bf16 (v_cvt_pk_bf16_f32,
// round-to-nearest-even) and writes them to LDS; the X tile is copied to LDS
// as bf16.  Waves then run v_mfma_f32_32x32x16_bf16 on 32x32 sub-tiles with
// float32 accumulators.  The next step's global loads are issued before the
// MFMAs of the current step so that HBM latency overlaps the math; the
// barriers order LDS only, so they do not wait for those loads.

#include "kernels.h"

namespace qint4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements): spreads rows over banks

// Workgroup barrier that orders LDS only: __syncthreads() would also wait for
// every outstanding global load, including the next step's prefetch.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// 8 codes of one word -> 8 bf16 weights (k order), as a uint4.
__device__ __forceinline__ uint4 dequant_word(uint32_t w, float s, float b) {
  uint32_t lo = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6 in bytes 0..3
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
  asm("" : "+v"(lo), "+v"(hi));
  uint4 r;
  r.x = pack_bf16x2(fmaf(s, (float)(lo & 0xFFu), b), fmaf(s, (float)(hi & 0xFFu), b));
  r.y = pack_bf16x2(fmaf(s, (float)((lo >> 8) & 0xFFu), b), fmaf(s, (float)((hi >> 8) & 0xFFu), b));
  r.z = pack_bf16x2(fmaf(s, (float)((lo >> 16) & 0xFFu), b), fmaf(s, (float)((hi >> 16) & 0xFFu), b));
  r.w = pack_bf16x2(fmaf(s, (float)(lo >> 24), b), fmaf(s, (float)(hi >> 24), b));
  return r;
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM * WN * 64) qgemm_kernel(const GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA tiles per wave
  constexpr int WCH = (2 * BN + NT - 1) / NT;  // W chunk loads per thread per step
  constexpr int XCH = (8 * BM + NT - 1) / NT;  // X 16-byte loads per thread per step
  static_assert(FM >= 1 && FN >= 1, "tile");

  __shared__ __attribute__((aligned(16))) uint16_t sx[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sw[BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // tile order: m fastest, so workgroups launched together share W columns
  const int mt = blockIdx.x % p.m_tiles;
  const int nt = blockIdx.x / p.m_tiles;
  const int64_t m0 = (int64_t)mt * BM;
  const int n0 = nt * BN;

  const int cpr = p.k_in / 32;                   // 32-code chunks per W row
  const int64_t gpr = (int64_t)p.k_in >> p.log2_group;
  const int nsteps = (p.k_in + BK - 1) / BK;
  const int sbb = p.sb_bf16 ? 2 : 4;

  // per-thread load assignments
  // (threads past the tile's chunk count idle: w_act / x_act false)
  int w_row[WCH], w_half[WCH];
  bool w_act[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int t = tid + i * NT;
    w_act[i] = t < 2 * BN;
    w_row[i] = w_act[i] ? (t >> 1) : 0;
    w_half[i] = t & 1;
  }
  int x_row[XCH], x_seg[XCH];
  bool x_act[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int t = tid + i * NT;
    x_act[i] = t < 8 * BM;
    x_row[i] = x_act[i] ? (t >> 3) : 0;
    x_seg[i] = t & 7;
  }

  uint4 wq[WCH];
  float ws_[WCH], wb_[WCH];
  uint4 xq[XCH];

  auto load_step = [&](int kt) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int o = n0 + w_row[i];
      const int kc = kt * 2 + w_half[i];
      const bool ok = w_act[i] && (o < p.n_out) && (kc < cpr);
      if (ok) {
        wq[i] = reinterpret_cast<const uint4 *>(p.codes)[(int64_t)o * (cpr) + kc];
        const int64_t gi = (int64_t)o * gpr + (((int64_t)kc * 32) >> p.log2_group);
        if (sbb == 2) {
          ws_[i] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p.scales)[gi] << 16);
          wb_[i] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p.biases)[gi] << 16);
        } else {
          ws_[i] = reinterpret_cast<const float *>(p.scales)[gi];
          wb_[i] = reinterpret_cast<const float *>(p.biases)[gi];
        }
      } else {
        wq[i] = make_uint4(0, 0, 0, 0);
        ws_[i] = 0.f;
        wb_[i] = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int64_t t = m0 + x_row[i];
      const int k = kt * BK + x_seg[i] * 8;
      if (x_act[i] && t < p.T && k < p.k_in)
        xq[i] = *reinterpret_cast<const uint4 *>(p.x + t * p.ldx + k);
      else
        xq[i] = make_uint4(0, 0, 0, 0);
    }
  };

  auto store_step = [&]() {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      if (!w_act[i]) continue;
      uint16_t *dst = sw + w_row[i] * LDK + w_half[i] * 32;
      const uint32_t w4[4] = {wq[i].x, wq[i].y, wq[i].z, wq[i].w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<uint4 *>(dst + jj * 8) = dequant_word(w4[jj], ws_[i], wb_[i]);
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i)
      if (x_act[i]) *reinterpret_cast<uint4 *>(sx + x_row[i] * LDK + x_seg[i] * 8) = xq[i];
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  load_step(0);
  for (int kt = 0; kt < nsteps; ++kt) {
    store_step();
    lds_barrier();
    if (kt + 1 < nsteps) load_step(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int koff = kk * 16 + (lane >> 5) * 8;
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int a = 0; a < FM; ++a)
        af[a] = *reinterpret_cast<const bf16x8_t *>(sx + (wm * TM + a * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
      for (int b = 0; b < FN; ++b)
        bfr[b] = *reinterpret_cast<const bf16x8_t *>(sw + (wn * TN + b * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
    lds_barrier();
  }

  // epilogue: accumulator element v of lane l is row 8*(v/4) + 4*(l/32) + v%4,
  // column l%32 of the 32x32 sub-tile
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      const int col = n0 + wn * TN + b * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * TM + a * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < p.T && col < p.n_out) {
          if (p.y_bf16)
            reinterpret_cast<__bf16 *>(p.y)[row * p.ldy + col] = (__bf16)acc[a][b][v];
          else
            reinterpret_cast<float *>(p.y)[row * p.ldy + col] = acc[a][b][v];
        }
      }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_tile(GemmParams p, hipStream_t stream) {
  p.m_tiles = (int)((p.T + BM - 1) / BM);
  p.n_tiles = (p.n_out + BN - 1) / BN;
  const int64_t grid = (int64_t)p.m_tiles * p.n_tiles;
  hipLaunchKernelGGL((qgemm_kernel<BM, BN, WM, WN>), dim3((unsigned)grid), dim3(WM * WN * 64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

// Tile by T (measured on MI355X at N = 17408, K = 5120): narrow tiles keep
// more workgroups per CU for short T; 8-wave 128x128 tiles up to T = 2048.
hipError_t launch_gemm(const GemmParams &p, hipStream_t stream) {
  if (p.T <= 32) return launch_tile<32, 64, 1, 2>(p, stream);
  if (p.T <= 64) return launch_tile<64, 64, 2, 2>(p, stream);
  if (p.T <= 256) return launch_tile<128, 64, 2, 2>(p, stream);
  if (p.T <= 2048) return launch_tile<128, 128, 2, 4>(p, stream);
  return launch_tile<128, 128, 2, 2>(p, stream);
}

}  // namespace qint4
