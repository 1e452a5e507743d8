// qgemm.hip -- prefill int4 dequant GEMM on gfx950 bf16 MFMA, LDS-tiled
// (the T > 64 path of qgemm_int4_padT, and every qgemm_int4_padT_multi call;
// qgemm_stream.hip serves qgemm_int4_padT at T <= 64).
//
//   Y_i[t][o] = sum_k bf16(s_i[o][k/g] * q_i[o][k] + b_i[o][k/g]) * X[t][k],  t < T
//
// Sources: thewafflehaus/FFAI pull 9, "Everything Bagel", commit adding the
// dequantGemmDynamicM T-padding driver (T rounded up to a multiple of 32 with
// zero rows, first T rows kept), and pull 14, commit adding the outDim % 32
// guard for that GEMM and the batched QKV / batched-4 projections sharing one
// input in one launch (M > 1: separate outputs).  Here the padding is
// virtual: X rows >= T load as zero and Y rows >= T are never stored, so
// neither buffer is copied or padded.
//
// Tiling (gfx950): a workgroup owns a BM x BN tile of one matrix's output (the
// weight tiles of all matrices of a call form one grid) and walks K in steps
// of 64 (one 64-group, or two 32-groups).  Per step every thread loads 32
// codes of one W row (a 128-bit load), dequantises them in float32 with that
// group's scale and bias, rounds to bf16 (v_cvt_pk_bf16_f32,
// round-to-nearest-even) and writes them to LDS; the X tile is copied to LDS
// as bf16.  Waves then run v_mfma_f32_32x32x16_bf16 on 32x32 sub-tiles with
// float32 accumulators.
//   * Tile order: workgroups are dealt to the eight XCDs round-robin, and each
//     XCD takes a contiguous range of a grouped order (4 token tiles per
//     weight tile, then the next weight tile), so the tiles resident on an
//     XCD share their weight and activation blocks in its L2 (T = 1024:
//     302 -> 267 us, T = 4096: 982 -> 893 us at N = 17408, K = 5120).
//   * The global loads of PF steps are kept in flight in a register ring, so
//     HBM latency is covered by PF steps of MFMA work rather than one; the
//     barriers order LDS only and never wait for those loads.  PF = 2 (3
//     and 4 measured 1-6% slower at N = 17408, K = 5120).
//   * Every load is a raw buffer load: rows past T or n_out and chunks past
//     k_in read as zero without touching memory, so no load sits behind a
//     branch (a branch around a load in the ring would make the compiler wait
//     for every load in flight).
//   * The scales and biases of the workgroup's BN rows for the whole K range
//     are copied into LDS once, with coalesced loads, when they fit next to
//     the tiles: per-step 2-byte loads from BN scattered rows otherwise cost
//     more memory-pipeline work than the code loads.

#include "kernels.h"

namespace qint4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements): spreads rows over banks
constexpr uint32_t kOOR = 0x80000000u;

// Workgroup barrier that orders LDS only: __syncthreads() would also wait for
// every outstanding global load, including the prefetched steps.
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

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// 8 codes of one word -> 8 bf16 weights (k order), as a uint4.  The word
// masked with 0x000F000F holds codes (n, n + 4) as the f16 subnormals q 2^-24,
// masked with 0x00F000F0 codes (n + 1, n + 5) as 16 q 2^-24; v_fma_mix_f32
// against the scale times 2^24 (s24) or 2^20 (s20) gives fmaf(s, q, b)
// exactly (scales below 2^104 in magnitude), then RNE to bf16.
__device__ __forceinline__ uint4 dequant_word(uint32_t w, float s24, float s20, float b) {
  const uint32_t w8 = w >> 8;
  const f16x2_t p0 = __builtin_bit_cast(f16x2_t, w & 0x000F000Fu);   // codes 0, 4
  const f16x2_t p1 = __builtin_bit_cast(f16x2_t, w & 0x00F000F0u);   // 1, 5 (times 16)
  const f16x2_t p2 = __builtin_bit_cast(f16x2_t, w8 & 0x000F000Fu);  // 2, 6
  const f16x2_t p3 = __builtin_bit_cast(f16x2_t, w8 & 0x00F000F0u);  // 3, 7 (times 16)
  uint4 r;
  r.x = pack_bf16x2(fmaf((float)p0.x, s24, b), fmaf((float)p1.x, s20, b));
  r.y = pack_bf16x2(fmaf((float)p2.x, s24, b), fmaf((float)p3.x, s20, b));
  r.z = pack_bf16x2(fmaf((float)p0.y, s24, b), fmaf((float)p1.y, s20, b));
  r.w = pack_bf16x2(fmaf((float)p2.y, s24, b), fmaf((float)p3.y, s20, b));
  return r;
}

// SBL: the scales and biases of the BN rows are staged in dynamic LDS.
template <int BM, int BN, int WM, int WN, int PF, bool SBL>
__global__ void __launch_bounds__(WM * WN * 64) qgemm_kernel(const GemmMultiParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA tiles per wave
  constexpr int WCH = (2 * BN + NT - 1) / NT;  // W chunk loads per thread per step
  constexpr int XCH = (8 * BM + NT - 1) / NT;  // X 16-byte loads per thread per step
  static_assert(FM >= 1 && FN >= 1, "tile");

  __shared__ __attribute__((aligned(16))) uint16_t sx[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sw[BN * LDK];
  // the scales then the biases of this workgroup's BN rows for the whole K
  // range (dynamic LDS, 2 * BN * sbrow bytes) when SBL
  extern __shared__ __attribute__((aligned(16))) unsigned char sbtab[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Tile order: workgroups are dealt to the eight XCDs round-robin (workgroup
  // b runs on XCD b % 8); each XCD takes a contiguous range of a grouped order
  // (GROUP_M token tiles per weight tile, then the next weight tile), so the
  // tiles resident on one XCD share weight and activation blocks in its L2.
  constexpr int GROUP_M = 4;
  const int bid = blockIdx.x;
  const int sq = (bid & 7) * p.per_xcd + (bid >> 3);
  if (sq >= p.tiles) return;
  const int grp = sq / (GROUP_M * p.n_tiles);
  const int rr = sq - grp * GROUP_M * p.n_tiles;
  const int gsz = min(GROUP_M, p.m_tiles - grp * GROUP_M);
  const int nt_all = rr / gsz;
  const int mt = grp * GROUP_M + (rr - nt_all * gsz);
  int mi = 0;
#pragma unroll
  for (int i = 1; i < kMaxMats; ++i) mi += nt_all >= p.m[i].tile0 ? 1 : 0;
  const GemmMat &M = p.m[mi];
  const int64_t m0 = (int64_t)mt * BM;
  const int n0 = (nt_all - M.tile0) * BN;

  const int cpr = p.k_in / 32;                   // 32-code chunks per W row
  const uint32_t gpr = (uint32_t)p.k_in >> p.log2_group;
  const uint32_t sbb = p.sb_bf16 ? 2 : 4;
  const uint32_t kwb = (uint32_t)p.k_in / 2;     // code bytes per row
  const uint32_t sbrow = gpr * sbb;              // scale (= bias) bytes per row
  // K steps rounded up to whole prefetch rounds; steps past the end load
  // out-of-range zeros and add nothing
  const int nsteps = ((p.k_in + BK - 1) / BK + PF - 1) / PF * PF;

  const __amdgpu_buffer_rsrc_t rc = rsrc(M.codes, (uint32_t)M.n_out * kwb);
  const __amdgpu_buffer_rsrc_t rs = rsrc(M.scales, (uint32_t)M.n_out * sbrow);
  const __amdgpu_buffer_rsrc_t rb = rsrc(M.biases, (uint32_t)M.n_out * sbrow);
  // X from this tile's first row on: rows past T lie outside the resource
  const int64_t rows_here = p.T - m0 < BM ? p.T - m0 : BM;
  const __amdgpu_buffer_rsrc_t rx =
      rsrc(p.x + m0 * p.ldx, (uint32_t)(((rows_here - 1) * p.ldx + p.k_in) * 2));

  if constexpr (SBL) {
    // one coalesced pass over the contiguous BN * sbrow bytes of each array
    // (16-, 4- or 2-byte units, whichever the alignment allows); rows past
    // n_out read as zero
    const uint32_t bytes = (uint32_t)BN * sbrow;
    const uint32_t base = (uint32_t)n0 * sbrow;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const __amdgpu_buffer_rsrc_t r = a ? rb : rs;
      const uintptr_t al = reinterpret_cast<uintptr_t>(a ? M.biases : M.scales) | base | bytes;
      unsigned char *dst = sbtab + (uint32_t)a * bytes;
      if ((al & 15) == 0) {
        for (uint32_t j = tid * 16; j < bytes; j += NT * 16)
          *reinterpret_cast<uint4 *>(dst + j) = ld128(r, base + j);
      } else if ((al & 3) == 0) {
        for (uint32_t j = tid * 4; j < bytes; j += NT * 4)
          *reinterpret_cast<uint32_t *>(dst + j) = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, base + j, 0, 0);
      } else {
        for (uint32_t j = tid * 2; j < bytes; j += NT * 2)
          *reinterpret_cast<uint16_t *>(dst + j) = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, base + j, 0, 0);
      }
    }
    lds_barrier();
  }

  // per-thread load assignments (threads past the tile's chunk count idle)
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

  struct Step {
    uint4 wq[WCH];
    uint32_t ws[WCH], wb[WCH];
    uint4 xq[XCH];
  };
  auto load_step = [&](int kt, Step &st) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int kc = kt * 2 + w_half[i];
      const bool ok = w_act[i] && kc < cpr;  // rows past n_out fall outside the resource
      const uint32_t o = (uint32_t)(n0 + w_row[i]);
      st.wq[i] = ld128(rc, ok ? o * kwb + (uint32_t)kc * 16 : kOOR);
      if constexpr (SBL) {  // read from the LDS table when the step is stored
        st.ws[i] = 0;
        st.wb[i] = 0;
      } else {
        const uint32_t os = ok ? o * sbrow + (((uint32_t)kc * 32) >> p.log2_group) * sbb : kOOR;
        if (p.sb_bf16) {
          st.ws[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, os, 0, 0) << 16;
          st.wb[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, os, 0, 0) << 16;
        } else {
          st.ws[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, 0);
          st.wb[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rb, os, 0, 0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int k = kt * BK + x_seg[i] * 8;
      const bool ok = x_act[i] && x_row[i] < rows_here && k < p.k_in;
      st.xq[i] = ld128(rx, ok ? (uint32_t)((x_row[i] * p.ldx + k) * 2) : kOOR);
    }
  };

  auto store_step = [&](int kt, const Step &st) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      if (!w_act[i]) continue;
      uint16_t *dst = sw + w_row[i] * LDK + w_half[i] * 32;
      const uint32_t w4[4] = {st.wq[i].x, st.wq[i].y, st.wq[i].z, st.wq[i].w};
      float sc = __uint_as_float(st.ws[i]), bi = __uint_as_float(st.wb[i]);
      if constexpr (SBL) {
        const int kc = kt * 2 + w_half[i];
        const uint32_t bytes = (uint32_t)BN * sbrow;
        // chunks past k_in read group 0 (finite) and meet zero codes
        const uint32_t o = (uint32_t)w_row[i] * sbrow +
                           (kc < cpr ? (((uint32_t)kc * 32) >> p.log2_group) * sbb : 0u);
        const unsigned char *ts = sbtab + o;
        if (p.sb_bf16) {
          sc = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(ts) << 16);
          bi = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(ts + bytes) << 16);
        } else {
          sc = *reinterpret_cast<const float *>(ts);
          bi = *reinterpret_cast<const float *>(ts + bytes);
        }
      }
      const float s24 = sc * 0x1p24f, s20 = sc * 0x1p20f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<uint4 *>(dst + jj * 8) = dequant_word(w4[jj], s24, s20, bi);
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i)
      if (x_act[i]) *reinterpret_cast<uint4 *>(sx + x_row[i] * LDK + x_seg[i] * 8) = st.xq[i];
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  Step ring[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) load_step(u, ring[u]);
  for (int k0 = 0; k0 < nsteps; k0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      store_step(k0 + u, ring[u]);
      lds_barrier();
      load_step(k0 + u + PF, ring[u]);  // refill the slot just stored
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
        if (row < p.T && col < M.n_out) {
          if (p.y_bf16)
            reinterpret_cast<__bf16 *>(M.y)[row * M.ldy + col] = (__bf16)acc[a][b][v];
          else
            reinterpret_cast<float *>(M.y)[row * M.ldy + col] = acc[a][b][v];
        }
      }
    }
}

template <int BM, int BN, int WM, int WN, int PF = 2>
hipError_t launch_tile(GemmMultiParams p, hipStream_t stream) {
  constexpr size_t kStatic = (size_t)(BM + BN) * LDK * 2;
  p.m_tiles = (int)((p.T + BM - 1) / BM);
  int t = 0;
  for (int i = 0; i < kMaxMats; ++i) {
    if (i < p.n_mats) {
      p.m[i].tile0 = t;
      t += (p.m[i].n_out + BN - 1) / BN;
    } else {
      p.m[i].tile0 = INT32_MAX;
    }
  }
  p.n_tiles = t;
  const int64_t tiles = (int64_t)p.m_tiles * p.n_tiles;
  if (tiles > INT32_MAX / 2) return hipErrorInvalidValue;
  p.tiles = (int32_t)tiles;
  p.per_xcd = (int32_t)((tiles + 7) / 8);
  const unsigned grid = (unsigned)(8 * p.per_xcd);
  // the scale / bias table in LDS when it fits next to the tiles
  const size_t sbrow = (size_t)(p.k_in >> p.log2_group) * (p.sb_bf16 ? 2 : 4);
  const size_t tab = 2 * (size_t)BN * sbrow;
  if (!(tab <= 96 * 1024 && kStatic + tab <= (size_t)kMaxLds)) {
    hipLaunchKernelGGL((qgemm_kernel<BM, BN, WM, WN, PF, false>), dim3(grid), dim3(WM * WN * 64), 0,
                       stream, p);
    return hipGetLastError();
  }
  auto kern = qgemm_kernel<BM, BN, WM, WN, PF, true>;
  // opt in to the LDS left next to the static tiles (once per device)
  hipError_t e = lds_opt_in(reinterpret_cast<const void *>(kern), (int)(kMaxLds - kStatic));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WM * WN * 64), tab, stream, p);
  return hipGetLastError();
}

}  // namespace

// Tile by T (measured on MI355X at N = 17408, K = 5120): narrow tiles keep
// more workgroups per CU for short T; 8-wave 128x128 tiles up to T = 2048.
hipError_t launch_gemm(const GemmMultiParams &p, hipStream_t stream) {
  if (p.n_mats < 1 || p.n_mats > kMaxMats) return hipErrorInvalidValue;
  if (p.T <= 32) return launch_tile<32, 64, 1, 2>(p, stream);
  if (p.T <= 64) return launch_tile<64, 64, 2, 2>(p, stream);
  if (p.T <= 256) return launch_tile<128, 64, 2, 2>(p, stream);
  if (p.T <= 2048) return launch_tile<128, 128, 2, 4>(p, stream);
  return launch_tile<128, 128, 2, 2>(p, stream);
}

}  // namespace qint4
