// moe_prefill.hip -- top-K mixture of experts for T tokens at once (prefill),
// as expert-sorted gather GEMMs on gfx950 bf16 MFMA.
//
// Sources (by page title and passage):
//   [FFAI #9]  thewafflehaus/FFAI pull 9, "Everything Bagel": the batched
//              MoE path fans the T * topK (token, slot) rows into one GEMM per
//              gate / up / down, sorted by expert id so that a row tile shares
//              one expert's weights; CSR expert offsets are built from the
//              sorted top-K ids; a scatter-sum unpermutes the results; the
//              m1 gather GEMM wiring.
//   [FFAI #14] thewafflehaus/FFAI pull 14, "feat(everything-bagel): clean
//              migration of PR #9 + #10 onto updated dev": the chain8
//              combine out = residual + sum_k w_k d_k, the fused SwiGLU.
//
// Stages (four launches on one stream, no host round trip):
//   1. moe_sort_kernel (one workgroup): counting sort of the P = T * top_k
//      pairs p = t * top_k + k by expert id.  Writes perm[slot] = p,
//      pos[p] = slot (or 0xFFFFFFFF for an id >= n_experts, which contributes
//      nothing), and a table of row tiles: tile i covers sorted slots
//      row0 .. row0 + rows - 1 of one expert (rows <= BM).  The order of the
//      pairs inside one expert's segment does not affect any result: every
//      GEMM row is computed independently of the other rows of its tile.
//   2. moe_gemm_kernel<GATEUP>: for each tile, the gathered activation rows
//      x[p / top_k] times the tile expert's gate and up matrices (weights
//      dequantised in float32, rounded to bf16 in LDS, as in the dense
//      prefill GEMM), float32 accumulators, then h = silu(g) * u.  h is kept
//      to float32 accuracy as two bf16 planes, hi = bf16(h), lo = bf16(h - hi)
//      (hi + lo carries 16 significant bits), in sorted order.
//   3. moe_gemm_kernel<DOWN>: h rows times the down matrix, as
//      hi * W + lo * W (two MFMAs per fragment), float32 result d in sorted
//      order.
//   4. moe_combine_kernel: out[t] = residual[t] + sum_k wts[t][k] d[pos[t][k]].

#include "kernels.h"

namespace qint4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements)
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// 1. sort
// ---------------------------------------------------------------------------

constexpr int kSortThreads = 1024;
constexpr int kSortBatch = 16;  // ids in flight per thread

// Exclusive scan of v[0..n) in LDS (n <= 4 * kSortThreads) by the whole
// workgroup; v[n] receives the total.  Each thread scans 4 consecutive
// entries, waves scan their threads' sums with shuffles, one wave scans the
// wave totals.
__device__ void block_exclusive_scan(uint32_t *v, int n, uint32_t *wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t loc[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * tid + i;
    loc[i] = j < n ? v[j] : 0u;
    s += loc[i];
  }
  uint32_t inc = s;  // inclusive scan over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wave_tot[wave] = inc;
  lds_barrier();
  if (wave == 0) {
    constexpr int NW = kSortThreads / 64;
    uint32_t t = lane < NW ? wave_tot[lane] : 0u, ti = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_up(ti, d);
      if (lane >= d) ti += o;
    }
    if (lane < NW) wave_tot[lane] = ti - t;   // exclusive wave offsets
    if (lane == NW - 1) wave_tot[NW] = ti;     // total
  }
  lds_barrier();
  uint32_t run = wave_tot[wave] + inc - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * tid + i;
    if (j < n) v[j] = run;
    run += loc[i];
  }
  if (tid == 0) v[n] = wave_tot[kSortThreads / 64];
  lds_barrier();
}

__global__ void __launch_bounds__(kSortThreads)
    moe_sort_kernel(const uint32_t *__restrict__ ids, int64_t n_pairs, int n_experts, int bm,
                    uint32_t *__restrict__ perm, uint32_t *__restrict__ pos,
                    uint32_t *__restrict__ tiles, int max_tiles) {
  // tiles: [0] tile count, then per tile (expert, row0, rows) at 1 + 3i
  __shared__ uint32_t cnt[kMaxExpertsPrefill + 1];
  __shared__ uint32_t tcnt[kMaxExpertsPrefill + 1];
  __shared__ uint32_t wave_tot[kSortThreads / 64 + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e <= n_experts; e += kSortThreads) cnt[e] = 0u;
  lds_barrier();
  // ids are read kSortBatch per thread at a time, all loads issued before
  // any is used: one memory round trip per batch rather than per id
  for (int64_t b = 0; b < n_pairs; b += (int64_t)kSortThreads * kSortBatch) {
    uint32_t e[kSortBatch];
#pragma unroll
    for (int u = 0; u < kSortBatch; ++u) {
      const int64_t p = b + tid + (int64_t)u * kSortThreads;
      e[u] = p < n_pairs ? ids[p] : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < kSortBatch; ++u)
      if (e[u] < (uint32_t)n_experts) atomicAdd(&cnt[e[u]], 1u);
  }
  lds_barrier();
  for (int e = tid; e < n_experts; e += kSortThreads) tcnt[e] = (cnt[e] + bm - 1) / bm;
  lds_barrier();
  block_exclusive_scan(cnt, n_experts, wave_tot);   // cnt[e] = first slot of expert e
  block_exclusive_scan(tcnt, n_experts, wave_tot);  // tcnt[e] = first tile of expert e
  const uint32_t n_tiles = tcnt[n_experts];
  if (tid == 0) tiles[0] = n_tiles <= (uint32_t)max_tiles ? n_tiles : 0u;  // never exceeded
  for (int e = tid; e < n_experts; e += kSortThreads) {
    const uint32_t r0 = cnt[e], n = cnt[e + 1] - r0, t0 = tcnt[e];
    for (uint32_t j = 0; j * bm < n; ++j) {
      const uint32_t i = t0 + j;
      if (i < (uint32_t)max_tiles) {
        tiles[1 + 3 * i] = (uint32_t)e;
        tiles[2 + 3 * i] = r0 + j * bm;
        tiles[3 + 3 * i] = min((uint32_t)bm, n - j * bm);
      }
    }
  }
  lds_barrier();
  // scatter: cnt[e] is now the next free slot of expert e
  for (int64_t b = 0; b < n_pairs; b += (int64_t)kSortThreads * kSortBatch) {
    uint32_t e[kSortBatch];
#pragma unroll
    for (int u = 0; u < kSortBatch; ++u) {
      const int64_t p = b + tid + (int64_t)u * kSortThreads;
      e[u] = p < n_pairs ? ids[p] : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < kSortBatch; ++u) {
      const int64_t p = b + tid + (int64_t)u * kSortThreads;
      if (p < n_pairs) {
        uint32_t slot = kNoSlot;
        if (e[u] < (uint32_t)n_experts) {
          slot = atomicAdd(&cnt[e[u]], 1u);
          perm[slot] = (uint32_t)p;
        }
        pos[p] = slot;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2./3. grouped gather GEMM
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// 8 codes of one word -> 8 bf16 weights (k order) as a uint4: float32
// s * q + b rounded to nearest even.  The word masked with 0x000F000F holds codes (n, n + 4) as the f16
// subnormals q 2^-24, masked with 0x00F000F0 codes (n + 1, n + 5) as
// 16 q 2^-24; v_fma_mix_f32 against the scale times 2^24 (s24) or 2^20 (s20)
// gives fmaf(s, q, b) exactly (scales below 2^104 in magnitude).
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

enum { MG_GATEUP = 0, MG_DOWN = 1 };

constexpr uint32_t kMgOOR = 0x80000000u;  // an offset past every resource: reads zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mg_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 mg_ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

template <int MODE, int BM, int BN, int WM, int WN, int PF>
__global__ void __launch_bounds__(WM * WN * 64) moe_gemm_kernel(const MoeGemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int NB = MODE == MG_GATEUP ? 2 : 1;  // weight matrices (gate, up) or (down)
  constexpr int NA = MODE == MG_GATEUP ? 1 : 2;  // activation planes (x) or (h hi, h lo)
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int WCH = (2 * BN * NB + NT - 1) / NT;  // 16-byte code loads per thread per step
  constexpr int XCH = (8 * BM * NA + NT - 1) / NT;  // 16-byte activation loads per thread per step
  static_assert(FM >= 1 && FN >= 1, "tile");

  __shared__ __attribute__((aligned(16))) uint16_t sa[NA][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sw[NB][BN * LDK];
  // p.sb_lds: the scales then biases of this workgroup's BN rows of each
  // matrix for the whole K range (dynamic LDS, 2 * NB * BN * sbrow bytes)
  extern __shared__ __attribute__((aligned(16))) unsigned char sbtab[];

  const int mt = blockIdx.x % p.max_mtiles;
  const int nt = blockIdx.x / p.max_mtiles;
  if (mt >= (int)p.tiles[0]) return;  // whole workgroup: past the last row tile
  const uint32_t e = p.tiles[1 + 3 * mt];
  const int64_t row0 = p.tiles[2 + 3 * mt];
  const int rows = (int)p.tiles[3 + 3 * mt];
  const int n0 = nt * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int cpr = p.k_in / 32;
  const uint32_t gpr = (uint32_t)p.k_in >> p.log2_group;
  const uint32_t sbb = p.sb_bf16 ? 2 : 4;
  const uint32_t kwb = (uint32_t)p.k_in / 2;   // code bytes per row
  const uint32_t sbrow = gpr * sbb;            // scale (= bias) bytes per row
  // K steps rounded up to whole prefetch rounds; steps past the end load
  // out-of-range zeros and add nothing
  const int nsteps = ((p.k_in + BK - 1) / BK + PF - 1) / PF * PF;

  // Raw buffer resources over this tile expert's slab of each weight matrix
  // (and the activation): an offset at or past the end reads zero without
  // touching memory, so every load below is unconditional.
  __amdgpu_buffer_rsrc_t rcw[NB], rsw[NB], rbw[NB];
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const unsigned char *c = reinterpret_cast<const unsigned char *>(m ? p.codes1 : p.codes0);
    const unsigned char *sc = reinterpret_cast<const unsigned char *>(m ? p.scales1 : p.scales0);
    const unsigned char *bi = reinterpret_cast<const unsigned char *>(m ? p.biases1 : p.biases0);
    rcw[m] = mg_rsrc(c + (uint64_t)e * p.n_out * kwb, (uint32_t)p.n_out * kwb);
    rsw[m] = mg_rsrc(sc + (uint64_t)e * p.n_out * sbrow, (uint32_t)p.n_out * sbrow);
    rbw[m] = mg_rsrc(bi + (uint64_t)e * p.n_out * sbrow, (uint32_t)p.n_out * sbrow);
  }

  // Scale / bias table: one coalesced pass over the contiguous BN * sbrow
  // bytes of each array (16-, 4- or 2-byte units, whichever the alignment
  // allows), instead of two scattered 2-byte loads per chunk and step.
  if (p.sb_lds) {
    const uint32_t bytes = (uint32_t)BN * sbrow;
#pragma unroll
    for (int a = 0; a < 2 * NB; ++a) {
      const __amdgpu_buffer_rsrc_t r = (a & 1) ? rbw[a >> 1] : rsw[a >> 1];
      const unsigned char *src = reinterpret_cast<const unsigned char *>((a & 1) ? ((a >> 1) ? p.biases1 : p.biases0)
                                                                                : ((a >> 1) ? p.scales1 : p.scales0)) +
                                 ((uint64_t)e * p.n_out + n0) * sbrow;
      const uint32_t base = (uint32_t)n0 * sbrow;   // offset of row n0 in the expert's slab
      unsigned char *dst = sbtab + (uint32_t)a * bytes;
      const uintptr_t al = reinterpret_cast<uintptr_t>(src) | bytes;
      if ((al & 15) == 0) {
        for (uint32_t j = tid * 16; j < bytes; j += NT * 16)
          *reinterpret_cast<uint4 *>(dst + j) = mg_ld128(r, base + j);
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

  // per-thread load assignments
  int w_mat[WCH], w_row[WCH], w_half[WCH];
  bool w_act[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int t = tid + i * NT;
    w_act[i] = t < 2 * BN * NB;
    // one matrix per wave (64 divides 2 * BN): the buffer resource stays scalar
    static_assert((2 * BN) % 64 == 0 && (8 * BM) % 64 == 0, "per-wave matrix / plane");
    w_mat[i] = __builtin_amdgcn_readfirstlane(w_act[i] ? t / (2 * BN) : 0);
    w_row[i] = (t % (2 * BN)) >> 1;
    w_half[i] = t & 1;
  }
  // activation loads: row base offset in bytes, or kMgOOR for a row past the tile
  uint32_t x_off[XCH];
  int x_pl[XCH], x_row[XCH], x_seg[XCH];
  bool x_act[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int t = tid + i * NT;
    x_act[i] = t < 8 * BM * NA;
    x_pl[i] = __builtin_amdgcn_readfirstlane(x_act[i] ? t / (8 * BM) : 0);
    x_row[i] = (t % (8 * BM)) >> 3;
    x_seg[i] = t & 7;
    x_off[i] = kMgOOR;
    if (x_act[i] && x_row[i] < rows) {
      const int64_t slot = row0 + x_row[i];
      if constexpr (MODE == MG_GATEUP)
        x_off[i] = (uint32_t)((int64_t)(p.perm[slot] / (uint32_t)p.top_k) * p.lda * 2);
      else
        x_off[i] = (uint32_t)(slot * p.lda * 2);
    }
  }
  const __amdgpu_buffer_rsrc_t rxa[2] = {mg_rsrc(p.a0, 0x7FFFFFF0u), mg_rsrc(NA > 1 ? p.a1 : p.a0, 0x7FFFFFF0u)};

  // register ring of PF prefetched steps
  struct Step {
    uint4 wq[WCH];
    uint32_t ws[WCH], wb[WCH];
    uint4 xq[XCH];
  };
  auto load_step = [&](int kt, Step &st) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int o = n0 + w_row[i];
      const int kc = kt * 2 + w_half[i];
      const bool ok = w_act[i] && kc < cpr;  // rows past n_out fall outside the resource
      const uint32_t oc = ok ? (uint32_t)o * kwb + (uint32_t)kc * 16 : kMgOOR;
      const uint32_t os = ok ? (uint32_t)o * sbrow + (((uint32_t)kc * 32) >> p.log2_group) * sbb : kMgOOR;
      const int m = w_mat[i];
      st.wq[i] = mg_ld128(m ? rcw[NB - 1] : rcw[0], oc);
      if (p.sb_lds) {  // read from the LDS table when the step is stored
        st.ws[i] = 0;
        st.wb[i] = 0;
      } else if (p.sb_bf16) {
        st.ws[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(m ? rsw[NB - 1] : rsw[0], os, 0, 0) << 16;
        st.wb[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(m ? rbw[NB - 1] : rbw[0], os, 0, 0) << 16;
      } else {
        st.ws[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(m ? rsw[NB - 1] : rsw[0], os, 0, 0);
        st.wb[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(m ? rbw[NB - 1] : rbw[0], os, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int k = kt * BK + x_seg[i] * 8;
      const uint32_t off = (x_off[i] != kMgOOR && k < p.k_in) ? x_off[i] + (uint32_t)k * 2 : kMgOOR;
      st.xq[i] = mg_ld128(x_pl[i] ? rxa[1] : rxa[0], off);
    }
  };

  auto store_step = [&](int kt, const Step &st) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      if (!w_act[i]) continue;
      uint16_t *dst = sw[w_mat[i]] + w_row[i] * LDK + w_half[i] * 32;
      const uint32_t w4[4] = {st.wq[i].x, st.wq[i].y, st.wq[i].z, st.wq[i].w};
      float sc = __uint_as_float(st.ws[i]), bi = __uint_as_float(st.wb[i]);
      if (p.sb_lds) {
        const int kc = kt * 2 + w_half[i];
        const uint32_t bytes = (uint32_t)BN * sbrow;
        // chunks past k_in read group 0 (finite) and meet zero codes
        const uint32_t o = (uint32_t)w_row[i] * sbrow +
                           (kc < cpr ? (((uint32_t)kc * 32) >> p.log2_group) * sbb : 0u);
        const unsigned char *ts = sbtab + (uint32_t)(2 * w_mat[i]) * bytes + o;
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
      if (x_act[i]) *reinterpret_cast<uint4 *>(sa[x_pl[i]] + x_row[i] * LDK + x_seg[i] * 8) = st.xq[i];
  };

  f32x16_t acc[NB][FM][FN];
#pragma unroll
  for (int m = 0; m < NB; ++m)
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][a][b][v] = 0.f;

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
      bf16x8_t af[NA][FM], bfr[NB][FN];
#pragma unroll
      for (int pl = 0; pl < NA; ++pl)
#pragma unroll
        for (int a = 0; a < FM; ++a)
          af[pl][a] = *reinterpret_cast<const bf16x8_t *>(sa[pl] + (wm * TM + a * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int b = 0; b < FN; ++b)
          bfr[m][b] = *reinterpret_cast<const bf16x8_t *>(sw[m] + (wn * TN + b * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
          for (int b = 0; b < FN; ++b)
#pragma unroll
            for (int pl = 0; pl < NA; ++pl)
              acc[m][a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[pl][a], bfr[m][b], acc[m][a][b], 0, 0, 0);
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
        const int r = wm * TM + a * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (r < rows && col < p.n_out) {
          const int64_t i = (row0 + r) * p.n_out + col;
          if constexpr (MODE == MG_GATEUP) {
            const float g = acc[0][a][b][v], u = acc[1][a][b][v];
            const float h = (g / (1.f + __expf(-g))) * u;
            const __bf16 hi = (__bf16)h;
            reinterpret_cast<__bf16 *>(p.y0)[i] = hi;
            reinterpret_cast<__bf16 *>(p.y1)[i] = (__bf16)(h - (float)hi);
          } else {
            reinterpret_cast<float *>(p.y0)[i] = acc[0][a][b][v];
          }
        }
      }
    }
}

// ---------------------------------------------------------------------------
// 4. unpermute + combine
// ---------------------------------------------------------------------------

// One thread per (token, 8 consecutive outputs).
__global__ void __launch_bounds__(256)
    moe_combine_kernel(const float *__restrict__ d, const uint32_t *__restrict__ pos,
                       const float *__restrict__ wts, int top_k, const void *__restrict__ residual,
                       void *__restrict__ out, int out_bf16, int64_t T, int hidden) {
  const int n8 = hidden / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * n8) return;
  const int64_t t = i / n8;
  const int c = (int)(i % n8) * 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  // every slot's loads are issued before the first is used (a skipped slot
  // reads row 0 and adds nothing); the slots are still added in order k
  uint32_t sl[kMaxTopK];
  float w[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    sl[k] = k < top_k ? pos[t * top_k + k] : kNoSlot;
    w[k] = k < top_k ? wts[t * top_k + k] : 0.f;
  }
  float4 a[kMaxTopK], b[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    const float4 *src =
        reinterpret_cast<const float4 *>(d + (int64_t)(sl[k] == kNoSlot ? 0u : sl[k]) * hidden + c);
    a[k] = src[0];
    b[k] = src[1];
  }
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (sl[k] == kNoSlot) continue;
    acc[0] = fmaf(w[k], a[k].x, acc[0]);
    acc[1] = fmaf(w[k], a[k].y, acc[1]);
    acc[2] = fmaf(w[k], a[k].z, acc[2]);
    acc[3] = fmaf(w[k], a[k].w, acc[3]);
    acc[4] = fmaf(w[k], b[k].x, acc[4]);
    acc[5] = fmaf(w[k], b[k].y, acc[5]);
    acc[6] = fmaf(w[k], b[k].z, acc[6]);
    acc[7] = fmaf(w[k], b[k].w, acc[7]);
  }
  const int64_t o = t * hidden + c;
  if (out_bf16) {
    if (residual) {
      const uint4 r = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(residual) + o);
      const uint32_t rr[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(rr[j] << 16);
        acc[2 * j + 1] += __uint_as_float(rr[j] & 0xFFFF0000u);
      }
    }
    uint4 v;
    v.x = pack_bf16x2(acc[0], acc[1]);
    v.y = pack_bf16x2(acc[2], acc[3]);
    v.z = pack_bf16x2(acc[4], acc[5]);
    v.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out) + o) = v;
  } else {
    if (residual) {
      const float4 *r = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(residual) + o);
      const float4 a = r[0], b = r[1];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + o);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

template <int MODE, int BM, int BN, int WM, int WN, int PF = 3>
hipError_t launch_mg(MoeGemmParams p, hipStream_t stream) {
  constexpr int NB = MODE == MG_GATEUP ? 2 : 1, NA = MODE == MG_GATEUP ? 1 : 2;
  constexpr size_t kStatic = (size_t)(NA * BM + NB * BN) * LDK * 2;
  const int64_t grid = (int64_t)p.max_mtiles * ((p.n_out + BN - 1) / BN);
  // the scale / bias table in LDS when it fits next to the tiles
  const size_t sbrow = (size_t)(p.k_in >> p.log2_group) * (p.sb_bf16 ? 2 : 4);
  const size_t tab = 2 * (size_t)NB * BN * sbrow;
  p.sb_lds = tab <= 96 * 1024 && kStatic + tab <= (size_t)kMaxLds;
  const size_t dyn = p.sb_lds ? tab : 0;
  auto kern = moe_gemm_kernel<MODE, BM, BN, WM, WN, PF>;
  // opt in to the LDS left next to the static tiles (once per device)
  if (dyn > 0) {
    hipError_t e = lds_opt_in(reinterpret_cast<const void *>(kern), (int)(kMaxLds - kStatic));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WM * WN * 64), dyn, stream, p);
  return hipGetLastError();
}

// Tiles and ring depths by row-tile height (measured on MI355X, 128
// experts, hidden 2048, inter 768): the down product (N = hidden) runs best
// on 128-wide column tiles with a 2-step ring; the gate/up pair (two weight
// tiles per step) on 64-wide ones, except 32-row tiles, which stream
// 128-wide tiles 4 steps ahead.
template <int MODE>
hipError_t launch_mode(const MoeGemmParams &p, int bm, hipStream_t stream) {
  if constexpr (MODE == MG_DOWN) {
    if (bm == 32) return launch_mg<MODE, 32, 128, 1, 4, 2>(p, stream);
    if (bm == 64) return launch_mg<MODE, 64, 128, 2, 2, 2>(p, stream);
    if (bm == 128) return launch_mg<MODE, 128, 128, 2, 4, 2>(p, stream);
  } else {
    if (bm == 32) return launch_mg<MODE, 32, 128, 1, 4, 4>(p, stream);
    if (bm == 64) return launch_mg<MODE, 64, 64, 2, 2>(p, stream);
    if (bm == 128) return launch_mg<MODE, 128, 64, 2, 2>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_moe_sort(const uint32_t *ids, int64_t n_pairs, int n_experts, int bm, uint32_t *perm,
                           uint32_t *pos, uint32_t *tiles, int max_tiles, hipStream_t stream) {
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(kSortThreads), 0, stream, ids, n_pairs, n_experts,
                     bm, perm, pos, tiles, max_tiles);
  return hipGetLastError();
}

hipError_t launch_moe_gemm(const MoeGemmParams &p, int down, int bm, hipStream_t stream) {
  return down ? launch_mode<MG_DOWN>(p, bm, stream) : launch_mode<MG_GATEUP>(p, bm, stream);
}

hipError_t launch_moe_combine(const float *d, const uint32_t *pos, const float *wts, int top_k,
                              const void *residual, void *out, int out_bf16, int64_t T, int hidden,
                              hipStream_t stream) {
  const int64_t n = T * (hidden / 8);
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)grid), dim3(256), 0, stream, d, pos, wts,
                     top_k, residual, out, out_bf16, T, hidden);
  return hipGetLastError();
}

}  // namespace qint4
