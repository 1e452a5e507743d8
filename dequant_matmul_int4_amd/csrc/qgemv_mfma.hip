// qgemv_mfma.hip -- small-M int4 products with bf16 activations, 1..16
// activation rows (stored outputs of up to 8 matrices, or the gate/up pair
// with the SwiGLU epilogue), on gfx950 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Sources (by page title and passage):
//   [FFAI #14] thewafflehaus/FFAI pull 14, "feat(everything-bagel): clean
//              migration of PR #9 + #10 onto updated dev": int4 GEMV wrappers
//              (weight, scales, biases, in_dim, group_size); batched QKV
//              (several projections of one input in one launch).
//   [ds4 #844] antirez/ds4 pull 844, "Ornith 1.5 + Qwen 3.8 27B hybrid
//              runtime + DFlash speculative decoding on Metal": small row
//              counts (speculative-verify rounds below the MMA tile) and the
//              contract that a batched call reproduces sequential calls
//              bit for bit.
//
// The product per row and group is the factorised affine form used by the
// GEMV kernels:
//     sum_k (s q_k + b) x_k = s * (sum_k (128 + q_k) x_k - 128 sum x) + b sum x,
// with (128 + q) formed exactly as bf16 (bits 0x4300 | q).  Here the inner
// sums come from MFMA instead of v_dot2: the codes are the B operand (16 rows
// of a tile as its N columns), the staged activation rows the A operand (its
// M rows; rows past T repeat the last token and are never stored).  Every
// output element is one column of the product, so a token's result does not
// depend on how many tokens share the launch: a T-row call equals T one-row
// calls bit for bit.
//
// Work decomposition (gfx950 specific, not from the pages):
//   * A workgroup takes tiles of 16 rows of one matrix (tiles blockIdx.x,
//     blockIdx.x + gridDim.x, ...: one each when every tile has its own
//     workgroup, more when the staged rows limit the chip to one workgroup
//     per CU); its KS waves split k_in into slices of kChunksPerWave chunks
//     of 32 codes (steps of 128).  The activation slices are staged once per
//     workgroup and serve all of its tiles.
//   * Lane (r, kb) = (lane % 16, lane / 16) loads, per step, the 16-byte
//     chunk 4*step + kb of row r: a load instruction covers 16 rows x 64
//     contiguous bytes.  An MFMA takes 8 codes (one word) per lane, and its
//     32-deep K must stay inside one group; a 4 x 4 exchange of words between
//     the lanes 16 apart (two permlane32 and two permlane16 swaps) leaves lane
//     (r, kb) with word kb of each of the step's 4 chunks, so MFMA i covers
//     exactly chunk 4*step + i.
//   * Each wave stages its own activation slice (all T rows) in its own LDS
//     region, permuted to the nibble-pair order of the decoded words, with the
//     per-group sums of every row, and the (scale, bias) pairs of its 16 rows
//     and groups: no workgroup barrier until the final reduction.
//   * After each group's chunks, lane (r, kb) applies row r's scale and bias
//     to its 4 accumulators (tokens 4*kb .. 4*kb + 3).  At the end the waves
//     write their accumulators to LDS and the workgroup sums the K slices in
//     wave order and stores the T x 16 outputs.

#include "kernels.h"

namespace qint4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChunksPerWave = 16;  // 32-code chunks per wave (8 and 32 measured no faster)
constexpr int kSteps = kChunksPerWave / 4;                   // 128-k steps per wave
static_assert(kChunksPerWave % 4 == 0 && kChunksPerWave >= 4, "whole 128-k steps");
constexpr int kTileRows = 16;
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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Touch every 64-byte line of the kernel arguments with back-to-back scalar
// loads and one wait, rather than several dependent rounds of misses.
__device__ __forceinline__ void warm_kernargs() {
  typedef const uint32_t __attribute__((address_space(4))) *kptr;
  const kptr ka = (kptr)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (i * 64 < (int)sizeof(GemvParams)) ? ka[i * 16] : 0u;
  asm volatile("" ::"s"(v[0]), "s"(v[1]), "s"(v[2]), "s"(v[3]), "s"(v[4]), "s"(v[5]), "s"(v[6]),
               "s"(v[7]));
}

// Workgroup barrier ordering LDS only (no drain of outstanding vector loads).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned segments of 2^L2 lanes (L2 = 2, 3 or 4); all lanes active.
template <int L2>
__device__ __forceinline__ float seg_sum(float v) {
  v += dpp_mov<0xB1>(v);                    // lane ^ 1
  v += dpp_mov<0x4E>(v);                    // lane ^ 2
  if constexpr (L2 >= 3) v += dpp_mov<0x141>(v);  // other quad of 8
  if constexpr (L2 >= 4) v += dpp_mov<0x140>(v);  // other half of 16
  return v;
}

__device__ __forceinline__ void store_out(void *y, int64_t i, float v, int bf16) {
  if (bf16)
    reinterpret_cast<__bf16 *>(y)[i] = (__bf16)v;
  else
    reinterpret_cast<float *>(y)[i] = v;
}

// LDS bytes of one wave's region: TT staged rows of the slice (plus 16 bytes
// of padding per row against bank conflicts), the per-group sums of 16 token
// slots, and the (scale, bias) pairs of 16 rows for each of the NS code
// streams -- at least NS KB, since that last part also takes the wave's
// accumulators for each tile's final reduction.
constexpr int wave_region_bytes(int tt, int cpg, int ns) {
  const int ng = kChunksPerWave / cpg;
  const int tb = ns * ng * 16 * 8;
  return tt * (kChunksPerWave * 64 + 16) + ng * 16 * 4 + (tb > ns * 1024 ? tb : ns * 1024);
}

// NS = 1: stored outputs of up to kMaxMats matrices (tile t of matrix i from
// task0[i]).  NS = 2: the gate/up pair (m[0], m[1]) with the SwiGLU epilogue
// h = silu(gate) * up written to m[0].y.
template <int SBT, int CPG, int TT, int NS>
__global__ void __launch_bounds__(1024) qgemv_mfma_kernel(const GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  warm_kernargs();
  constexpr int NG = kChunksPerWave / CPG;  // groups per wave
  constexpr int TS = kChunksPerWave * 64 + 16;
  constexpr int WR = wave_region_bytes(TT, CPG, NS);
  constexpr uint32_t SBB = (SBT == 1) ? 2 : 4;
  constexpr int TE = (NG * 16 + 63) / 64;  // (scale, bias) entries per lane
  // several tiles per workgroup from 8 tokens on; up to 4 tokens every tile
  // has its own workgroup (the host launches one per tile), and the kernel
  // keeps the registers of a single pass
  constexpr bool kPersist = TT >= 8;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = p.n_tok;
  const uint32_t kwb = (uint32_t)p.kwb, sbrow = (uint32_t)p.sbrow;
  const int r = lane & 15, kb = lane >> 4;
  const int c0 = wv * kChunksPerWave;  // first chunk of this wave's slice
  const int g0 = c0 / CPG;

  unsigned char *reg = smem + wv * WR;
  unsigned char *xst = reg;                                                // [TT][chunks][4 words] x 16 B
  float *xsum = reinterpret_cast<float *>(reg + TT * TS);                  // [NG][16 tokens]
  constexpr int TBL = TT * TS + NG * 16 * 4;  // (scale, bias) table, then each tile's accumulators
  float2 *tbl = reinterpret_cast<float2 *>(reg + TBL);                     // [NS][NG][16 rows]

  // Matrix, first row and row count of a tile (the count of later matrix
  // starts at or below the tile picks the matrix).
  struct TileAt {
    int m, row0, n_rows;
  };
  auto tile_at = [&](int tile) {
    int m = 0, first = 0;
    if constexpr (NS == 1) {
#pragma unroll
      for (int i = 1; i < kMaxMats; ++i) {
        const int t0 = p.task0[i];
        const bool in = tile >= t0;
        m += in ? 1 : 0;
        first = in ? t0 : first;
      }
    }
    return TileAt{m, (tile - first) * kTileRows, (int)p.m[m].n_out};
  };
  // scales/biases, then codes, of a tile (into the registers below)
  uint32_t sr[NS][TE], br[NS][TE];
  uint4 cw[NS][kSteps];
  auto load_tile = [&](const TileAt &ti) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const GemvMat &mat = p.m[ti.m + st];
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(mat.scales, (uint32_t)ti.n_rows * sbrow);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(mat.biases, (uint32_t)ti.n_rows * sbrow);
#pragma unroll
      for (int j = 0; j < TE; ++j) {
        const int e = lane + 64 * j;  // entry (group e / 16, row e % 16)
        const uint32_t off = e < NG * 16
                                 ? (uint32_t)(ti.row0 + (e & 15)) * sbrow + (uint32_t)(g0 + (e >> 4)) * SBB
                                 : kOutOfRange;
        sr[st][j] = buf_load_sb<SBT>(rs, off);
        br[st][j] = buf_load_sb<SBT>(rb, off);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.m[ti.m + st].codes, (uint32_t)ti.n_rows * kwb);
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
        cw[st][s] = buf_load_b128(rc, (uint32_t)(ti.row0 + r) * kwb + (uint32_t)(c0 + 4 * s + kb) * 16);
    }
  };

  // ---- loads: activation rows first (L2), then the first tile's ----
  // the slice of a token is U 16-byte units (8 elements each); unit
  // u = lane + 64 i of the wave's TT * U is element 8 (u % U) of token u / U
  constexpr int U = kChunksPerWave * 4;
  constexpr int XR = (TT * U + 63) / 64;  // staging rounds
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(p.x, (uint32_t)(((int64_t)(T - 1) * p.ldx + (int64_t)p.ncx * 32) * 2));
  uint4 xv[XR];
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int u = lane + 64 * i, t = u / U, lu = u % U;
    const uint32_t off =
        t < T ? (uint32_t)(((int64_t)t * p.ldx + (int64_t)c0 * 32 + lu * 8) * 2) : kOutOfRange;
    xv[i] = buf_load_b128(rx, off);
  }
  // keep the issue order (activation, scales/biases, codes): the staging then
  // waits only for the activation loads
  __builtin_amdgcn_sched_barrier(0);
  int tile = blockIdx.x;  // tiles blockIdx.x, blockIdx.x + gridDim.x, ... (uniform)
  TileAt cur = tile_at(tile);
  load_tile(cur);

  // ---- stage the activation slice and its per-group sums (once) ----
  // (all lanes take part in every round: the group sums reduce over 4 * CPG
  // neighbouring lanes, which never straddle two tokens since U % 16 == 0)
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int u = lane + 64 * i, t = u / U, lu = u % U;
    const uint4 w = xv[i];
    uint4 pr;  // pairs (x_i, x_{i+4}): the order of the decoded nibble pairs
    pr.x = (w.x & 0xFFFFu) | (w.z << 16);
    pr.y = (w.x >> 16) | (w.z & 0xFFFF0000u);
    pr.z = (w.y & 0xFFFFu) | (w.w << 16);
    pr.w = (w.y >> 16) | (w.w & 0xFFFF0000u);
    if (t < T) *reinterpret_cast<uint4 *>(xst + t * TS + lu * 16) = pr;
    float s8 = ((bf16_lo(w.x) + bf16_hi(w.x)) + (bf16_lo(w.y) + bf16_hi(w.y))) +
               ((bf16_lo(w.z) + bf16_hi(w.z)) + (bf16_lo(w.w) + bf16_hi(w.w)));
    constexpr int L2 = CPG == 1 ? 2 : CPG == 2 ? 3 : 4;  // lanes of one group: 4 * CPG
    s8 = seg_sum<L2>(s8);
    if (t < T && (lu & (4 * CPG - 1)) == 0) xsum[(lu / (4 * CPG)) * 16 + t] = s8;
  }

  uint32_t magic = 0x43004300u;
  asm volatile("" : "+v"(magic));  // keep in a VGPR so AND-OR stays one VOP3
  const int nn = min(lane & 15, T - 1);  // token of this lane's A row
  const unsigned char *xa = xst + nn * TS + kb * 16;
  const int KS = p.waves_per_wg;

  while (true) {
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int j = 0; j < TE; ++j) {
        const int e = lane + 64 * j;
        if (e < NG * 16) tbl[st * NG * 16 + e] = make_float2(sb_value<SBT>(sr[st][j]), sb_value<SBT>(br[st][j]));
      }

    // ---- products ----
    f32x4_t acc[NS], c[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      acc[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      c[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      uint32_t wd[NS][4];
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        uint32_t w0 = cw[st][s].x, w1 = cw[st][s].y, w2 = cw[st][s].z, w3 = cw[st][s].w;
        // lane (r, kb) holds chunk 4s + kb; exchange so that it holds word kb of
        // chunks 4s .. 4s + 3 (a 4 x 4 transpose over the lanes 16 apart)
        auto a = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
        w0 = a[0];
        w2 = a[1];
        auto b = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
        w1 = b[0];
        w3 = b[1];
        auto e = __builtin_amdgcn_permlane16_swap(w0, w1, false, false);
        w0 = e[0];
        w1 = e[1];
        auto f = __builtin_amdgcn_permlane16_swap(w2, w3, false, false);
        w2 = f[0];
        w3 = f[1];
        wd[st][0] = w0;
        wd[st][1] = w1;
        wd[st][2] = w2;
        wd[st][3] = w3;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = 4 * s + i;  // chunk of the slice
        const uint4 xq = *reinterpret_cast<const uint4 *>(xa + ch * 64);
        const bf16x8_t ax = __builtin_bit_cast(bf16x8_t, xq);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          uint32_t pq[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) pq[k] = ((wd[st][i] >> (4 * k)) & 0x000F000Fu) | magic;
          const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, make_uint4(pq[0], pq[1], pq[2], pq[3]));
          const f32x4_t cin = (ch % CPG == 0) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : c[st];
          c[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, bw, cin, 0, 0, 0);
        }
        if ((ch + 1) % CPG == 0) {
          const int g = ch / CPG;
          const f32x4_t xs = *reinterpret_cast<const f32x4_t *>(xsum + g * 16 + 4 * kb);
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const float2 sbv = tbl[(st * NG + g) * 16 + r];
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
              const float d = c[st][mm] - 128.f * xs[mm];
              acc[st][mm] += fmaf(sbv.x, d, sbv.y * xs[mm]);
            }
          }
        }
      }
    }

    // ---- sum the K slices (wave order) and store ----
    auto reduce_store = [&](const TileAt &done) {
#pragma unroll
      for (int st = 0; st < NS; ++st)  // over this wave's table, which the products no longer read
        *reinterpret_cast<f32x4_t *>(reg + TBL + st * 1024 + lane * 16) = acc[st];
      lds_barrier();
      void *const y = p.m[done.m].y;
      for (int o = threadIdx.x; o < kTileRows * T; o += KS * 64) {
        const int rr = o & 15, n = o >> 4;
        const int src = (rr + 16 * (n >> 2)) * 16 + (n & 3) * 4;  // lane and accumulator of (n, rr)
        float v[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          v[st] = 0.f;
          for (int w = 0; w < KS; ++w)
            v[st] += *reinterpret_cast<const float *>(smem + w * WR + TBL + st * 1024 + src);
        }
        float out = v[0];
        if constexpr (NS == 2) out = (v[0] / (1.f + __expf(-v[0]))) * v[1];
        const int row = done.row0 + rr;
        if (row < done.n_rows) store_out(y, (int64_t)n * done.n_rows + row, out, p.y_bf16);
      }
    };
    const int next = tile + (int)gridDim.x;
    if (!kPersist || next >= p.n_tasks) {  // uniform: the workgroup's last tile
      reduce_store(cur);
      break;
    }
    // the next tile's loads overlap this tile's reduction
    const TileAt done = cur;
    cur = tile_at(next);
    load_tile(cur);
    reduce_store(done);
    lds_barrier();  // every wave has read the accumulators before the next tables land
    tile = next;
  }
}
template <int SBT, int CPG, int TT, int NS>
hipError_t launch_mfma(const GemvParams &p, int64_t grid, int ks, hipStream_t stream) {
  auto kern = qgemv_mfma_kernel<SBT, CPG, TT, NS>;
  const size_t lds = (size_t)ks * wave_region_bytes(TT, CPG, NS);
  if (lds > 64 * 1024) {
    hipError_t e = lds_opt_in(reinterpret_cast<const void *>(kern), kMaxLds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(ks * 64), lds, stream, p);
  return hipGetLastError();
}

template <int SBT, int CPG, int NS>
hipError_t launch_tt(const GemvParams &p, int tt, int64_t grid, int ks, hipStream_t s) {
  switch (tt) {
    case 1: return launch_mfma<SBT, CPG, 1, NS>(p, grid, ks, s);
    case 2: return launch_mfma<SBT, CPG, 2, NS>(p, grid, ks, s);
    case 4: return launch_mfma<SBT, CPG, 4, NS>(p, grid, ks, s);
    case 8: return launch_mfma<SBT, CPG, 8, NS>(p, grid, ks, s);
    case 16: return launch_mfma<SBT, CPG, 16, NS>(p, grid, ks, s);
    default: return hipErrorInvalidValue;
  }
}

template <int NS>
hipError_t launch_group(const GemvParams &p, int tt, int group_size, int sb_bf16, int64_t grid, int ks,
                        hipStream_t s) {
  switch (group_size) {
    case 32: return sb_bf16 ? launch_tt<1, 1, NS>(p, tt, grid, ks, s) : launch_tt<0, 1, NS>(p, tt, grid, ks, s);
    case 64: return sb_bf16 ? launch_tt<1, 2, NS>(p, tt, grid, ks, s) : launch_tt<0, 2, NS>(p, tt, grid, ks, s);
    case 128: return sb_bf16 ? launch_tt<1, 4, NS>(p, tt, grid, ks, s) : launch_tt<0, 4, NS>(p, tt, grid, ks, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t gemv_mfma_lds_bytes(int tt, int group_size, int64_t k_in, int streams) {
  const int cpg = group_size / 32;
  return (size_t)(k_in / (32 * kChunksPerWave)) * (size_t)wave_region_bytes(tt, cpg, streams);
}

int gemv_mfma_waves(int64_t k_in) { return (int)(k_in / (32 * kChunksPerWave)); }

bool gemv_mfma_supported(int64_t k_in, int group_size, int streams) {
  if (group_size != 32 && group_size != 64 && group_size != 128) return false;
  if (k_in % (32 * kChunksPerWave) != 0) return false;
  const int64_t ks = k_in / (32 * kChunksPerWave);
  if (ks < 1 || ks > 16) return false;
  // every token count takes this path or none does (rows of a T-row call equal
  // one-row calls bit for bit), so the largest staging must fit
  return gemv_mfma_lds_bytes(kMaxTokens, group_size, k_in, streams) <= (size_t)kMaxLds;
}

hipError_t launch_gemv_mfma(const GemvParams &p, int tt, int group_size, int sb_bf16, int swiglu,
                            int64_t grid, hipStream_t stream) {
  const int ks = p.waves_per_wg;
  if (ks < 1 || ks > 16 || grid < 1 || grid > p.n_tasks || (tt <= 4 && grid != p.n_tasks))
    return hipErrorInvalidValue;
  return swiglu ? launch_group<2>(p, tt, group_size, sb_bf16, grid, ks, stream)
                : launch_group<1>(p, tt, group_size, sb_bf16, grid, ks, stream);
}

}  // namespace qint4
