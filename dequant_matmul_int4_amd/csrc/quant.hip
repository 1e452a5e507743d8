// quant.hip -- the int4 group-affine quantiser (float weights -> codes,
// scales, biases) for gfx950.
//
// Source: antirez/ds4 pull 844, "Ornith 1.5 + Qwen 3.8 27B hybrid runtime +
// DFlash speculative decoding on Metal", PR body (verification list): the
// 4-bit group-64 affine type derives its codes from the serialised bf16
// scale and bias, not from the float32 values they were computed from.
//
// Per group of g consecutive weights of a row (the plain min/max affine
// reading; the page names the rule for the codes only):
//   lo = min w, hi = max w                       (float32, exact)
//   s  = (hi - lo) / 15,  b = lo                 (float32, correctly rounded)
//   s', b' = s, b as stored (bf16: round to nearest even)
//   q  = clamp(rint((w - b') / s'), 0, 15)       (float32, ties to even;
//                                                 q = 0 when s' == 0)
// so that s' q + b' is the stored grid point nearest to w.
//
// One thread per code word (8 consecutive weights); the g/8 threads of a group
// are adjacent lanes and reduce min/max with DPP inside a 16-lane row.  Loads
// are 128-bit and coalesced (consecutive lanes, consecutive words).

#include "kernels.h"

namespace qint4 {
namespace {

constexpr uint32_t kQuantOOR = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t q_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// min and max over aligned segments of GL lanes (GL = 4, 8 or 16), all lanes
// of a segment getting the result.  Whole wave active.
template <int GL>
__device__ __forceinline__ void seg_minmax(float &lo, float &hi) {
  lo = fminf(lo, dpp_f<0xB1>(lo));  // quad_perm [1,0,3,2]
  hi = fmaxf(hi, dpp_f<0xB1>(hi));
  lo = fminf(lo, dpp_f<0x4E>(lo));  // quad_perm [2,3,0,1]
  hi = fmaxf(hi, dpp_f<0x4E>(hi));
  if constexpr (GL >= 8) {
    lo = fminf(lo, dpp_f<0x141>(lo));  // row_half_mirror
    hi = fmaxf(hi, dpp_f<0x141>(hi));
  }
  if constexpr (GL >= 16) {
    lo = fminf(lo, dpp_f<0x140>(lo));  // row_mirror
    hi = fmaxf(hi, dpp_f<0x140>(hi));
  }
}

__device__ __forceinline__ float round_bf16(float v) { return (float)(__bf16)v; }

// w: [n_words * 8] weights (bf16 bits or float32), row-major; word i covers
// weights 8i .. 8i+7 and belongs to group i / GL.  The span of one launch
// stays below 2 GiB of weights (the host splits larger matrices).
template <int GL, bool W_BF16>
__global__ void __launch_bounds__(256)
    quantize_kernel(const void *__restrict__ w, int64_t n_words, int sb_bf16,
                    uint32_t *__restrict__ codes, void *__restrict__ scales,
                    void *__restrict__ biases) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  constexpr uint32_t WB = W_BF16 ? 16u : 32u;  // weight bytes per word
  const __amdgpu_buffer_rsrc_t rw = q_rsrc(w, (uint32_t)(n_words * WB));
  const uint32_t off = i < n_words ? (uint32_t)i * WB : kQuantOOR;

  float v[8];
  if constexpr (W_BF16) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i r = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float((uint32_t)r[k] << 16);
      v[2 * k + 1] = __uint_as_float((uint32_t)r[k] & 0xFFFF0000u);
    }
  } else {
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i a = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
    const v4i b = __builtin_amdgcn_raw_buffer_load_b128(rw, off + 16, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = __int_as_float(a[k]);
      v[4 + k] = __int_as_float(b[k]);
    }
  }

  float lo = v[0], hi = v[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    lo = fminf(lo, v[k]);
    hi = fmaxf(hi, v[k]);
  }
  seg_minmax<GL>(lo, hi);

  float s = (hi - lo) / 15.f;
  float b = lo;
  if (sb_bf16) {
    s = round_bf16(s);
    b = round_bf16(b);
  }
  uint32_t word = 0;
  if (s > 0.f) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float t = rintf((v[k] - b) / s);
      const uint32_t q = (uint32_t)fminf(fmaxf(t, 0.f), 15.f);
      word |= q << (4 * k);
    }
  }
  if (i < n_words) {
    codes[i] = word;
    if ((threadIdx.x & (GL - 1)) == 0) {
      const int64_t g = i / GL;
      if (sb_bf16) {
        reinterpret_cast<__bf16 *>(scales)[g] = (__bf16)s;  // exact: s is a bf16 value
        reinterpret_cast<__bf16 *>(biases)[g] = (__bf16)b;
      } else {
        reinterpret_cast<float *>(scales)[g] = s;
        reinterpret_cast<float *>(biases)[g] = b;
      }
    }
  }
}

template <int GL>
hipError_t launch_gl(const void *w, int w_bf16, int64_t n_words, int sb_bf16, uint32_t *codes,
                     void *scales, void *biases, hipStream_t stream) {
  const int64_t grid = (n_words + 255) / 256;
  if (w_bf16)
    hipLaunchKernelGGL((quantize_kernel<GL, true>), dim3((unsigned)grid), dim3(256), 0, stream, w,
                       n_words, sb_bf16, codes, scales, biases);
  else
    hipLaunchKernelGGL((quantize_kernel<GL, false>), dim3((unsigned)grid), dim3(256), 0, stream, w,
                       n_words, sb_bf16, codes, scales, biases);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void *w, int w_bf16, int64_t n_words, int group_size, int sb_bf16,
                           uint32_t *codes, void *scales, void *biases, hipStream_t stream) {
  switch (group_size) {
    case 32: return launch_gl<4>(w, w_bf16, n_words, sb_bf16, codes, scales, biases, stream);
    case 64: return launch_gl<8>(w, w_bf16, n_words, sb_bf16, codes, scales, biases, stream);
    case 128: return launch_gl<16>(w, w_bf16, n_words, sb_bf16, codes, scales, biases, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qint4
