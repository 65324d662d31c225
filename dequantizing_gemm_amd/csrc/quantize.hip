// quantize.hip -- block-wise symmetric INT4 quantization and nibble packing
// on gfx950.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, quantize_int4): for row n and group gi
// (k in [gi*group, min((gi+1)*group, K))):
//   scale = binary16(absmax / 7)        absmax / 7 as a binary32 IEEE division
//   q     = clip(rint(w / float(scale)), -8, 7), or 0 if scale == 0
// and byte j of the packed row = (q[2j] & 0xF) | (q[2j+1] & 0xF) << 4.
//
// Bit-exactness: the division is the correctly rounded binary32 division
// (this file is compiled with -fhip-fp32-correctly-rounded-divide-sqrt and
// without fast-math, so `a / b` is the IEEE operation, not a reciprocal
// multiply), binary32 -> binary16 is v_cvt_f16_f32 in round-to-nearest-even
// with fp16 denormals kept, and rintf is v_rndne_f32 (ties to even).
//
// Work decomposition (vector kernel): one wavefront per 512-element segment
// of a row; lane l owns elements [8l, 8l+8) of the segment, read as two
// 16-byte loads (a wavefront reads 2 KiB contiguously). A group of g
// elements spans g/8 adjacent lanes, and its absmax is a butterfly max over
// those lanes. Each lane writes its 8 codes as one 32-bit store (256
// contiguous bytes per wavefront), and the first lane of each group writes the
// group's scale. HBM traffic per weight: 4 B read, 0.5 B written, plus 2 B per
// group.
#include "device_common.h"
#include "kernels.h"

namespace int4dq {

__device__ __forceinline__ uint32_t code_of(float w, float sf) {
  if (sf == 0.0f) return 0u;                       // a group of zeros -> codes 0
  float r = __builtin_rintf(w / sf);               // IEEE division, ties-to-even
  r = __builtin_fminf(__builtin_fmaxf(r, -8.0f), 7.0f);
  return (uint32_t)(int)r & 0xFu;
}

// LANES = group / 8, a power of two in [1, 64].
template <int LANES>
__global__ __launch_bounds__(256) void quantize_vec_kernel(
    const float* __restrict__ w, int64_t K, int64_t G, int64_t segs_per_row,
    int64_t total_segs, uint8_t* __restrict__ packed, uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (seg >= total_segs) return;                   // whole wavefronts only
  const int64_t n = seg / segs_per_row;
  const int64_t k = (seg - n * segs_per_row) * 512 + (int64_t)lane * 8;
  const bool valid = k < K;                        // K % 8 == 0: all 8 or none
  float v[8];
  if (valid) {
    const float4_t* p = reinterpret_cast<const float4_t*>(w + n * K + k);
    const float4_t a = __builtin_nontemporal_load(p);
    const float4_t b = __builtin_nontemporal_load(p + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < LANES; o <<= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o));

  const float s32 = amax / 7.0f;
  const _Float16 s16 = (_Float16)s32;
  const float sf = (float)s16;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= code_of(v[i], sf) << (4 * i);
  if (valid) {
    *reinterpret_cast<uint32_t*>(packed + n * (K >> 1) + (k >> 1)) = word;
    if ((lane & (LANES - 1)) == 0)
      scales[n * G + k / (LANES * 8)] = __builtin_bit_cast(uint16_t, s16);
  }
}

// General kernels: any K, any group, any alignment. First one thread per
// (row, group) writes the scales, then one thread per packed byte reads them
// back (stream order separates the two launches) -- a byte may straddle two
// groups when the group size is odd.
__global__ __launch_bounds__(256) void quantize_scales_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, int64_t group, int64_t G,
    uint16_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N * G) return;
  const int64_t n = t / G, gi = t - n * G;
  const int64_t k0 = gi * group;
  const int64_t k1 = k0 + group < K ? k0 + group : K;
  float amax = 0.0f;
  for (int64_t k = k0; k < k1; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(w[n * K + k]));
  const _Float16 s16 = (_Float16)(amax / 7.0f);
  scales[t] = __builtin_bit_cast(uint16_t, s16);
}

__global__ __launch_bounds__(256) void quantize_pack_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, int64_t group, int64_t G,
    const uint16_t* __restrict__ scales, uint8_t* __restrict__ packed) {
  const int64_t B = (K + 1) >> 1;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N * B) return;
  const int64_t n = t / B, j = t - n * B;
  const int64_t k = 2 * j;
  const float sf0 = half_bits_to_float(scales[n * G + k / group]);
  uint32_t byte = code_of(w[n * K + k], sf0);
  if (k + 1 < K) {
    const float sf1 = half_bits_to_float(scales[n * G + (k + 1) / group]);
    byte |= code_of(w[n * K + k + 1], sf1) << 4;
  }
  packed[t] = (uint8_t)byte;
}

// ---------------------------------------------------------------------------
// Affine codes ("Build a Blockwise INT4 Inference Engine", step 2; the range
// widened to include zero, "Quantizing a Language Model From Scratch": the
// zero point makes 0.0 exact):
//   lo = min(min_g w, 0), hi = max(max_g w, 0)
//   scale = binary16((hi - lo) / 15)      binary32 subtraction and division
//   zp    = clip(rint(-lo / float(scale)), 0, 15), or 0 if scale == 0
//   u     = clip(rint(w / float(scale) + zp), 0, 15), or 0 if scale == 0
// w / scale is a binary32 division; zp is added to it in binary64, where the
// sum is exact, and the sum rounded half to even (a binary32 sum could round
// a value just off a half-integer onto it). Codes are unsigned nibbles in the
// same layout; the zero points are one byte per group.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t affine_zp(float lo, float sf) {
  if (sf == 0.0f) return 0u;
  float z = __builtin_rintf(-lo / sf);
  z = __builtin_fminf(__builtin_fmaxf(z, 0.0f), 15.0f);
  return (uint32_t)z;
}

__device__ __forceinline__ uint32_t affine_code(float w, float sf, uint32_t zp) {
  if (sf == 0.0f) return 0u;
  const double t = (double)(w / sf) + (double)zp;  // exact
  double r = __builtin_rint(t);
  r = __builtin_fmin(__builtin_fmax(r, 0.0), 15.0);
  return (uint32_t)r;
}

template <int LANES>
__global__ __launch_bounds__(256) void quantize_affine_vec_kernel(
    const float* __restrict__ w, int64_t K, int64_t G, int64_t segs_per_row,
    int64_t total_segs, uint8_t* __restrict__ packed, uint16_t* __restrict__ scales,
    uint8_t* __restrict__ zeros) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (seg >= total_segs) return;                   // whole wavefronts only
  const int64_t n = seg / segs_per_row;
  const int64_t k = (seg - n * segs_per_row) * 512 + (int64_t)lane * 8;
  const bool valid = k < K;
  float v[8];
  if (valid) {
    const float4_t* p = reinterpret_cast<const float4_t*>(w + n * K + k);
    const float4_t a = __builtin_nontemporal_load(p);
    const float4_t b = __builtin_nontemporal_load(p + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float lo = 0.0f, hi = 0.0f;                      // the range includes zero
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lo = __builtin_fminf(lo, v[i]);
    hi = __builtin_fmaxf(hi, v[i]);
  }
#pragma unroll
  for (int o = 1; o < LANES; o <<= 1) {
    lo = __builtin_fminf(lo, __shfl_xor(lo, o));
    hi = __builtin_fmaxf(hi, __shfl_xor(hi, o));
  }
  const _Float16 s16 = (_Float16)((hi - lo) / 15.0f);
  const float sf = (float)s16;
  const uint32_t zp = affine_zp(lo, sf);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= affine_code(v[i], sf, zp) << (4 * i);
  if (valid) {
    *reinterpret_cast<uint32_t*>(packed + n * (K >> 1) + (k >> 1)) = word;
    if ((lane & (LANES - 1)) == 0) {
      const int64_t gi = n * G + k / (LANES * 8);
      scales[gi] = __builtin_bit_cast(uint16_t, s16);
      zeros[gi] = (uint8_t)zp;
    }
  }
}

__global__ __launch_bounds__(256) void quantize_affine_params_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, int64_t group, int64_t G,
    uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N * G) return;
  const int64_t n = t / G, gi = t - n * G;
  const int64_t k0 = gi * group;
  const int64_t k1 = k0 + group < K ? k0 + group : K;
  float lo = 0.0f, hi = 0.0f;
  for (int64_t k = k0; k < k1; ++k) {
    lo = __builtin_fminf(lo, w[n * K + k]);
    hi = __builtin_fmaxf(hi, w[n * K + k]);
  }
  const _Float16 s16 = (_Float16)((hi - lo) / 15.0f);
  scales[t] = __builtin_bit_cast(uint16_t, s16);
  zeros[t] = (uint8_t)affine_zp(lo, (float)s16);
}

__global__ __launch_bounds__(256) void quantize_affine_pack_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, int64_t group, int64_t G,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros,
    uint8_t* __restrict__ packed) {
  const int64_t B = (K + 1) >> 1;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N * B) return;
  const int64_t n = t / B, j = t - n * B;
  const int64_t k = 2 * j;
  const int64_t g0 = n * G + k / group;
  uint32_t byte = affine_code(w[n * K + k], half_bits_to_float(scales[g0]), zeros[g0]);
  if (k + 1 < K) {
    const int64_t g1 = n * G + (k + 1) / group;
    byte |= affine_code(w[n * K + k + 1], half_bits_to_float(scales[g1]), zeros[g1]) << 4;
  }
  packed[t] = (uint8_t)byte;
}

bool quantize_vec_supported(const float* w, int64_t K, int64_t group, const uint8_t* packed,
                            const uint16_t* scales) {
  const bool pow2 = group >= 8 && group <= 512 && (group & (group - 1)) == 0;
  return pow2 && K % 8 == 0 && ((uintptr_t)w % 16) == 0 && ((uintptr_t)packed % 4) == 0 &&
         ((uintptr_t)scales % 2) == 0;
}

hipError_t launch_quantize(const float* w, int64_t N, int64_t K, int64_t group, uint8_t* packed,
                           uint16_t* scales, hipStream_t stream) {
  const int64_t G = (K + group - 1) / group;
  if (quantize_vec_supported(w, K, group, packed, scales)) {
    const int64_t segs_per_row = (K + 511) / 512;
    const int64_t total = N * segs_per_row;
    const dim3 grid((unsigned)((total + 3) / 4)), block(256);
    switch (group) {
#define INT4DQ_Q(Gs)                                                                        \
  case Gs:                                                                                  \
    hipLaunchKernelGGL(quantize_vec_kernel<Gs / 8>, grid, block, 0, stream, w, K, G,      \
                       segs_per_row, total, packed, scales);                               \
    break;
      INT4DQ_Q(8) INT4DQ_Q(16) INT4DQ_Q(32) INT4DQ_Q(64) INT4DQ_Q(128) INT4DQ_Q(256) INT4DQ_Q(512)
#undef INT4DQ_Q
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int64_t B = (K + 1) / 2;
  hipLaunchKernelGGL(quantize_scales_kernel, dim3((unsigned)((N * G + 255) / 256)), dim3(256), 0,
                     stream, w, N, K, group, G, scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quantize_pack_kernel, dim3((unsigned)((N * B + 255) / 256)), dim3(256), 0,
                     stream, w, N, K, group, G, scales, packed);
  return hipGetLastError();
}

hipError_t launch_quantize_affine(const float* w, int64_t N, int64_t K, int64_t group,
                                  uint8_t* packed, uint16_t* scales, uint8_t* zeros,
                                  hipStream_t stream) {
  const int64_t G = (K + group - 1) / group;
  if (quantize_vec_supported(w, K, group, packed, scales)) {
    const int64_t segs_per_row = (K + 511) / 512;
    const int64_t total = N * segs_per_row;
    const dim3 grid((unsigned)((total + 3) / 4)), block(256);
    switch (group) {
#define INT4DQ_QA(Gs)                                                                       \
  case Gs:                                                                                  \
    hipLaunchKernelGGL(quantize_affine_vec_kernel<Gs / 8>, grid, block, 0, stream, w, K, G, \
                       segs_per_row, total, packed, scales, zeros);                        \
    break;
      INT4DQ_QA(8) INT4DQ_QA(16) INT4DQ_QA(32) INT4DQ_QA(64) INT4DQ_QA(128) INT4DQ_QA(256) INT4DQ_QA(512)
#undef INT4DQ_QA
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int64_t B = (K + 1) / 2;
  hipLaunchKernelGGL(quantize_affine_params_kernel, dim3((unsigned)((N * G + 255) / 256)), dim3(256),
                     0, stream, w, N, K, group, G, scales, zeros);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quantize_affine_pack_kernel, dim3((unsigned)((N * B + 255) / 256)), dim3(256),
                     0, stream, w, N, K, group, G, scales, zeros, packed);
  return hipGetLastError();
}

}  // namespace int4dq
