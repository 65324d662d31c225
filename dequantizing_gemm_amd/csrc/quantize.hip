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
// with fp16 denormals kept, and rintf is v_rndne_f32 (ties to even). The
// per-element division is only carried out where it can change the code
// (quotient_for_rint): elsewhere a reciprocal multiply rounds to the same
// integer.
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

// The quotient w / scale as far as rounding it to an integer is concerned.
// t = w * rcp(scale) is within 2^-22 |t| of the correctly rounded quotient
// (v_rcp_f32 is within 1 ulp, the product rounds once), and |t| < 32 here
// (|w| <= 7.01 scale, or 15.02 scale for affine codes; subnormal binary16
// scales stay below 22), so within 2^-17: rint gives the same integer unless
// a half-integer lies that close. Those elements (|t - rint(t)| within 2^-14
// of 0.5; a true tie always is) take the IEEE division; a wavefront whose
// lanes have none skips it. Exact: the codes are the ones the division gives.
__device__ __forceinline__ bool near_half_integer(float t) {
  const float d = __builtin_fabsf(t - __builtin_rintf(t));   // exact for |t| < 2^22
  return __builtin_fabsf(d - 0.5f) < 0x1p-14f;
}

__device__ __forceinline__ float quotient_for_rint(float w, float sf, float rsf) {
  float t = w * rsf;
  if (__builtin_expect(near_half_integer(t), 0)) t = w / sf;   // IEEE division
  return t;
}

// rcp(sf) once per group, and 0 for a zero scale: then t = 0, which is no
// half-integer, so a zero group gets codes 0 without a branch.
__device__ __forceinline__ float scale_rcp(float sf) {
  return sf == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(sf);
}

__device__ __forceinline__ uint32_t code_of(float w, float sf, float rsf) {
  float r = __builtin_rintf(quotient_for_rint(w, sf, rsf));   // ties-to-even
  r = __builtin_fminf(__builtin_fmaxf(r, -8.0f), 7.0f);
  return (uint32_t)(int)r & 0xFu;
}

// Group extremes across lanes, as an unsigned maximum of binary32 patterns.
// The lane values reduced here never are NaN (fmax / fmin from 0 drop NaN
// operands) and have one sign: non-negative values (an absmax, or the upper
// end of a range from 0) order like their patterns; non-positive values (the
// lower end of a range from 0) order reversed, so their minimum has the
// largest pattern. (For a lower end the result may be -0 where a float min
// gives +0; the scale hi - lo and the zero point rint(-lo / s) are the same
// either way.) 0 is the identity of the unsigned max, so each butterfly step
// is one DPP max instruction.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
  return v > o ? v : o;
}
template <int LANES>
__device__ __forceinline__ float run_umax_bits(float a) {
  uint32_t v = __builtin_bit_cast(uint32_t, a);
  if constexpr (LANES >= 2) v = dpp_umax<0xB1>(v);
  if constexpr (LANES >= 4) v = dpp_umax<0x4E>(v);
  if constexpr (LANES >= 8) v = dpp_umax<0x141>(v);
  if constexpr (LANES >= 16) v = dpp_umax<0x140>(v);
#pragma unroll
  for (int o = 16; o < LANES; o <<= 1) {
    const uint32_t u = (uint32_t)__shfl_xor((int)v, o);
    v = v > u ? v : u;
  }
  return __builtin_bit_cast(float, v);
}

// LANES = group / 8, a power of two in [1, 64]. Grid: x covers the 512-code
// segments of a row, four per block (one per wavefront); y walks the rows.
template <int LANES>
__global__ __launch_bounds__(256) void quantize_vec_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, int64_t G, int64_t segs_per_row,
    uint8_t* __restrict__ packed, uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (seg >= segs_per_row) return;                 // whole wavefronts only
  for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
    const int64_t k = seg * 512 + (int64_t)lane * 8;
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
    amax = run_umax_bits<LANES>(amax);

    const float s32 = amax / 7.0f;
    const _Float16 s16 = (_Float16)s32;
    const float sf = (float)s16;
    const float rsf = scale_rcp(sf);
    // code_of for the lane's 8 elements, with one branch around the divisions
    // (each element is clamped on its own path, so no NaN quieting is needed
    // where the two paths meet)
    float c[8];
    bool near = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = v[i] * rsf;
      const float q = __builtin_rintf(t);
      near |= __builtin_fabsf(__builtin_fabsf(t - q) - 0.5f) < 0x1p-14f;   // near_half_integer(t)
      c[i] = __builtin_fminf(__builtin_fmaxf(q, -8.0f), 7.0f);
    }
    if (__builtin_expect(near, 0)) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (near_half_integer(v[i] * rsf))
          c[i] = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(v[i] / sf), -8.0f), 7.0f);   // IEEE division
    }
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= ((uint32_t)(int)c[i] & 0xFu) << (4 * i);
    if (valid) {
      *reinterpret_cast<uint32_t*>(packed + n * (K >> 1) + (k >> 1)) = word;
      if ((lane & (LANES - 1)) == 0)
        scales[n * G + k / (LANES * 8)] = __builtin_bit_cast(uint16_t, s16);
    }
  }
}

// General kernels: any K, any group, any alignment. First one thread per
// (row, group) writes the scales, then one thread per packed byte reads them
// back (stream order separates the two launches) -- a byte may straddle two
// groups when the group size is odd.
__global__ __launch_bounds__(256) void quantize_scales_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, int64_t group, int64_t G,
    uint16_t* __restrict__ scales) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < N * G;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = t / G, gi = t - n * G;
    const int64_t k0 = gi * group;
    const int64_t k1 = k0 + group < K ? k0 + group : K;
    float amax = 0.0f;
    for (int64_t k = k0; k < k1; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(w[n * K + k]));
    const _Float16 s16 = (_Float16)(amax / 7.0f);
    scales[t] = __builtin_bit_cast(uint16_t, s16);
  }
}

__global__ __launch_bounds__(256) void quantize_pack_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, int64_t group, int64_t G,
    const uint16_t* __restrict__ scales, uint8_t* __restrict__ packed) {
  const int64_t B = (K + 1) >> 1;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < N * B;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = t / B, j = t - n * B;
    const int64_t k = 2 * j;
    const float sf0 = half_bits_to_float(scales[n * G + k / group]);
    uint32_t byte = code_of(w[n * K + k], sf0, scale_rcp(sf0));
    if (k + 1 < K) {
      const float sf1 = half_bits_to_float(scales[n * G + (k + 1) / group]);
      byte |= code_of(w[n * K + k + 1], sf1, scale_rcp(sf1)) << 4;
    }
    packed[t] = (uint8_t)byte;
  }
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

// rint(w / sf + zp) with the exact sum. Away from a half-integer the integer
// zp does not change the rounding, so rint(t + zp) = rint(t) + zp with t as in
// quotient_for_rint. Near one (a tie above all: rint(0.5 + 1) = 2 but
// rint(0.5) + 1 = 1), the IEEE quotient plus zp in binary64, where the sum is
// exact, is rounded half to even.
__device__ __forceinline__ uint32_t affine_code(float w, float sf, float rsf, uint32_t zp) {
  const float t = w * rsf;                         // 0 for a zero scale (rsf = 0, zp = 0)
  float r;
  if (__builtin_expect(near_half_integer(t), 0))
    r = (float)__builtin_rint((double)(w / sf) + (double)zp);   // IEEE division, exact sum
  else
    r = __builtin_rintf(t) + (float)zp;                         // integers < 2^24: exact
  r = __builtin_fminf(__builtin_fmaxf(r, 0.0f), 15.0f);
  return (uint32_t)r;
}

template <int LANES>
__global__ __launch_bounds__(256) void quantize_affine_vec_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, int64_t G, int64_t segs_per_row,
    uint8_t* __restrict__ packed, uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t seg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (seg >= segs_per_row) return;                 // whole wavefronts only
  for (int64_t n = blockIdx.y; n < N; n += gridDim.y) {
    const int64_t k = seg * 512 + (int64_t)lane * 8;
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
    lo = run_umax_bits<LANES>(lo);
    hi = run_umax_bits<LANES>(hi);
    const _Float16 s16 = (_Float16)((hi - lo) / 15.0f);
    const float sf = (float)s16;
    const float rsf = scale_rcp(sf);
    const uint32_t zp = affine_zp(lo, sf);
    // affine_code for the lane's 8 elements, with one branch around the
    // divisions (each element is clamped on its own path)
    float c[8];
    bool near = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = v[i] * rsf;
      const float q = __builtin_rintf(t);
      near |= __builtin_fabsf(__builtin_fabsf(t - q) - 0.5f) < 0x1p-14f;   // near_half_integer(t)
      c[i] = __builtin_fminf(__builtin_fmaxf(q + (float)zp, 0.0f), 15.0f);
    }
    if (__builtin_expect(near, 0)) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (near_half_integer(v[i] * rsf)) c[i] = (float)affine_code(v[i], sf, rsf, zp);
    }
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= (uint32_t)c[i] << (4 * i);
    if (valid) {
      *reinterpret_cast<uint32_t*>(packed + n * (K >> 1) + (k >> 1)) = word;
      if ((lane & (LANES - 1)) == 0) {
        const int64_t gi = n * G + k / (LANES * 8);
        scales[gi] = __builtin_bit_cast(uint16_t, s16);
        zeros[gi] = (uint8_t)zp;
      }
    }
  }
}

__global__ __launch_bounds__(256) void quantize_affine_params_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, int64_t group, int64_t G,
    uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < N * G;
       t += (int64_t)gridDim.x * blockDim.x) {
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
}

__global__ __launch_bounds__(256) void quantize_affine_pack_kernel(
    const float* __restrict__ w, int64_t N, int64_t K, int64_t group, int64_t G,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros,
    uint8_t* __restrict__ packed) {
  const int64_t B = (K + 1) >> 1;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < N * B;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = t / B, j = t - n * B;
    const int64_t k = 2 * j;
    const int64_t g0 = n * G + k / group;
    const float sf0 = half_bits_to_float(scales[g0]);
    uint32_t byte = affine_code(w[n * K + k], sf0, scale_rcp(sf0), zeros[g0]);
    if (k + 1 < K) {
      const int64_t g1 = n * G + (k + 1) / group;
      const float sf1 = half_bits_to_float(scales[g1]);
      byte |= affine_code(w[n * K + k + 1], sf1, scale_rcp(sf1), zeros[g1]) << 4;
    }
    packed[t] = (uint8_t)byte;
  }
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
    const dim3 grid((unsigned)((segs_per_row + 3) / 4), (unsigned)(N < 65535 ? N : 65535)), block(256);
    switch (group) {
#define INT4DQ_Q(Gs)                                                                        \
  case Gs:                                                                                  \
    hipLaunchKernelGGL(quantize_vec_kernel<Gs / 8>, grid, block, 0, stream, w, N, K, G,   \
                       segs_per_row, packed, scales);                                      \
    break;
      INT4DQ_Q(8) INT4DQ_Q(16) INT4DQ_Q(32) INT4DQ_Q(64) INT4DQ_Q(128) INT4DQ_Q(256) INT4DQ_Q(512)
#undef INT4DQ_Q
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int64_t B = (K + 1) / 2;
  hipLaunchKernelGGL(quantize_scales_kernel, dim3(stride_grid((N * G + 255) / 256)), dim3(256), 0,
                     stream, w, N, K, group, G, scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quantize_pack_kernel, dim3(stride_grid((N * B + 255) / 256)), dim3(256), 0,
                     stream, w, N, K, group, G, scales, packed);
  return hipGetLastError();
}

hipError_t launch_quantize_affine(const float* w, int64_t N, int64_t K, int64_t group,
                                  uint8_t* packed, uint16_t* scales, uint8_t* zeros,
                                  hipStream_t stream) {
  const int64_t G = (K + group - 1) / group;
  if (quantize_vec_supported(w, K, group, packed, scales)) {
    const int64_t segs_per_row = (K + 511) / 512;
    const dim3 grid((unsigned)((segs_per_row + 3) / 4), (unsigned)(N < 65535 ? N : 65535)), block(256);
    switch (group) {
#define INT4DQ_QA(Gs)                                                                       \
  case Gs:                                                                                  \
    hipLaunchKernelGGL(quantize_affine_vec_kernel<Gs / 8>, grid, block, 0, stream, w, N, K, \
                       G, segs_per_row, packed, scales, zeros);                            \
    break;
      INT4DQ_QA(8) INT4DQ_QA(16) INT4DQ_QA(32) INT4DQ_QA(64) INT4DQ_QA(128) INT4DQ_QA(256) INT4DQ_QA(512)
#undef INT4DQ_QA
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int64_t B = (K + 1) / 2;
  hipLaunchKernelGGL(quantize_affine_params_kernel, dim3(stride_grid((N * G + 255) / 256)), dim3(256),
                     0, stream, w, N, K, group, G, scales, zeros);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quantize_affine_pack_kernel, dim3(stride_grid((N * B + 255) / 256)), dim3(256),
                     0, stream, w, N, K, group, G, scales, zeros, packed);
  return hipGetLastError();
}

}  // namespace int4dq
