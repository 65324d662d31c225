// dequantize.hip -- packed INT4 codes and binary16 scales -> w_hat = q * scale
// (binary32 or binary16) on gfx950.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement: the reconstruction is the code times
// its group's scale). This is the materialising step of the unfused
// dequantize-then-GEMM baseline the engine page compares the fused kernel
// against ("Build a Blockwise INT4 Inference Engine", fused GEMM and
// benchmark sections); the fused matmul never runs it.
//
// Arithmetic: q has at most 4 significant bits and the widened scale 11, so
// q * scale is exact in binary32; the binary16 output is that exact product
// rounded to nearest even (one fp16 multiply of two exact fp16 operands rounds
// the same exact product), overflowing to infinity past 65504.
//
// Fast path (K and group multiples of 32, 16-byte aligned bases): one thread
// per 16 packed bytes = 32 codes of one row, which lie in one group; codes
// become exact fp16 with codes_to_half_natural, one packed fp16 multiply per
// pair (binary16 out) or a widening and one fp32 multiply per code (binary32
// out), and 64 or 128 bytes of 16-byte stores. HBM-bound: 0.5 B read and 2 or
// 4 B written per weight. Anything else: one thread per output element, the
// grid striding over them.
//
// Affine codes ("Build a Blockwise INT4 Inference Engine", step 2): the
// value is (u - zp) * scale with the group's zero point zp; u - zp in
// [-15, 15] is exact in fp16 (codes_to_half_natural_zp) and the products stay
// exact in binary32.
#include "device_common.h"
#include "kernels.h"

namespace int4dq {

template <bool HALF, bool AFF>
__global__ __launch_bounds__(256) void dequantize_flat_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int64_t chunks, int64_t chunks_per_row, int64_t G,
    int64_t group, void* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const int64_t n = c / chunks_per_row;
  const int64_t k0 = 32 * (c - n * chunks_per_row);            // first code of the chunk
  const uint16_t sbits = scales[n * G + k0 / group];
  const uint32_t zb = AFF ? zp_bias_natural(zeros[n * G + k0 / group]) : 0u;
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(packed + 16 * c);
  const uint32_t words[4] = {v.x, v.y, v.z, v.w};
  auto expand = [&](uint32_t d, half2_t hw[4]) {
    if constexpr (AFF) codes_to_half_natural_zp(d, hw, zb);
    else codes_to_half_natural(d, hw);
  };
  if constexpr (HALF) {
    const _Float16 s = __builtin_bit_cast(_Float16, sbits);
    const half2_t s2 = {s, s};
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(static_cast<_Float16*>(out) + 32 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t hw[4];
      expand(words[i], hw);
      u32x4_t o;
      o.x = __builtin_bit_cast(uint32_t, hw[0] * s2);
      o.y = __builtin_bit_cast(uint32_t, hw[1] * s2);
      o.z = __builtin_bit_cast(uint32_t, hw[2] * s2);
      o.w = __builtin_bit_cast(uint32_t, hw[3] * s2);
      dst[i] = o;
    }
  } else {
    const float s = half_bits_to_float(sbits);
    float4_t* dst = reinterpret_cast<float4_t*>(static_cast<float*>(out) + 32 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t hw[4];
      expand(words[i], hw);
      float4_t a, b;
      a.x = (float)hw[0].x * s; a.y = (float)hw[0].y * s; a.z = (float)hw[1].x * s; a.w = (float)hw[1].y * s;
      b.x = (float)hw[2].x * s; b.y = (float)hw[2].y * s; b.z = (float)hw[3].x * s; b.w = (float)hw[3].y * s;
      dst[2 * i] = a;
      dst[2 * i + 1] = b;
    }
  }
}

template <bool HALF, bool AFF>
__global__ __launch_bounds__(256) void dequantize_elem_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int64_t N, int64_t K, int64_t G, int64_t group,
    void* __restrict__ out) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < N * K;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = t / K, k = t - n * K;
    const uint32_t b = packed[n * ((K + 1) >> 1) + (k >> 1)];
    const uint32_t u = (b >> (4 * (k & 1))) & 0xFu;
    const int q = AFF ? (int)u - (int)zeros[n * G + k / group] : sx4(u);
    const float v = (float)q * half_bits_to_float(scales[n * G + k / group]);   // exact
    if constexpr (HALF) static_cast<_Float16*>(out)[t] = (_Float16)v;           // nearest even
    else static_cast<float*>(out)[t] = v;
  }
}

template <bool AFF>
static void launch_dequantize_t(const uint8_t* packed, const uint16_t* scales,
                                const uint8_t* zeros, int64_t N, int64_t K, int64_t group,
                                bool half, void* out, hipStream_t stream) {
  const int64_t G = (K + group - 1) / group;
  if (K % 32 == 0 && group % 32 == 0 && (uintptr_t)packed % 16 == 0 && (uintptr_t)out % 16 == 0) {
    // (one thread per 32 codes: the grid stays below 2^32 threads for any
    // output that fits a device, 2^37 codes being 256 GiB of binary16)
    const int64_t per_row = K / 32, chunks = N * per_row;
    const dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
    if (half)
      hipLaunchKernelGGL((dequantize_flat_kernel<true, AFF>), grid, block, 0, stream, packed, scales, zeros, chunks, per_row, G, group, out);
    else
      hipLaunchKernelGGL((dequantize_flat_kernel<false, AFF>), grid, block, 0, stream, packed, scales, zeros, chunks, per_row, G, group, out);
  } else {
    const dim3 grid(stride_grid((N * K + 255) / 256)), block(256);
    if (half)
      hipLaunchKernelGGL((dequantize_elem_kernel<true, AFF>), grid, block, 0, stream, packed, scales, zeros, N, K, G, group, out);
    else
      hipLaunchKernelGGL((dequantize_elem_kernel<false, AFF>), grid, block, 0, stream, packed, scales, zeros, N, K, G, group, out);
  }
}

hipError_t launch_dequantize(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros,
                             int64_t N, int64_t K, int64_t group, bool half, void* out,
                             hipStream_t stream) {
  if (zeros) launch_dequantize_t<true>(packed, scales, zeros, N, K, group, half, out, stream);
  else launch_dequantize_t<false>(packed, scales, zeros, N, K, group, half, out, stream);
  return hipGetLastError();
}

}  // namespace int4dq
