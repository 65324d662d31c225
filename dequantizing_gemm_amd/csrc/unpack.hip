// unpack.hip -- packed INT4 codes -> sign-extended int8 on gfx950.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, unpack_int4): out[n, k] is the
// sign-extended 4-bit code of element k of row n; element 2j is the low
// nibble of byte j, element 2j+1 the high nibble; the pad nibble of an odd K
// is dropped.
//
// Even K: the packed array and the output are the same byte stream read at
// 1:2, so the kernel is flat. Each thread turns two 8-byte loads into two
// 16-byte stores: per 32-bit word, low and high nibbles are split with two
// masks, sign-extended bytewise (v | ((v & 8) * 0x1E) sets bits 4..7 exactly
// when bit 3 is set, with no carry between bytes), and interleaved with two
// byte permutes. HBM traffic per weight: 0.5 B read + 1 B written.
// Odd K: rows are not byte-aligned in the output, so a simple kernel writes
// each row's bytes one by one.
#include "device_common.h"
#include "kernels.h"

namespace int4dq {

__device__ __forceinline__ u32x2_t unpack_word(uint32_t w) {
  uint32_t lo = w & 0x0F0F0F0Fu;
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  lo |= (lo & 0x08080808u) * 0x1Eu;
  hi |= (hi & 0x08080808u) * 0x1Eu;
  u32x2_t r;
  r.x = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // lo0 hi0 lo1 hi1
  r.y = __builtin_amdgcn_perm(hi, lo, 0x07030602u);   // lo2 hi2 lo3 hi3
  return r;
}

// A wavefront takes 1 KB of packed bytes: lane l reads the 8 bytes at 8 l and
// at 512 + 8 l, so each of its two 16-byte stores lands in one contiguous
// kilobyte of output per wavefront instruction (a lane owning 16 consecutive
// bytes would store two half-filled 32-byte strides instead).
__global__ __launch_bounds__(256) void unpack_flat_kernel(const uint8_t* __restrict__ packed,
                                                          int64_t nbytes, int8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  for (int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 1024; base < nbytes;
       base += (int64_t)gridDim.x * 4 * 1024) {
    if (base + 1024 <= nbytes) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t b0 = base + 512 * h + 8 * lane;
        const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(packed + b0));
        const u32x2_t a = unpack_word(v.x), b = unpack_word(v.y);
        u32x4_t o;
        o.x = a.x; o.y = a.y; o.z = b.x; o.w = b.y;
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out + 2 * b0));
      }
    } else {
      for (int h = 0; h < 2; ++h)
        for (int64_t b = base + 512 * h + 8 * lane; b < base + 512 * h + 8 * lane + 8 && b < nbytes; ++b) {
          const uint32_t v = packed[b];
          out[2 * b] = (int8_t)sx4(v & 0xFu);
          out[2 * b + 1] = (int8_t)sx4(v >> 4);
        }
    }
  }
}

__global__ __launch_bounds__(256) void unpack_rows_kernel(const uint8_t* __restrict__ packed,
                                                          int64_t N, int64_t K,
                                                          int8_t* __restrict__ out) {
  const int64_t B = (K + 1) >> 1;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < N * B;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = t / B, j = t - n * B;
    const uint32_t v = packed[t];
    out[n * K + 2 * j] = (int8_t)sx4(v & 0xFu);
    if (2 * j + 1 < K) out[n * K + 2 * j + 1] = (int8_t)sx4(v >> 4);
  }
}

hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* out,
                         hipStream_t stream) {
  if (K % 2 == 0 && ((uintptr_t)packed % 16) == 0 && ((uintptr_t)out % 16) == 0) {
    const int64_t nbytes = N * (K / 2);
    const int64_t kb = (nbytes + 1023) / 1024;                 // one wavefront per KB
    hipLaunchKernelGGL(unpack_flat_kernel, dim3(stride_grid((kb + 3) / 4)), dim3(256), 0,
                       stream, packed, nbytes, out);
  } else {
    const int64_t total = N * ((K + 1) / 2);
    hipLaunchKernelGGL(unpack_rows_kernel, dim3(stride_grid((total + 255) / 256)), dim3(256), 0,
                       stream, packed, N, K, out);
  }
  return hipGetLastError();
}

}  // namespace int4dq
