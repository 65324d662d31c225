// device_common.h -- small device-side helpers shared by the gfx950 kernels.
//
// Nibble layout (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement): byte j of a packed row holds weight
// 2j in bits 0..3 and weight 2j+1 in bits 4..7, each a 4-bit two's complement
// code in [-8, 7]. A 32-bit word of a row therefore holds 8 consecutive codes,
// code i in bits 4i..4i+3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace int4dq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Sign extension of a 4-bit code v in [0, 15]: v - 16 * [v >= 8].
__device__ __forceinline__ int sx4(uint32_t v) { return (int)(v ^ 8u) - 8; }

// ---------------------------------------------------------------------------
// Code -> fp16 conversion without per-element converts.
//
// For a nibble u in [0, 15], the binary16 pattern 0x6400 | u is exactly
// 1024 + u, and 0x6400 | (u << 4) is exactly 1024 + 16u. Flipping bit 3 of
// every nibble first (u = v ^ 8) makes u - 8 the signed code. So with one
// AND-OR per pair of codes and one packed fp16 op per pair we get the exact
// integer codes as fp16 (|code| <= 8 is exact in fp16).
// ---------------------------------------------------------------------------

// "Spread" order: from one word d of 8 codes c0..c7 produce four fp16 pairs
//   (c0, c4), (c1, c5), (c2, c6), (c3, c7).
// Since the masked code bits and the exponent bits 0x6400 do not overlap,
// ((d & mask) ^ 8-per-code) | 0x6400 == (d & mask) ^ (0x6400 | 8-per-code):
// one AND-XOR (a single v_bitop3_b32 on gfx950) per pair, plus one packed fp16
// op per pair and one shift per word -- 9 VALU ops per 8 codes. The matching
// activations must be arranged in the same order (see spread_perm_x).
__device__ __forceinline__ void codes_to_half_spread(uint32_t d, half2_t out[4]) {
  const uint32_t v = d >> 8;
  const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  out[0] = __builtin_bit_cast(half2_t, (d & 0x000F000Fu) ^ 0x64086408u) + bias;
  out[1] = __builtin_elementwise_fma(
      __builtin_bit_cast(half2_t, (d & 0x00F000F0u) ^ 0x64806480u), sixteenth, bias16);
  out[2] = __builtin_bit_cast(half2_t, (v & 0x000F000Fu) ^ 0x64086408u) + bias;
  out[3] = __builtin_elementwise_fma(
      __builtin_bit_cast(half2_t, (v & 0x00F000F0u) ^ 0x64806480u), sixteenth, bias16);
}

// Natural order: from one word d of 8 codes produce (c0,c1), (c2,c3), (c4,c5),
// (c6,c7). Byte b (codes 2b, 2b+1) is copied into both 16-bit halves with a
// byte permute, then the low half keeps bits 0..3 and the high half bits 4..7
// (AND-XOR with the exponent and the flipped sign bits, as above).
// 12 VALU ops per 8 codes.
__device__ __forceinline__ void codes_to_half_natural(uint32_t d, half2_t out[4]) {
  const half2_t scale = {(_Float16)1.0f, (_Float16)0.0625f};
  const half2_t bias = {(_Float16)-1032.0f, (_Float16)-72.0f};
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // v_perm_b32 selector: result bytes = [d.b, 0, d.b, 0]
    const uint32_t sel = (uint32_t)b | 0x0C000C00u | ((uint32_t)b << 16);
    const uint32_t dup = __builtin_amdgcn_perm(0u, d, sel);
    out[b] = __builtin_elementwise_fma(
        __builtin_bit_cast(half2_t, (dup & 0x00F0000Fu) ^ 0x64806408u), scale, bias);
  }
}

// ---------------------------------------------------------------------------
// Affine codes ("Build a Blockwise INT4 Inference Engine", step 2: an unsigned
// code u in [0, 15] and a per-group zero point zp, value u - zp).
//
// The same bit trick without the flip of bit 3 gives 1024 + u (and
// 1024 + 16u, i.e. 64 + u after the 1/16 scaling), so a per-group bias of
// -(1024 + zp) (resp. -(64 + zp)) leaves u - zp exactly. For zp in [0, 15]
// the binary16 patterns are -(1024 + zp) = 0xE400 | zp and -(64 + zp) =
// 0xD400 | (zp << 4): the bias words are a few integer ops per group.
// ---------------------------------------------------------------------------

// Natural-order bias pair {-(1024 + zp), -(64 + zp)} (low, high half).
__device__ __forceinline__ uint32_t zp_bias_natural(uint32_t zp) {
  return 0xD400E400u | zp | (zp << 20);
}
// Spread-order bias pairs: {-(1024 + zp)} x 2 and {-(64 + zp)} x 2.
__device__ __forceinline__ uint32_t zp_bias_lo(uint32_t zp) { return 0xE400E400u | zp | (zp << 16); }
__device__ __forceinline__ uint32_t zp_bias_hi(uint32_t zp) {
  return 0xD400D400u | (zp << 4) | (zp << 20);
}

// codes_to_half_spread for affine codes: (c0 - zp, c4 - zp), ... (9 VALU ops
// per 8 codes, like the symmetric form).
__device__ __forceinline__ void codes_to_half_spread_zp(uint32_t d, half2_t out[4], uint32_t blo,
                                                        uint32_t bhi) {
  const uint32_t v = d >> 8;
  const half2_t b0 = __builtin_bit_cast(half2_t, blo), b1 = __builtin_bit_cast(half2_t, bhi);
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  out[0] = __builtin_bit_cast(half2_t, (d & 0x000F000Fu) | 0x64006400u) + b0;
  out[1] = __builtin_elementwise_fma(
      __builtin_bit_cast(half2_t, (d & 0x00F000F0u) | 0x64006400u), sixteenth, b1);
  out[2] = __builtin_bit_cast(half2_t, (v & 0x000F000Fu) | 0x64006400u) + b0;
  out[3] = __builtin_elementwise_fma(
      __builtin_bit_cast(half2_t, (v & 0x00F000F0u) | 0x64006400u), sixteenth, b1);
}

// codes_to_half_natural for affine codes: (c0 - zp, c1 - zp), ... with the
// bias pair from zp_bias_natural.
__device__ __forceinline__ void codes_to_half_natural_zp(uint32_t d, half2_t out[4], uint32_t bnat) {
  const half2_t scale = {(_Float16)1.0f, (_Float16)0.0625f};
  const half2_t bias = __builtin_bit_cast(half2_t, bnat);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t sel = (uint32_t)b | 0x0C000C00u | ((uint32_t)b << 16);
    const uint32_t dup = __builtin_amdgcn_perm(0u, d, sel);
    out[b] = __builtin_elementwise_fma(
        __builtin_bit_cast(half2_t, (dup & 0x00F0000Fu) | 0x64006400u), scale, bias);
  }
}

// Rearrange 8 consecutive fp16 activations (x0..x7, natural order in 4 words)
// into the spread order (x0,x4),(x1,x5),(x2,x6),(x3,x7).
__device__ __forceinline__ u32x4_t spread_perm_x(u32x4_t n) {
  u32x4_t r;
  r.x = __builtin_amdgcn_perm(n.z, n.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(n.z, n.x, 0x07060302u);
  r.z = __builtin_amdgcn_perm(n.w, n.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(n.w, n.y, 0x07060302u);
  return r;
}

__device__ __forceinline__ half8_t as_half8(const half2_t h[4]) {
  u32x4_t w;
  w.x = __builtin_bit_cast(uint32_t, h[0]);
  w.y = __builtin_bit_cast(uint32_t, h[1]);
  w.z = __builtin_bit_cast(uint32_t, h[2]);
  w.w = __builtin_bit_cast(uint32_t, h[3]);
  return __builtin_bit_cast(half8_t, w);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses
// (lgkmcnt) and then for all waves. Unlike __syncthreads() it does not wait
// for outstanding global loads, so weight prefetches stay in flight across it.
// The "memory" clobber keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// A dispatch holds fewer than 2^32 work items along each grid dimension, so a
// grid of one thread (or one wavefront) per element stops launching at a few
// billion elements, which one 288 GB device can hold. The element-wise kernels
// therefore walk their elements with the grid's stride over at most this many
// blocks of 256 threads (16.8 M threads, many times what the CUs hold at once).
constexpr int64_t kStrideBlocks = int64_t(1) << 16;

// Grid size for a kernel that would want `blocks` blocks, capped as above.
inline unsigned stride_grid(int64_t blocks) {
  return (unsigned)(blocks < kStrideBlocks ? (blocks > 0 ? blocks : 1) : kStrideBlocks);
}

}  // namespace int4dq
