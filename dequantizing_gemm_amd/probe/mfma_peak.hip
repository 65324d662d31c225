// mfma_peak.hip -- measurement probe, not part of the library's path: the
// dense binary16 matrix-core rate the chip sustains when it does nothing else,
// the ceiling the MFMA-bound matmul is compared with beside the nominal peak.
//
// Every wavefront runs eight independent accumulator chains of
// v_mfma_f32_32x32x16_f16 (the instruction the tiled matmul uses) on nonzero
// operands that differ per lane, with no memory traffic in the loop. The
// accumulators are folded at the end and written only if the fold equals a
// constant that these operands never give, which keeps every MFMA.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  half8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.0625f + 0.001953125f * (float)((lane + i) & 15));
    b[i] = (_Float16)(0.03125f - 0.0009765625f * (float)((lane * 3 + i) & 15));
  }
  float16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == -1234.5f) sink[0] = s;
}

}  // namespace

// Launches `blocks` blocks of four wavefronts, each running `iters` rounds of
// eight 32x32x16 binary16 MFMAs: blocks * 4 * iters * 8 * 32768 flops. sink:
// one device float, written only in the case above. Returns a hipError_t as
// int.
extern "C" int int4dq_probe_mfma(int blocks, int iters, void* sink, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, iters,
                     static_cast<float*>(sink));
  return (int)hipGetLastError();
}
