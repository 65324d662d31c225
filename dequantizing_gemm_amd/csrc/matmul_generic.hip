// matmul_generic.hip -- general dequantizing matmul (any M, N, K, group,
// alignment; binary32 or binary16 activations; symmetric or affine codes) on
// the vector ALUs.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, int4_matmul):
//   y[m, n] = sum over groups gi of scale[n, gi] * (sum over k in gi of x[m, k] * q[n, k])
// i.e. x times the group's integer codes first, then the group's scale. With
// affine codes ("Build a Blockwise INT4 Inference Engine", step 2) the integer
// weight is the unsigned code minus the group's zero point.
//
// One wavefront per output y[m, n] (the grid strides over the outputs). The
// wavefront walks the groups of row n;
// inside a group the 64 lanes stride over k (coalesced reads of x and of the
// packed bytes), each lane forms its share of the group's integer-weighted sum
// in fp32 and multiplies it by the group's scale; the lane sums are reduced at
// the end. This path exists for shapes and dtypes the MFMA kernels do not
// take (binary32 x, odd K, unaligned rows, group sizes other than 32, 64 or a
// multiple of 128); it is not the fast path.
#include "device_common.h"
#include "kernels.h"

namespace int4dq {

template <typename XT>
__device__ __forceinline__ float load_x(const XT* p) { return (float)*p; }

template <typename XT, bool AFF>
__global__ __launch_bounds__(256) void matmul_generic_kernel(
    const XT* __restrict__ x, int64_t M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t N, int64_t K,
    int64_t group, int64_t G,
    void* __restrict__ y, Epilogue ep) {
  const int lane = threadIdx.x & (kWave - 1);
  // the output index is uniform over the wavefront, so whole wavefronts
  // leave the loop together
  for (int64_t out = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); out < M * N;
       out += (int64_t)gridDim.x * 4) {
    const int64_t m = out / N, n = out - m * N;
    const XT* xr = x + m * K;
    const uint8_t* pr = packed + n * ((K + 1) >> 1);
    const uint16_t* sr = scales + n * G;
    float acc = 0.0f;
    for (int64_t gi = 0; gi < G; ++gi) {
      const int64_t k0 = gi * group;
      const int64_t k1 = k0 + group < K ? k0 + group : K;
      float part = 0.0f;
      const int zp = AFF ? (int)zeros[n * G + gi] : 0;
      for (int64_t k = k0 + lane; k < k1; k += kWave) {
        const uint32_t byte = pr[k >> 1];
        const uint32_t u = (byte >> (4 * (int)(k & 1))) & 0xFu;
        const int q = AFF ? (int)u - zp : sx4(u);
        part = __builtin_fmaf(load_x(xr + k), (float)q, part);
      }
      acc = __builtin_fmaf(half_bits_to_float(sr[gi]), part, acc);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) ep.store(y, m * N + n, acc, n);
  }
}

template <typename XT, bool AFF>
static void launch_generic_t(const void* x, int64_t M, const uint8_t* packed,
                             const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                             int64_t group, void* y, Epilogue ep, hipStream_t stream) {
  const int64_t G = (K + group - 1) / group;
  const int64_t outs = M * N;
  const dim3 grid(stride_grid((outs + 3) / 4)), block(256);   // one wavefront per output
  hipLaunchKernelGGL((matmul_generic_kernel<XT, AFF>), grid, block, 0, stream,
                     static_cast<const XT*>(x), M, packed, scales, zeros, N, K, group, G, y, ep);
}

hipError_t launch_matmul_generic(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                                 const uint16_t* scales, const uint8_t* zeros, int64_t N,
                                 int64_t K, int64_t group, void* y, Epilogue ep,
                                 hipStream_t stream) {
  if (x_dtype == 0) {
    if (zeros) launch_generic_t<float, true>(x, M, packed, scales, zeros, N, K, group, y, ep, stream);
    else launch_generic_t<float, false>(x, M, packed, scales, zeros, N, K, group, y, ep, stream);
  } else {
    if (zeros) launch_generic_t<_Float16, true>(x, M, packed, scales, zeros, N, K, group, y, ep, stream);
    else launch_generic_t<_Float16, false>(x, M, packed, scales, zeros, N, K, group, y, ep, stream);
  }
  return hipGetLastError();
}

}  // namespace int4dq
