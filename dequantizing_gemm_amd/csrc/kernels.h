// kernels.h -- internal launch functions behind the C ABI (include/int4dq.h).
// Arguments here are already validated by api.cpp; these functions only pick a
// kernel variant and enqueue it on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace int4dq {

// Output step of every matmul kernel (the engine page's fused kernel and
// layer forward): y = act(v + bias[n]) with act = identity or ReLU; ReLU keeps
// a value greater than zero and gives +0 otherwise. y is binary32, or binary16
// (the fp32 result rounded to nearest even) so that a following layer can take
// it as its activations without a conversion pass.
struct Epilogue {
  const float* bias;   // [N] binary32, or nullptr
  int relu;            // 0 or 1
  int half;            // 1: y is binary16, 0: binary32
  // The bias of output column n (0 when there is none), read once per column
  // by kernels that store many outputs of one column: the compiler cannot
  // prove that the stores to y leave the bias unchanged, and would otherwise
  // reload it before every store.
  __device__ __forceinline__ float column(int64_t n) const { return bias ? bias[n] : 0.0f; }
  __device__ __forceinline__ float apply(float v, float b) const {
    if (bias) v += b;
    return relu ? (v > 0.0f ? v : 0.0f) : v;
  }
  __device__ __forceinline__ float operator()(float v, int64_t n) const { return apply(v, column(n)); }
  // y[i] = act(v + bias[n]) in y's precision.
  __device__ __forceinline__ void store(void* y, int64_t i, float v, int64_t n) const {
    const float r = apply(v, column(n));
    if (half) static_cast<_Float16*>(y)[i] = (_Float16)r;
    else static_cast<float*>(y)[i] = r;
  }
};

// Split of K for the tiled kernel: S shares of `steps` sub-steps each, whose
// partial tiles go to part ([S, M, N] binary32). S = 1: no split, part unused.
struct TiledSplit {
  float* part;
  int S;
  int steps;
};

// Split of K for the skinny kernel: S shares of kb_per_share K-blocks each
// (blockIdx.y is the share), whose partial tiles go to part ([S, M, N]
// binary32). S = 1: no split, part unused.
struct SkinnySplit {
  float* part;
  int S;
  int kb_per_share;
};

// y[m, n] = act(sum over shares q = 0 .. S-1, in that order, of
// part[q, m, n] + bias[n]) in y's precision: the second step of every split
// of K.
hipError_t launch_split_reduce(const float* part, int S, int64_t M, int64_t N, void* y, Epilogue ep,
                               hipStream_t stream);

hipError_t launch_quantize(const float* w, int64_t N, int64_t K, int64_t group, uint8_t* packed,
                           uint16_t* scales, hipStream_t stream);

// Affine codes (unsigned nibbles, one zero point byte per group).
hipError_t launch_quantize_affine(const float* w, int64_t N, int64_t K, int64_t group,
                                  uint8_t* packed, uint16_t* scales, uint8_t* zeros,
                                  hipStream_t stream);

hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* out,
                         hipStream_t stream);

// zeros: nullptr for symmetric codes, else [N, G] zero points (affine codes),
// here and in every matmul launcher below.
hipError_t launch_dequantize(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros,
                             int64_t N, int64_t K, int64_t group, bool half, void* out,
                             hipStream_t stream);

hipError_t launch_matmul_generic(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                                 const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int64_t group,
                                 void* y, Epilogue ep, hipStream_t stream);

// nullptr if the kernel takes these arguments, else the reason it does not.
const char* matmul_skinny_unsupported(int x_dtype, int64_t M, const void* x,
                                      const uint8_t* packed, int64_t N, int64_t K, int64_t group);
// Whether the automatic choice takes the skinny kernel for a supported shape.
bool matmul_skinny_preferred(int64_t M, int64_t N);
// workspace: nullptr, or workspace_bytes of device memory for a split of K
// (any contents), taken only when it holds matmul_skinny_workspace(M, N, K,
// group) bytes; that is 0 when the shape is not split.
hipError_t launch_matmul_skinny(const void* x, int64_t M, const uint8_t* packed,
                                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int64_t group,
                                void* y, Epilogue ep, void* workspace, int64_t workspace_bytes,
                                hipStream_t stream);
int64_t matmul_skinny_workspace(int64_t M, int64_t N, int64_t K, int64_t group);

const char* matmul_gemv_unsupported(int x_dtype, int64_t M, const void* x,
                                    const uint8_t* packed, int64_t N, int64_t K, int64_t group);
hipError_t launch_matmul_gemv(const void* x, int64_t M, const uint8_t* packed, const uint16_t* scales,
                              const uint8_t* zeros, int64_t N, int64_t K, int64_t group, void* y, Epilogue ep,
                              hipStream_t stream);

const char* matmul_tiled_unsupported(int x_dtype, int64_t M, const void* x, const uint8_t* packed,
                                     int64_t N, int64_t K, int64_t group);
// workspace: nullptr, or workspace_bytes of device memory for a split of K
// (any contents). The split is taken only when the workspace holds
// matmul_tiled_workspace(M, N, K, group) bytes; that is 0 when the shape is
// not split.
hipError_t launch_matmul_tiled(const void* x, int64_t M, const uint8_t* packed,
                               const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int64_t group,
                               void* y, Epilogue ep, void* workspace, int64_t workspace_bytes,
                               hipStream_t stream);
int64_t matmul_tiled_workspace(int64_t M, int64_t N, int64_t K, int64_t group);

}  // namespace int4dq
