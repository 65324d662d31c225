// api.cpp -- the C ABI declared in include/int4dq.h: argument validation,
// kernel selection, launch on the caller's stream, and the thread-local error
// text. No HIP call is made before the arguments have been validated, so
// every invalid-argument path can be exercised on a host without a GPU.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdarg.h>

#include <mutex>

#include "../../include/int4dq.h"
#include "kernels.h"

// Scratch of int4_linear_noalloc: the workspace of a split of K for callers
// that cannot allocate. Every GPU the library runs on holds its own copy, from
// module load to the end of the process. The split plans need at most
// 16 MiB (the tiled kernel's: four shares of a [512, 2048] binary32 result,
// or eight of a quarter of that; the skinny kernel's: at most eight shares of
// a [64, 2032] result, 4 MiB), so the array is that size. In host code its name is only a
// stand-in: the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[16 << 20];

namespace {

constexpr int64_t kScratchBytes = 16 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};         // device address of scratch, per device

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return INT4DQ_OK;
}

// a * b with overflow check into *out (both non-negative).
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(INT4DQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Shared validation of int4_matmul arguments; on success fills the sizes.
int check_matmul(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                 const uint16_t* scales, int64_t N, int64_t K, int64_t group, const void* y) {
  if (M < 0) return fail(INT4DQ_EINVAL, "int4_matmul: M must be >= 0 (got %lld)", (long long)M);
  if (N < 1 || K < 1) return fail(INT4DQ_EINVAL, "int4_matmul: N and K must be >= 1 (got N=%lld K=%lld)", (long long)N, (long long)K);
  if (group < 1) return fail(INT4DQ_EINVAL, "int4_matmul: group must be >= 1 (got %lld)", (long long)group);
  if (x_dtype != INT4DQ_X_F32 && x_dtype != INT4DQ_X_F16)
    return fail(INT4DQ_EINVAL, "int4_matmul: unknown x_dtype %d", x_dtype);
  int64_t t;
  const int64_t G = (K + group - 1) / group;
  if (!mul_ok(M, K, &t) || !mul_ok(t, 4, &t) || !mul_ok(M, N, &t) || !mul_ok(t, 4, &t) ||
      !mul_ok(N, (K + 1) / 2, &t) || !mul_ok(N, G, &t) || !mul_ok(t, 2, &t))
    return fail(INT4DQ_EINVAL, "int4_matmul: sizes overflow int64");
  if (!packed || !scales) return fail(INT4DQ_EINVAL, "int4_matmul: packed and scales must be non-NULL");
  if (M > 0 && (!x || !y)) return fail(INT4DQ_EINVAL, "int4_matmul: x and y must be non-NULL when M > 0");
  return INT4DQ_OK;
}

// Shared body of every matmul entry point (zeros: nullptr for symmetric
// codes; y of y_dtype).
int matmul_impl(const char* fn, const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int64_t group,
                const float* bias, int act, void* y, int y_dtype, int path, void* stream,
                void* workspace = nullptr, int64_t workspace_bytes = 0);

int choose_path(const void* x, int x_dtype, int64_t M, const uint8_t* packed, int64_t N,
                int64_t K, int64_t group) {
  if (!int4dq::matmul_gemv_unsupported(x_dtype, M, x, packed, N, K, group)) return INT4DQ_PATH_GEMV;
  if (!int4dq::matmul_skinny_unsupported(x_dtype, M, x, packed, N, K, group) &&
      int4dq::matmul_skinny_preferred(M, N))
    return INT4DQ_PATH_SKINNY;
  if (!int4dq::matmul_tiled_unsupported(x_dtype, M, x, packed, N, K, group)) return INT4DQ_PATH_TILED;
  return INT4DQ_PATH_GENERIC;
}

int dequantize_impl(const char* fn, const uint8_t* packed, const uint16_t* scales,
                    const uint8_t* zeros, int64_t N, int64_t K, int64_t group, int out_dtype,
                    void* out, void* stream) {
  if (N < 1 || K < 1) return fail(INT4DQ_EINVAL, "%s: N and K must be >= 1 (got N=%lld K=%lld)", fn, (long long)N, (long long)K);
  if (group < 1) return fail(INT4DQ_EINVAL, "%s: group must be >= 1 (got %lld)", fn, (long long)group);
  if (out_dtype != INT4DQ_OUT_F32 && out_dtype != INT4DQ_OUT_F16)
    return fail(INT4DQ_EINVAL, "%s: unknown out_dtype %d", fn, out_dtype);
  int64_t t;
  if (!mul_ok(N, K, &t) || !mul_ok(t, 4, &t) || !mul_ok(N, (K + group - 1) / group, &t) || !mul_ok(t, 2, &t))
    return fail(INT4DQ_EINVAL, "%s: sizes overflow int64", fn);
  if (!packed || !scales || !out) return fail(INT4DQ_EINVAL, "%s: packed, scales and out must be non-NULL", fn);
  return hip_status(int4dq::launch_dequantize(packed, scales, zeros, N, K, group, out_dtype == INT4DQ_OUT_F16,
                                              out, (hipStream_t)stream),
                    "int4_dequantize launch");
}

}  // namespace

extern "C" {

int64_t int4_num_groups(int64_t K, int64_t group) {
  if (K < 1 || group < 1) return -1;
  return K / group + (K % group != 0);
}

int64_t int4_packed_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1) return -1;
  int64_t t;
  if (!mul_ok(N, K / 2 + (K % 2), &t)) return -1;
  return t;
}

int int4_quantize(const float* w, int64_t N, int64_t K, int64_t group, uint8_t* packed,
                  uint16_t* scales, void* stream) {
  if (N < 1 || K < 1) return fail(INT4DQ_EINVAL, "int4_quantize: N and K must be >= 1 (got N=%lld K=%lld)", (long long)N, (long long)K);
  if (group < 1) return fail(INT4DQ_EINVAL, "int4_quantize: group must be >= 1 (got %lld)", (long long)group);
  int64_t t;
  if (!mul_ok(N, K, &t) || !mul_ok(t, 4, &t) || !mul_ok(N, (K + group - 1) / group, &t) || !mul_ok(t, 2, &t))
    return fail(INT4DQ_EINVAL, "int4_quantize: sizes overflow int64");
  if (!w || !packed || !scales) return fail(INT4DQ_EINVAL, "int4_quantize: w, packed and scales must be non-NULL");
  return hip_status(int4dq::launch_quantize(w, N, K, group, packed, scales, (hipStream_t)stream),
                    "int4_quantize launch");
}

int int4_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* out, void* stream) {
  if (N < 1 || K < 1) return fail(INT4DQ_EINVAL, "int4_unpack: N and K must be >= 1 (got N=%lld K=%lld)", (long long)N, (long long)K);
  int64_t t;
  if (!mul_ok(N, K, &t)) return fail(INT4DQ_EINVAL, "int4_unpack: sizes overflow int64");
  if (!packed || !out) return fail(INT4DQ_EINVAL, "int4_unpack: packed and out must be non-NULL");
  return hip_status(int4dq::launch_unpack(packed, N, K, out, (hipStream_t)stream), "int4_unpack launch");
}

int int4_dequantize(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K,
                    int64_t group, int out_dtype, void* out, void* stream) {
  return dequantize_impl("int4_dequantize", packed, scales, nullptr, N, K, group, out_dtype, out, stream);
}

int int4_dequantize_affine(const uint8_t* packed, const uint16_t* scales, const uint8_t* zeros,
                           int64_t N, int64_t K, int64_t group, int out_dtype, void* out,
                           void* stream) {
  if (!zeros) return fail(INT4DQ_EINVAL, "int4_dequantize_affine: zeros must be non-NULL");
  return dequantize_impl("int4_dequantize_affine", packed, scales, zeros, N, K, group, out_dtype, out, stream);
}

int int4_quantize_affine(const float* w, int64_t N, int64_t K, int64_t group, uint8_t* packed,
                         uint16_t* scales, uint8_t* zeros, void* stream) {
  if (N < 1 || K < 1) return fail(INT4DQ_EINVAL, "int4_quantize_affine: N and K must be >= 1 (got N=%lld K=%lld)", (long long)N, (long long)K);
  if (group < 1) return fail(INT4DQ_EINVAL, "int4_quantize_affine: group must be >= 1 (got %lld)", (long long)group);
  int64_t t;
  if (!mul_ok(N, K, &t) || !mul_ok(t, 4, &t) || !mul_ok(N, (K + group - 1) / group, &t) || !mul_ok(t, 2, &t))
    return fail(INT4DQ_EINVAL, "int4_quantize_affine: sizes overflow int64");
  if (!w || !packed || !scales || !zeros)
    return fail(INT4DQ_EINVAL, "int4_quantize_affine: w, packed, scales and zeros must be non-NULL");
  return hip_status(int4dq::launch_quantize_affine(w, N, K, group, packed, scales, zeros, (hipStream_t)stream),
                    "int4_quantize_affine launch");
}

int int4_matmul_path(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                     const uint16_t* scales, int64_t N, int64_t K, int64_t group,
                     const float* bias, int act, float* y, int path, void* stream) {
  return matmul_impl("int4_matmul_path", x, x_dtype, M, packed, scales, nullptr, N, K, group, bias,
                     act, y, INT4DQ_Y_F32, path, stream);
}

int int4_matmul_affine(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                       const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                       int64_t group, const float* bias, int act, float* y, int path, void* stream) {
  if (!zeros) return fail(INT4DQ_EINVAL, "int4_matmul_affine: zeros must be non-NULL");
  return matmul_impl("int4_matmul_affine", x, x_dtype, M, packed, scales, zeros, N, K, group, bias,
                     act, y, INT4DQ_Y_F32, path, stream);
}

int int4_linear(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int64_t group,
                const float* bias, int act, void* y, int y_dtype, void* stream) {
  return matmul_impl("int4_linear", x, x_dtype, M, packed, scales, zeros, N, K, group, bias, act, y,
                     y_dtype, INT4DQ_PATH_AUTO, stream);
}

int64_t int4_linear_workspace_bytes(int x_dtype, int64_t M, int64_t N, int64_t K, int64_t group) {
  if (M < 0 || N < 1 || K < 1 || group < 1 || (x_dtype != INT4DQ_X_F32 && x_dtype != INT4DQ_X_F16)) return -1;
  if (M == 0) return 0;
  // The kernel choice of an aligned call (the skinny and tiled kernels split K).
  static const uint8_t aligned_probe[16] __attribute__((aligned(16))) = {0};
  const int path = choose_path(aligned_probe, x_dtype, M, aligned_probe, N, K, group);
  if (path == INT4DQ_PATH_SKINNY) return int4dq::matmul_skinny_workspace(M, N, K, group);
  if (path == INT4DQ_PATH_TILED) return int4dq::matmul_tiled_workspace(M, N, K, group);
  return 0;
}

int int4_linear_ws(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                   const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int64_t group,
                   const float* bias, int act, void* y, int y_dtype, void* workspace,
                   int64_t workspace_bytes, void* stream) {
  if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace))
    return fail(INT4DQ_EINVAL, "int4_linear_ws: workspace_bytes must be >= 0, with a non-NULL workspace when > 0");
  if ((uintptr_t)workspace % 256)
    return fail(INT4DQ_EINVAL, "int4_linear_ws: workspace must be 256-byte aligned");
  return matmul_impl("int4_linear_ws", x, x_dtype, M, packed, scales, zeros, N, K, group, bias, act, y,
                     y_dtype, INT4DQ_PATH_AUTO, stream, workspace, workspace_bytes);
}

int int4_linear_noalloc(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                        const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                        int64_t group, const float* bias, int act, void* y, int y_dtype, void* stream) {
  const int rc = check_matmul(x, x_dtype, M, packed, scales, N, K, group, y);
  if (rc != INT4DQ_OK) return rc;
  const int64_t need = int4_linear_workspace_bytes(x_dtype, M, N, K, group);
  if (need > kScratchBytes)
    return fail(INT4DQ_EINVAL, "int4_linear_noalloc: this shape needs %lld bytes of scratch, more than the "
                               "%lld the library holds per device", (long long)need, (long long)kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "int4_linear_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
      return fail(INT4DQ_EUNSUPPORTED, "int4_linear_noalloc: device %d is beyond the %d the scratch table holds",
                  dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {                 // once per device, with that device current
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, "int4_linear_noalloc: hipGetSymbolAddress(scratch)");
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  return matmul_impl("int4_linear_noalloc", x, x_dtype, M, packed, scales, zeros, N, K, group, bias, act, y,
                     y_dtype, INT4DQ_PATH_AUTO, stream, ws, ws ? kScratchBytes : 0);
}

int int4_matmul(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                const uint16_t* scales, int64_t N, int64_t K, int64_t group, float* y,
                void* stream) {
  return int4_matmul_path(x, x_dtype, M, packed, scales, N, K, group, nullptr, INT4DQ_ACT_NONE, y,
                          INT4DQ_PATH_AUTO, stream);
}

int int4_matmul_ex(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                   const uint16_t* scales, int64_t N, int64_t K, int64_t group,
                   const float* bias, int act, float* y, void* stream) {
  return int4_matmul_path(x, x_dtype, M, packed, scales, N, K, group, bias, act, y,
                          INT4DQ_PATH_AUTO, stream);
}

int int4_matmul_select(const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                       const uint16_t* scales, int64_t N, int64_t K, int64_t group,
                       const float* y) {
  if (check_matmul(x, x_dtype, M, packed, scales, N, K, group, y) != INT4DQ_OK) return -1;
  return choose_path(x, x_dtype, M, packed, N, K, group);
}

const char* int4_last_error(void) { return g_err; }

}  // extern "C"

namespace {

int matmul_impl(const char* fn, const void* x, int x_dtype, int64_t M, const uint8_t* packed,
                const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K, int64_t group,
                const float* bias, int act, void* y, int y_dtype, int path, void* stream,
                void* workspace, int64_t workspace_bytes) {
  int rc = check_matmul(x, x_dtype, M, packed, scales, N, K, group, y);
  if (rc != INT4DQ_OK) return rc;
  if (act != INT4DQ_ACT_NONE && act != INT4DQ_ACT_RELU)
    return fail(INT4DQ_EINVAL, "%s: unknown activation %d", fn, act);
  if (y_dtype != INT4DQ_Y_F32 && y_dtype != INT4DQ_Y_F16)
    return fail(INT4DQ_EINVAL, "%s: unknown y_dtype %d", fn, y_dtype);
  const int4dq::Epilogue ep{bias, act == INT4DQ_ACT_RELU ? 1 : 0, y_dtype == INT4DQ_Y_F16 ? 1 : 0};
  if (path < INT4DQ_PATH_AUTO || path > INT4DQ_PATH_GEMV)
    return fail(INT4DQ_EINVAL, "%s: unknown path %d", fn, path);
  if (M == 0) return ok();
  if (path == INT4DQ_PATH_AUTO) path = choose_path(x, x_dtype, M, packed, N, K, group);
  const hipStream_t s = (hipStream_t)stream;
  switch (path) {
    case INT4DQ_PATH_SKINNY: {
      const char* why = int4dq::matmul_skinny_unsupported(x_dtype, M, x, packed, N, K, group);
      if (why) return fail(INT4DQ_EUNSUPPORTED, "%s: %s", fn, why);
      return hip_status(int4dq::launch_matmul_skinny(x, M, packed, scales, zeros, N, K, group, y, ep,
                                                     workspace, workspace_bytes, s),
                        "int4_matmul skinny launch");
    }
    case INT4DQ_PATH_GEMV: {
      const char* why = int4dq::matmul_gemv_unsupported(x_dtype, M, x, packed, N, K, group);
      if (why) return fail(INT4DQ_EUNSUPPORTED, "%s: %s", fn, why);
      return hip_status(int4dq::launch_matmul_gemv(x, M, packed, scales, zeros, N, K, group, y, ep, s),
                        "int4_matmul gemv launch");
    }
    case INT4DQ_PATH_TILED: {
      const char* why = int4dq::matmul_tiled_unsupported(x_dtype, M, x, packed, N, K, group);
      if (why) return fail(INT4DQ_EUNSUPPORTED, "%s: %s", fn, why);
      return hip_status(int4dq::launch_matmul_tiled(x, M, packed, scales, zeros, N, K, group, y, ep,
                                                    workspace, workspace_bytes, s),
                        "int4_matmul tiled launch");
    }
    default:
      return hip_status(int4dq::launch_matmul_generic(x, x_dtype, M, packed, scales, zeros, N, K, group, y, ep, s),
                        "int4_matmul generic launch");
  }
}

}  // namespace
