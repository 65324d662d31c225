// stub_launchers.cpp -- host stand-ins for the kernel launchers and kernel
// choice functions that api.cpp calls (dequantizing_gemm_amd/csrc/kernels.h),
// for the sanitizer build of the C ABI on a machine without a GPU: each
// records its call and launches nothing. What the choice functions answer is
// set by the driver through the stub_* globals.
//
// Test infrastructure: built only by tests/test_sanitize_cpu.py.
#include "../../dequantizing_gemm_amd/csrc/kernels.h"

int stub_calls[8];                 // per launcher: quantize, quantize_affine, unpack, dequantize,
                                   // generic, skinny, gemv, tiled
int64_t stub_last_M = -1, stub_last_ws_bytes = -1;
void* stub_last_ws = nullptr;
bool stub_gemv_ok = true, stub_skinny_ok = true, stub_skinny_pref = true, stub_tiled_ok = true;
int64_t stub_tiled_ws = 0;         // what matmul_tiled_workspace answers
int64_t stub_skinny_ws = 0;        // what matmul_skinny_workspace answers

namespace int4dq {

hipError_t launch_quantize(const float*, int64_t, int64_t, int64_t, uint8_t*, uint16_t*, hipStream_t) {
  ++stub_calls[0];
  return hipSuccess;
}
hipError_t launch_quantize_affine(const float*, int64_t, int64_t, int64_t, uint8_t*, uint16_t*, uint8_t*,
                                  hipStream_t) {
  ++stub_calls[1];
  return hipSuccess;
}
hipError_t launch_unpack(const uint8_t*, int64_t, int64_t, int8_t*, hipStream_t) {
  ++stub_calls[2];
  return hipSuccess;
}
hipError_t launch_dequantize(const uint8_t*, const uint16_t*, const uint8_t*, int64_t, int64_t, int64_t, bool,
                             void*, hipStream_t) {
  ++stub_calls[3];
  return hipSuccess;
}
hipError_t launch_matmul_generic(const void*, int, int64_t M, const uint8_t*, const uint16_t*, const uint8_t*,
                                 int64_t, int64_t, int64_t, void*, Epilogue, hipStream_t) {
  ++stub_calls[4];
  stub_last_M = M;
  return hipSuccess;
}
const char* matmul_skinny_unsupported(int, int64_t, const void*, const uint8_t*, int64_t, int64_t, int64_t) {
  return stub_skinny_ok ? nullptr : "skinny stub refuses";
}
bool matmul_skinny_preferred(int64_t, int64_t) { return stub_skinny_pref; }
hipError_t launch_matmul_skinny(const void*, int64_t M, const uint8_t*, const uint16_t*, const uint8_t*, int64_t,
                                int64_t, int64_t, void*, Epilogue, void* workspace, int64_t workspace_bytes,
                                hipStream_t) {
  ++stub_calls[5];
  stub_last_M = M;
  stub_last_ws = workspace;
  stub_last_ws_bytes = workspace_bytes;
  return hipSuccess;
}
int64_t matmul_skinny_workspace(int64_t, int64_t, int64_t, int64_t) { return stub_skinny_ws; }
const char* matmul_gemv_unsupported(int, int64_t, const void*, const uint8_t*, int64_t, int64_t, int64_t) {
  return stub_gemv_ok ? nullptr : "gemv stub refuses";
}
hipError_t launch_matmul_gemv(const void*, int64_t M, const uint8_t*, const uint16_t*, const uint8_t*, int64_t,
                              int64_t, int64_t, void*, Epilogue, hipStream_t) {
  ++stub_calls[6];
  stub_last_M = M;
  return hipSuccess;
}
const char* matmul_tiled_unsupported(int, int64_t, const void*, const uint8_t*, int64_t, int64_t, int64_t) {
  return stub_tiled_ok ? nullptr : "tiled stub refuses";
}
hipError_t launch_matmul_tiled(const void*, int64_t M, const uint8_t*, const uint16_t*, const uint8_t*, int64_t,
                               int64_t, int64_t, void*, Epilogue, void* workspace, int64_t workspace_bytes,
                               hipStream_t) {
  ++stub_calls[7];
  stub_last_M = M;
  stub_last_ws = workspace;
  stub_last_ws_bytes = workspace_bytes;
  return hipSuccess;
}
int64_t matmul_tiled_workspace(int64_t, int64_t, int64_t, int64_t) { return stub_tiled_ws; }

}  // namespace int4dq
