// api_driver.cpp -- drives the C ABI (include/int4dq.h, implemented in
// dequantizing_gemm_amd/csrc/api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with the kernel launchers replaced by the host
// stubs of stub_launchers.cpp: every argument check, the int64 overflow
// checks, the size helpers, the path choice, the workspace checks of the
// split-of-K calls and the per-thread error text. Pointers passed to calls
// that pass validation are never dereferenced (the stubs launch nothing).
//
// Test infrastructure: built and run only by tests/test_sanitize_cpu.py.
// Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <thread>

#include "../../include/int4dq.h"

extern int stub_calls[8];
extern int64_t stub_last_M, stub_last_ws_bytes;
extern void* stub_last_ws;
extern bool stub_gemv_ok, stub_skinny_ok, stub_skinny_pref, stub_tiled_ok;
extern int64_t stub_tiled_ws, stub_skinny_ws;

static int failures = 0;
#define CHECK(cond, what)                                                          \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      ++failures;                                                                  \
      fprintf(stderr, "FAIL line %d: %s (last error: \"%s\")\n", __LINE__, what,   \
              int4_last_error());                                                  \
    }                                                                              \
  } while (0)

// rc is EINVAL and the error text names the function
static void expect_einval(int rc, const char* fn, const char* what) {
  CHECK(rc == INT4DQ_EINVAL, what);
  CHECK(strstr(int4_last_error(), fn) != nullptr, what);
}

static int total_calls() {
  int s = 0;
  for (int c : stub_calls) s += c;
  return s;
}

int main() {
  // Fake, never dereferenced device pointers (the workspace one 256-aligned).
  alignas(256) static unsigned char arena[4096];
  void* const P = arena;
  const float* w = reinterpret_cast<const float*>(arena);
  uint8_t* packed = arena;
  uint16_t* scales = reinterpret_cast<uint16_t*>(arena + 1024);
  uint8_t* zeros = arena + 2048;
  float* y = reinterpret_cast<float*>(arena + 3072);
  const int64_t BIG = INT64_MAX / 2;

  // size helpers
  CHECK(int4_num_groups(301, 128) == 3, "num_groups 301/128");
  CHECK(int4_num_groups(128, 128) == 1, "num_groups 128/128");
  CHECK(int4_num_groups(5, 128) == 1, "num_groups group > K");
  CHECK(int4_num_groups(INT64_MAX, 1) == INT64_MAX, "num_groups INT64_MAX");
  CHECK(int4_num_groups(INT64_MAX, 2) == INT64_MAX / 2 + 1, "num_groups INT64_MAX / 2");
  CHECK(int4_num_groups(0, 1) == -1 && int4_num_groups(1, 0) == -1 && int4_num_groups(-5, 3) == -1, "num_groups bad");
  CHECK(int4_packed_bytes(48, 301) == 7248, "packed_bytes c2");
  CHECK(int4_packed_bytes(1, 1) == 1, "packed_bytes 1x1");
  CHECK(int4_packed_bytes(INT64_MAX, 4) == -1, "packed_bytes overflow");
  CHECK(int4_packed_bytes(3, INT64_MAX) == -1, "packed_bytes overflow in K");
  CHECK(int4_packed_bytes(0, 4) == -1 && int4_packed_bytes(4, -1) == -1, "packed_bytes bad");

  // quantize
  expect_einval(int4_quantize(nullptr, 4, 4, 4, packed, scales, nullptr), "int4_quantize", "quantize null w");
  expect_einval(int4_quantize(w, 0, 4, 4, packed, scales, nullptr), "int4_quantize", "quantize N=0");
  expect_einval(int4_quantize(w, 4, -3, 4, packed, scales, nullptr), "int4_quantize", "quantize K<0");
  expect_einval(int4_quantize(w, 4, 4, 0, packed, scales, nullptr), "int4_quantize", "quantize group 0");
  expect_einval(int4_quantize(w, BIG, BIG, 1, packed, scales, nullptr), "int4_quantize", "quantize overflow");
  expect_einval(int4_quantize(w, 4, 4, 4, packed, nullptr, nullptr), "int4_quantize", "quantize null scales");
  CHECK(total_calls() == 0, "no launch before validation passes");
  CHECK(int4_quantize(w, 48, 301, 128, packed, scales, nullptr) == INT4DQ_OK && stub_calls[0] == 1, "quantize ok");
  CHECK(int4_last_error()[0] == '\0', "success clears the error text");
  expect_einval(int4_quantize_affine(w, 4, 4, 4, packed, scales, nullptr, nullptr), "int4_quantize_affine",
                "affine null zeros");
  expect_einval(int4_quantize_affine(w, BIG, 8, 1, packed, scales, zeros, nullptr), "int4_quantize_affine",
                "affine overflow");
  CHECK(int4_quantize_affine(w, 4, 4, 4, packed, scales, zeros, nullptr) == INT4DQ_OK && stub_calls[1] == 1,
        "affine ok");

  // unpack, dequantize
  expect_einval(int4_unpack(packed, 4, 0, reinterpret_cast<int8_t*>(P), nullptr), "int4_unpack", "unpack K=0");
  expect_einval(int4_unpack(packed, BIG, 4, reinterpret_cast<int8_t*>(P), nullptr), "int4_unpack", "unpack overflow");
  expect_einval(int4_unpack(nullptr, 4, 4, reinterpret_cast<int8_t*>(P), nullptr), "int4_unpack", "unpack null");
  CHECK(int4_unpack(packed, 4, 5, reinterpret_cast<int8_t*>(P), nullptr) == INT4DQ_OK && stub_calls[2] == 1, "unpack ok");
  expect_einval(int4_dequantize(packed, scales, 4, 4, 4, 7, P, nullptr), "int4_dequantize", "dequantize dtype");
  expect_einval(int4_dequantize(packed, scales, 4, 4, 4, INT4DQ_OUT_F16, nullptr, nullptr), "int4_dequantize",
                "dequantize null out");
  expect_einval(int4_dequantize_affine(packed, scales, nullptr, 4, 4, 4, INT4DQ_OUT_F32, P, nullptr),
                "int4_dequantize_affine", "dequantize_affine null zeros");
  CHECK(int4_dequantize(packed, scales, 4, 4, 4, INT4DQ_OUT_F16, P, nullptr) == INT4DQ_OK && stub_calls[3] == 1,
        "dequantize ok");

  // matmul validation
  expect_einval(int4_matmul(P, INT4DQ_X_F16, -1, packed, scales, 4, 4, 4, y, nullptr), "int4_matmul", "M<0");
  expect_einval(int4_matmul(P, 9, 1, packed, scales, 4, 4, 4, y, nullptr), "int4_matmul", "x dtype");
  expect_einval(int4_matmul(nullptr, INT4DQ_X_F16, 1, packed, scales, 4, 4, 4, y, nullptr), "int4_matmul", "null x");
  expect_einval(int4_matmul(P, INT4DQ_X_F16, BIG, packed, scales, 4, BIG, 4, y, nullptr), "int4_matmul",
                "matmul overflow");
  expect_einval(int4_matmul_ex(P, INT4DQ_X_F16, 1, packed, scales, 4, 4, 4, nullptr, 5, y, nullptr),
                "int4_matmul", "activation");
  expect_einval(int4_matmul_path(P, INT4DQ_X_F16, 1, packed, scales, 4, 4, 4, nullptr, 0, y, 9, nullptr),
                "int4_matmul_path", "path");
  expect_einval(int4_linear(P, INT4DQ_X_F16, 1, packed, scales, nullptr, 4, 4, 4, nullptr, 0, y, 3, nullptr),
                "int4_linear", "y dtype");
  expect_einval(int4_matmul_affine(P, INT4DQ_X_F16, 1, packed, scales, nullptr, 4, 4, 4, nullptr, 0, y, 0,
                                   nullptr),
                "int4_matmul_affine", "affine matmul null zeros");
  const int before = total_calls();
  CHECK(int4_matmul(nullptr, INT4DQ_X_F16, 0, packed, scales, 4, 4, 4, nullptr, nullptr) == INT4DQ_OK &&
            total_calls() == before,
        "M = 0 is a no-op");

  // path choice follows what the kernels accept
  CHECK(int4_matmul_select(P, INT4DQ_X_F16, 1, packed, scales, 4, 64, 32, y) == INT4DQ_PATH_GEMV, "select gemv");
  stub_gemv_ok = false;
  CHECK(int4_matmul_select(P, INT4DQ_X_F16, 8, packed, scales, 4, 64, 32, y) == INT4DQ_PATH_SKINNY, "select skinny");
  stub_skinny_pref = false;
  CHECK(int4_matmul_select(P, INT4DQ_X_F16, 8, packed, scales, 4, 64, 32, y) == INT4DQ_PATH_TILED, "select tiled");
  stub_tiled_ok = false;
  CHECK(int4_matmul_select(P, INT4DQ_X_F16, 8, packed, scales, 4, 64, 32, y) == INT4DQ_PATH_GENERIC,
        "select generic");
  CHECK(int4_matmul_select(nullptr, INT4DQ_X_F16, 8, packed, scales, 4, 64, 32, y) == -1, "select invalid");
  CHECK(int4_matmul(P, INT4DQ_X_F32, 3, packed, scales, 4, 64, 32, y, nullptr) == INT4DQ_OK && stub_calls[4] == 1 &&
            stub_last_M == 3,
        "generic launch");
  CHECK(int4_matmul_path(P, INT4DQ_X_F16, 3, packed, scales, 4, 64, 32, nullptr, 0, y, INT4DQ_PATH_TILED,
                         nullptr) == INT4DQ_EUNSUPPORTED,
        "forced path the kernel refuses");
  CHECK(strstr(int4_last_error(), "tiled stub refuses") != nullptr, "refusal reason in the error text");
  stub_gemv_ok = stub_skinny_ok = stub_skinny_pref = stub_tiled_ok = true;

  // split-of-K workspace calls
  expect_einval(int4_linear_ws(P, INT4DQ_X_F16, 8, packed, scales, nullptr, 4, 64, 32, nullptr, 0, y, 0, nullptr,
                               -1, nullptr),
                "int4_linear_ws", "negative workspace size");
  expect_einval(int4_linear_ws(P, INT4DQ_X_F16, 8, packed, scales, nullptr, 4, 64, 32, nullptr, 0, y, 0, nullptr,
                               64, nullptr),
                "int4_linear_ws", "null workspace with a size");
  expect_einval(int4_linear_ws(P, INT4DQ_X_F16, 8, packed, scales, nullptr, 4, 64, 32, nullptr, 0, y, 0,
                               arena + 16, 64, nullptr),
                "int4_linear_ws", "misaligned workspace");
  CHECK(int4_linear_workspace_bytes(INT4DQ_X_F16, -1, 4, 4, 4) == -1, "workspace_bytes M<0");
  CHECK(int4_linear_workspace_bytes(7, 1, 4, 4, 4) == -1, "workspace_bytes dtype");
  CHECK(int4_linear_workspace_bytes(INT4DQ_X_F16, 0, 4, 4, 4) == 0, "workspace_bytes M=0");
  stub_gemv_ok = stub_skinny_ok = false;
  stub_tiled_ws = 12345;
  CHECK(int4_linear_workspace_bytes(INT4DQ_X_F16, 128, 4096, 4096, 128) == 12345, "workspace_bytes tiled");
  CHECK(int4_linear_ws(P, INT4DQ_X_F16, 128, packed, scales, nullptr, 4096, 4096, 128, nullptr, 0, y, 0, arena,
                       4096, nullptr) == INT4DQ_OK &&
            stub_last_ws == arena && stub_last_ws_bytes == 4096,
        "workspace passed to the tiled launcher");
  stub_tiled_ws = (16ll << 20) + 1;             // more than the library's scratch
  expect_einval(int4_linear_noalloc(P, INT4DQ_X_F16, 128, packed, scales, nullptr, 4096, 4096, 128, nullptr, 0, y,
                                    0, nullptr),
                "int4_linear_noalloc", "scratch too small");
  CHECK(strstr(int4_last_error(), "scratch") != nullptr, "noalloc names the scratch limit");
  stub_tiled_ws = 0;                            // no split: no scratch, no HIP call
  CHECK(int4_linear_noalloc(P, INT4DQ_X_F16, 128, packed, scales, nullptr, 4096, 4096, 128, nullptr, 0, y, 0,
                            nullptr) == INT4DQ_OK &&
            stub_last_ws == nullptr && stub_last_ws_bytes == 0,
        "noalloc without a split");
  stub_gemv_ok = stub_skinny_ok = true;
  // the skinny kernel's split takes the workspace the same way
  stub_gemv_ok = false;
  stub_skinny_ws = 777;
  CHECK(int4_linear_workspace_bytes(INT4DQ_X_F16, 16, 768, 3072, 32) == 777, "workspace_bytes skinny");
  CHECK(int4_linear_ws(P, INT4DQ_X_F16, 16, packed, scales, nullptr, 768, 3072, 32, nullptr, 0, y, 0, arena,
                       1024, nullptr) == INT4DQ_OK &&
            stub_last_ws == arena && stub_last_ws_bytes == 1024,
        "workspace passed to the skinny launcher");
  stub_skinny_ws = 0;
  stub_gemv_ok = true;

  // the error text belongs to the thread that made the call
  std::string t1, t2;
  std::thread a([&] {
    int4_quantize(w, 0, 4, 4, packed, scales, nullptr);
    t1 = int4_last_error();
  });
  std::thread b([&] {
    int4_unpack(packed, 4, 0, reinterpret_cast<int8_t*>(P), nullptr);
    t2 = int4_last_error();
  });
  a.join();
  b.join();
  CHECK(t1.find("int4_quantize") != std::string::npos && t2.find("int4_unpack") != std::string::npos,
        "per-thread error text");

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("api driver: all checks passed\n");
  return 0;
}
