// matmul_tiled.hip -- dequantizing matmul for many activation rows (binary16
// x) on gfx950: an LDS-tiled MFMA kernel bound by matrix-core throughput.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, int4_matmul): y = x @ dequantize(W).T,
// one group at a time -- x times the group's integer codes first, then the
// group's scale on each output column. Full-precision weights never reach
// memory ("Build a Blockwise INT4 Inference Engine", architecture overview:
// the fusion boundary); here they exist only as an fp16 tile of exact integer
// codes in LDS for the duration of one K-block.
//
// Block tile BM x BN = 128 x 128, 256 threads as 2 x 2 wavefronts, each
// wavefront owning a 64 x 64 output tile of 4 x 4 MFMA tiles
// (v_mfma_f32_16x16x32_f16, fp32 accumulation). Per K-block of KB codes
// (KB = 128 for group sizes that are multiples of 128, else KB = group):
//   1. the block's x tile [128 x KB] fp16 and packed tile [128 x KB/2] bytes
//      were fetched into registers during the previous K-block;
//   2. they are written to LDS -- the packed codes expanded to exact fp16
//      integers (codes_to_half_natural) once per block, not once per wavefront;
//   3. each wavefront runs its 4 x 4 x (KB/32) MFMAs into a zeroed group
//      accumulator while the next K-block's global loads are in flight;
//   4. the group accumulator is scaled by the group's scale of its output
//      column and added to the running accumulator (integer-first order).
// LDS rows are padded by 16 bytes so that the 16 rows read by one MFMA
// operand load fall in different banks.
#include "device_common.h"
#include "kernels.h"

namespace int4dq {

namespace {
constexpr int kBM = 128, kBN = 128, kThreads = 256;
}

template <int KB>
__global__ __launch_bounds__(kThreads) void matmul_tiled_kernel(
    const _Float16* __restrict__ x, int64_t M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, int64_t N, int64_t K, int64_t group, int64_t G,
    float* __restrict__ y) {
  constexpr int LDK = KB + 8;                         // padded LDS row, halves
  constexpr int XP = kBM * KB / 8 / kThreads;         // 16-B x pieces per thread
  constexpr int WPR = KB / 32;                        // 16-B packed pieces per row
  constexpr int WP = (kBN * WPR + kThreads - 1) / kThreads;  // packed pieces per thread
  constexpr int SLOTS = KB / 32;                      // MFMA k-steps per K-block
  __shared__ __attribute__((aligned(16))) _Float16 As[kBM * LDK];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[kBN * LDK];
  __shared__ float Ss[kBN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 15, h = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;

  // Fixed per-thread global coordinates of the pieces it stages.
  u32x4_t xr[XP];
  u32x4_t wr[WP];
  uint16_t sr = 0;

  auto fetch = [&](int64_t kb) {
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int piece = tid + p * kThreads;
      const int r = piece / (KB / 8), c = piece % (KB / 8);
      const int64_t m = m0 + r;
      if (m < M)
        xr[p] = *reinterpret_cast<const u32x4_t*>(x + m * K + kb + 8 * c);
      else
        xr[p] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < WP; ++p) {
      const int piece = tid + p * kThreads;
      if (piece < kBN * WPR) {
        const int r = piece / WPR, c = piece % WPR;
        int64_t n = n0 + r;
        if (n >= N) n = N - 1;                        // tail rows: read, discard
        wr[p] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(packed + n * (K >> 1) + (kb >> 1) + 16 * c));
      }
    }
    if (tid < kBN) {
      int64_t n = n0 + tid;
      if (n >= N) n = N - 1;
      sr = scales[n * G + kb / group];
    }
  };

  auto stage = [&]() {
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const int piece = tid + p * kThreads;
      const int r = piece / (KB / 8), c = piece % (KB / 8);
      *reinterpret_cast<u32x4_t*>(As + r * LDK + 8 * c) = xr[p];
    }
#pragma unroll
    for (int p = 0; p < WP; ++p) {
      const int piece = tid + p * kThreads;
      if (piece < kBN * WPR) {
        const int r = piece / WPR, c = piece % WPR;
        _Float16* dst = Bs + r * LDK + 32 * c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          half2_t hw[4];
          codes_to_half_natural(wr[p][i], hw);
          *reinterpret_cast<half8_t*>(dst + 8 * i) = as_half8(hw);
        }
      }
    }
    if (tid < kBN) Ss[tid] = half_bits_to_float(sr);
  };

  float4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t nkb = K / KB;
  fetch(0);
  for (int64_t t = 0; t < nkb; ++t) {
    lds_barrier();                                    // previous K-block's readers done
    stage();
    lds_barrier();                                    // (next K-block's loads stay in flight)
    if (t + 1 < nkb) fetch((t + 1) * KB);             // next loads overlap the MFMAs

    float4_t dg[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) dg[a][b] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      half8_t af[4], bf[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        af[a] = *reinterpret_cast<const half8_t*>(As + (wm * 64 + a * 16 + col) * LDK + 32 * s + 8 * h);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        bf[b] = *reinterpret_cast<const half8_t*>(Bs + (wn * 64 + b * 16 + col) * LDK + 32 * s + 8 * h);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          dg[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[a], bf[b], dg[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float sf = Ss[wn * 64 + b * 16 + col];
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a][b] += sf * dg[a][b];
    }
  }

  // Lane l holds rows 4*(l/16)+r of column l%16 of each 16x16 tile.
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t n = n0 + wn * 64 + b * 16 + col;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + a * 16 + 4 * h + r;
        if (m < M) y[m * N + n] = acc[a][b][r];
      }
    }
}

static int tiled_kb(int64_t group) {
  if (group % 128 == 0) return 128;
  if (group == 64) return 64;
  if (group == 32) return 32;
  return 0;
}

const char* matmul_tiled_unsupported(int x_dtype, const void* x, const uint8_t* packed,
                                     int64_t K, int64_t group) {
  if (x_dtype != 1) return "tiled kernel takes binary16 activations only";
  const int KB = tiled_kb(group);
  if (KB == 0) return "tiled kernel takes group 32, 64 or a multiple of 128";
  if (K % KB != 0) return "tiled kernel needs K to be a multiple of min(group, 128)";
  if ((uintptr_t)x % 16 || (uintptr_t)packed % 16) return "tiled kernel needs 16-byte aligned x and packed";
  return nullptr;
}

hipError_t launch_matmul_tiled(const void* x, int64_t M, const uint8_t* packed,
                               const uint16_t* scales, int64_t N, int64_t K, int64_t group,
                               float* y, hipStream_t stream) {
  const int KB = tiled_kb(group);
  const int64_t G = (K + group - 1) / group;
  const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM)),
      block(kThreads);
  const _Float16* xh = static_cast<const _Float16*>(x);
  switch (KB) {
    case 128:
      hipLaunchKernelGGL(matmul_tiled_kernel<128>, grid, block, 0, stream, xh, M, packed, scales, N,
                         K, group, G, y);
      break;
    case 64:
      hipLaunchKernelGGL(matmul_tiled_kernel<64>, grid, block, 0, stream, xh, M, packed, scales, N,
                         K, group, G, y);
      break;
    default:
      hipLaunchKernelGGL(matmul_tiled_kernel<32>, grid, block, 0, stream, xh, M, packed, scales, N,
                         K, group, G, y);
      break;
  }
  return hipGetLastError();
}

}  // namespace int4dq
