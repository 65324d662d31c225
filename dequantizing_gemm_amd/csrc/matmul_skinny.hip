// matmul_skinny.hip -- dequantizing matmul for few activation rows (M <= 16,
// binary16 x) on gfx950: a weight-streaming kernel bound by HBM bandwidth.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, int4_matmul): y = x @ dequantize(W).T,
// one group at a time -- x times the group's integer codes, then the group's
// scale on the output column. ("Build a Blockwise INT4 Inference Engine",
// architecture overview: the weights are never expanded to full precision in
// memory; the takeaways put the bottleneck in memory bandwidth.)
//
// At M <= 16 every packed byte is used 2*M times, far below the machine's
// flop/byte balance, so the kernel is built to stream the packed weights
// once at full bandwidth and spend as few vector-ALU ops per byte as possible:
//
//  * The contraction runs on the matrix cores: v_mfma_f32_16x16x32_f16 with
//    the 16 weight rows of a block as B (16 columns) and the M <= 16
//    activation rows as A (rows >= M are zero). The integer codes are exact in
//    fp16, products are exact, and sums are fp32.
//  * A lane never converts codes one by one: a 32-bit word of 8 codes becomes
//    four exact fp16 pairs with one AND-OR and one packed fp16 op per pair
//    (codes_to_half_spread, 10 VALU ops per 8 codes). That routine pairs code c
//    with code c+4, so the activations are staged into LDS once per block in
//    the same order, and every A fragment is then one 16-byte LDS read.
//  * Lane l of a wavefront owns weight row (l mod 16) and one contiguous
//    quarter of each K-block (KB = 128 codes for group sizes that are
//    multiples of 128, else KB = group = 64 or 32), i.e. one 16-byte (KB=128)
//    load per K-block: 16 rows x 64 contiguous bytes per wavefront load.
//    The block's waves take interleaved K-blocks, so at any moment a block
//    reads neighbouring stretches of its 16 rows.
//  * Per K-block each MFMA chain starts from zero, and the group's scale is
//    applied to that fp32 partial on the output column (lane l holds column
//    l mod 16) -- the integer-first order of the statement.
//  * The waves' partial tiles are summed through LDS at the end; no atomics,
//    results are deterministic.
#include "device_common.h"
#include "kernels.h"

namespace int4dq {

namespace {

constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyLdsX = 48 * 1024;   // bytes of LDS for the staged activations

template <int KB> struct WLoad;
template <> struct WLoad<128> { typedef u32x4_t T; };
template <> struct WLoad<64> { typedef u32x2_t T; };
template <> struct WLoad<32> { typedef uint32_t T; };

template <int KB>
__device__ __forceinline__ uint32_t word_at(const typename WLoad<KB>::T& v, int i) {
  if constexpr (KB == 32) {
    return v;
  } else {
    return v[i];
  }
}

}  // namespace

// U = K-blocks whose weight loads a wave issues before consuming any of them.
template <int KB, int U>
__global__ __launch_bounds__(kSkinnyWaves * 64) void matmul_skinny_kernel(
    const _Float16* __restrict__ x, int M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, int64_t N, int64_t K, int64_t group, int64_t G,
    int64_t KC, float* __restrict__ y) {
  typedef typename WLoad<KB>::T wvec_t;
  constexpr int DW = KB / 32;                 // code words per lane per K-block = MFMAs
  // Dynamic LDS: wave partials [waves][64][4] fp32, then the staged x chunk.
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* red = reinterpret_cast<float*>(lds);
  _Float16* xs = reinterpret_cast<_Float16*>(lds + kSkinnyWaves * 64 * 4 * sizeof(float));

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, h = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nrow = (n0 + col < N) ? n0 + col : N - 1;     // tail rows: read, discard
  const uint8_t* prow = packed + nrow * (K >> 1) + h * (KB / 8);
  const uint16_t* srow = scales + nrow * G;
  const int xstride = (int)KC + 8;                             // halves; +16 B vs bank conflicts
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};

  for (int64_t kc0 = 0; kc0 < K; kc0 += KC) {
    const int kcn = (int)((K - kc0) < KC ? (K - kc0) : KC);
    __syncthreads();
    const int pieces = kcn / 8;
    for (int p = tid; p < M * pieces; p += kSkinnyWaves * 64) {
      const int m = p / pieces, c = p - m * pieces;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + (int64_t)m * K + kc0 + 8 * c);
      *reinterpret_cast<u32x4_t*>(xs + m * xstride + 8 * c) = spread_perm_x(v);
    }
    __syncthreads();

    const int nkb = kcn / KB;
    const _Float16* xa = xs + col * xstride + h * (KB / 4);
    for (int j0 = wave; j0 < nkb; j0 += kSkinnyWaves * U) {
      wvec_t wv[U];
      float sf[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * kSkinnyWaves;
        if (j < nkb) {
          const int64_t kb = kc0 + (int64_t)j * KB;
          wv[u] = __builtin_nontemporal_load(reinterpret_cast<const wvec_t*>(prow + (kb >> 1)));
          sf[u] = half_bits_to_float(srow[kb / group]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * kSkinnyWaves;
        if (j < nkb) {
          float4_t dg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int i = 0; i < DW; ++i) {
            half2_t hw[4];
            codes_to_half_spread(word_at<KB>(wv[u], i), hw);
            half8_t a = {};
            if (col < M) a = *reinterpret_cast<const half8_t*>(xa + j * KB + 8 * i);
            dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, as_half8(hw), dg, 0, 0, 0);
          }
          acc += sf[u] * dg;
        }
      }
    }
  }

  // Sum the waves' 16x16 partial tiles. Lane l holds rows 4*(l/16) + r of column l%16.
  *reinterpret_cast<float4_t*>(red + (wave * 64 + lane) * 4) = acc;
  __syncthreads();
  if (tid < 16 * M) {
    const int m = tid >> 4, nn = tid & 15;
    const int src = ((m >> 2) * 16 + nn) * 4 + (m & 3);
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves; ++w) s += red[w * 256 + src];
    if (n0 + nn < N) y[(int64_t)m * N + n0 + nn] = s;
  }
}

// KB for a group size, or 0 if the skinny kernel does not take it.
static int skinny_kb(int64_t group) {
  if (group % 128 == 0) return 128;
  if (group == 64) return 64;
  if (group == 32) return 32;
  return 0;
}

const char* matmul_skinny_unsupported(int x_dtype, int64_t M, const void* x,
                                      const uint8_t* packed, int64_t K, int64_t group) {
  if (x_dtype != 1) return "skinny kernel takes binary16 activations only";
  if (M > 16) return "skinny kernel takes M <= 16";
  const int KB = skinny_kb(group);
  if (KB == 0) return "skinny kernel takes group 32, 64 or a multiple of 128";
  if (K % KB != 0) return "skinny kernel needs K to be a multiple of min(group, 128)";
  if ((uintptr_t)x % 16 || (uintptr_t)packed % 16) return "skinny kernel needs 16-byte aligned x and packed";
  return nullptr;
}

hipError_t launch_matmul_skinny(const void* x, int64_t M, const uint8_t* packed,
                                const uint16_t* scales, int64_t N, int64_t K, int64_t group,
                                float* y, hipStream_t stream) {
  const int KB = skinny_kb(group);
  const int64_t G = (K + group - 1) / group;
  // Largest multiple of KB whose M padded rows fit the staging buffer.
  int64_t KC = ((int64_t)(kSkinnyLdsX / 2) / M - 8) / KB * KB;
  if (KC > K) KC = K;
  const size_t lds = kSkinnyWaves * 64 * 4 * sizeof(float) + (size_t)M * (KC + 8) * 2;
  const dim3 grid((unsigned)((N + 15) / 16)), block(kSkinnyWaves * 64);
  const _Float16* xh = static_cast<const _Float16*>(x);
  const int Mi = (int)M;
  switch (KB) {
    case 128:
      hipLaunchKernelGGL((matmul_skinny_kernel<128, 4>), grid, block, lds, stream, xh, Mi, packed,
                         scales, N, K, group, G, KC, y);
      break;
    case 64:
      hipLaunchKernelGGL((matmul_skinny_kernel<64, 4>), grid, block, lds, stream, xh, Mi, packed,
                         scales, N, K, group, G, KC, y);
      break;
    default:
      hipLaunchKernelGGL((matmul_skinny_kernel<32, 8>), grid, block, lds, stream, xh, Mi, packed,
                         scales, N, K, group, G, KC, y);
      break;
  }
  return hipGetLastError();
}

}  // namespace int4dq
