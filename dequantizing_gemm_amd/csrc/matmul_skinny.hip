// matmul_skinny.hip -- dequantizing matmul for few activation rows (M <= 64,
// binary16 x; M = 1 normally takes matmul_gemv.hip) on gfx950: a
// weight-streaming kernel bound by HBM bandwidth.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, int4_matmul): y = x @ dequantize(W).T,
// one group at a time -- x times the group's integer codes, then the group's
// scale on the output column. ("Build a Blockwise INT4 Inference Engine",
// architecture overview: the weights are never expanded to full precision in
// memory; the takeaways put the bottleneck in memory bandwidth.)
//
// At M <= 64 every packed byte is used 2*M times, far below the machine's
// flop/byte balance. The kernel streams the packed weights once and keeps
// each block's critical path short, because at these sizes (1-120 MB per
// call) a launch is a single round of loads and its latency chain, not a
// steady stream:
//
//  * The contraction runs on the matrix cores: v_mfma_f32_16x16x32_f16 with
//    16 weight rows as B (one per lane column) and the activation rows as A.
//    Lanes of A rows >= M load row M-1 again: those output rows are computed
//    and discarded, so nothing has to be zeroed or masked. The integer codes
//    are exact in fp16, products are exact, sums are fp32.
//  * A 32-bit word of 8 codes becomes four exact fp16 pairs. For M <= 4 each
//    wave stages its own slice of x in LDS, permuted to the "spread" order
//    that codes_to_half_spread produces (9 VALU ops per 8 codes); for larger
//    M each lane's A fragment is 8 consecutive activations loaded straight
//    from global memory (x is tiny and stays in L2) and the codes are expanded
//    in natural order (codes_to_half_natural, 12 ops). No block barrier
//    stands between a wave's loads and its first MFMA.
//  * Lane l owns weight row (l mod 16) and one quarter of each K-block
//    (KB = 128 codes for group sizes 128 * 2^p, else KB = group = 64 or 32):
//    one 16-byte weight load per K-block for KB = 128, and a wavefront load
//    covers 16 rows x 64 contiguous bytes. The block's waves take interleaved
//    K-blocks. Every wave issues all loads of its share (U K-blocks: weights,
//    scales, activations) before it waits for any of them.
//  * Per K-block the MFMA chain starts from zero and the group's scale is
//    applied to that fp32 partial on the output column (lane l holds column
//    l mod 16): the integer-first order of the statement.
//  * The waves' partial 16x16 tiles are summed through LDS at the end (the
//    only barrier); no atomics, results are deterministic.
//  * Affine codes ("Build a Blockwise INT4 Inference Engine", step 2): the AFF
//    form loads each K-block's zero point next to its scale and expands the
//    codes to u - zp (codes_to_half_*_zp, same op counts).
#include "device_common.h"
#include "kernels.h"

namespace int4dq {

namespace {

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

// WAVES waves per block, each handling up to U K-blocks (K-blocks j = wave,
// wave + WAVES, ...; the launch guarantees WAVES * U >= K / KB).
// MR > 0 (M <= MR <= 4): the wave stages its own slice of x (MR rows x U
// K-blocks; rows >= M repeat row M-1) into a wave-private LDS region in the
// spread order and expands the codes with codes_to_half_spread (9 VALU ops per
// 8 codes). MR == 0: each lane loads its A fragments from global memory in
// natural order (codes_to_half_natural, 12 ops per 8 codes). Staging moves one
// copy of x per wave instead of one 16-byte load per lane and MFMA, and is used
// for small M where the slices fit LDS.
// RG > 1 (MR == 0 only): the block owns RG groups of 16 weight rows, and each
// activation fragment a lane loads serves all RG of them, which divides the
// activation traffic per weight byte by RG (x is re-read by every block).
// MT > 1 (MR == 0 only): M up to 16 MT rows of x as MT tiles of 16; each
// expanded code word feeds MT MFMAs, one per tile.
template <int KB, int WAVES, int U, int MR, int RG, bool AFF, int MT = 1>
__global__ __launch_bounds__(WAVES * 64) void matmul_skinny_kernel(
    const _Float16* __restrict__ x, int M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N, int K, int G,
    int kb_shift, void* __restrict__ y, Epilogue ep) {
  typedef typename WLoad<KB>::T wvec_t;
  constexpr int DW = KB / 32;                 // code words per lane per K-block = MFMAs
  constexpr int XB = (RG > 1 || MT > 1) ? 1 : (U < 4 ? U : 4);   // K-blocks per batch of direct x loads
  static_assert(MR == 0 || (RG == 1 && MT == 1), "row groups and row tiles with direct x loads only");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* red = reinterpret_cast<float*>(lds);                  // [WAVES][RG][MT][64][4]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int col = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * 16 * RG;
  const uint8_t* prow[RG];
  const uint16_t* srow[RG];
  const uint8_t* zrow[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int nrow = (n0 + 16 * r + col < N) ? n0 + 16 * r + col : N - 1;   // tail rows: read, discard
    prow[r] = packed + (int64_t)nrow * (K >> 1) + h * (KB / 8);
    srow[r] = scales + (int64_t)nrow * G;
    zrow[r] = AFF ? zeros + (int64_t)nrow * G : nullptr;
  }
  const int nkb = K / KB;

  // Weight and scale loads of the wave's share, K-block by K-block. They are
  // issued after the (smaller) x staging loads, so that each K-block's
  // compute waits only for its own weights (loads return in order).
  wvec_t wv[RG][U];
  uint32_t sraw[RG][U], zraw[RG][U];
  // Straight-line, unconditional loads: a K-block index past the end is
  // clamped to the wave's last valid one (the value is loaded and ignored), so
  // no branch splits the sequence and no use is scheduled between the loads.
  // Scales first: the compiler converts them to fp32 as soon as they arrive,
  // and with the weights issued after them that wait does not cover the weights.
  auto load_w = [&]() {
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = wave + u * WAVES < nkb ? wave + u * WAVES : nkb - 1;
        sraw[r][u] = srow[r][j >> kb_shift];
      }
    if constexpr (AFF) {
#pragma unroll
      for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = wave + u * WAVES < nkb ? wave + u * WAVES : nkb - 1;
          zraw[r][u] = zrow[r][j >> kb_shift];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const int j = wave + u * WAVES < nkb ? wave + u * WAVES : nkb - 1;
        wv[r][u] = __builtin_nontemporal_load(reinterpret_cast<const wvec_t*>(prow[r] + j * (KB / 2)));
      }
  };

  float4_t acc[RG][MT];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (MR > 0) {
    // Wave-private region: [MR][U][KB] halves, spread order within each 8.
    _Float16* xw = reinterpret_cast<_Float16*>(lds + WAVES * 64 * 4 * sizeof(float)) +
                   (size_t)wave * MR * U * KB;
    constexpr int PPB = KB / 8;                // 16-byte pieces per K-block row
    constexpr int BPI = 64 / PPB;              // K-blocks covered by one wave load
    constexpr int XR = (U + BPI - 1) / BPI;    // wave loads per x row
    // Straight-line: all x loads, then the weights, then the LDS writes (which
    // wait for x only). Indices past the end are clamped, values unused.
    u32x4_t xv[MR][XR];
#pragma unroll
    for (int mm = 0; mm < MR; ++mm)
#pragma unroll
      for (int r = 0; r < XR; ++r) {
        const int u = r * BPI + lane / PPB, c = lane % PPB;
        const int uu = u < U ? u : U - 1;
        const int j = wave + uu * WAVES < nkb ? wave + uu * WAVES : nkb - 1;
        const int m = mm < M ? mm : M - 1;
        xv[mm][r] = *reinterpret_cast<const u32x4_t*>(x + (int64_t)m * K + j * KB + 8 * c);
      }
    load_w();
#pragma unroll
    for (int mm = 0; mm < MR; ++mm)
#pragma unroll
      for (int r = 0; r < XR; ++r) {
        const int u = r * BPI + lane / PPB, c = lane % PPB;
        if (u < U)
          *reinterpret_cast<u32x4_t*>(xw + (mm * U + u) * KB + 8 * c) = spread_perm_x(xv[mm][r]);
      }
    // A wave's LDS operations complete in order, so no barrier is needed
    // between these writes and the reads below; keep the compiler from
    // moving the reads above the writes.
    __builtin_amdgcn_wave_barrier();
    const _Float16* xa = xw + (col < MR ? col : MR - 1) * U * KB + h * (KB / 4);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (wave + u * WAVES < nkb) {
        half8_t a[DW];
#pragma unroll
        for (int i = 0; i < DW; ++i) a[i] = *reinterpret_cast<const half8_t*>(xa + u * KB + 8 * i);
        float4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
        const uint32_t zlo = AFF ? zp_bias_lo(zraw[0][u]) : 0u, zhi = AFF ? zp_bias_hi(zraw[0][u]) : 0u;
#pragma unroll
        for (int i = 0; i < DW; ++i) {
          half2_t hw[4];
          if constexpr (AFF) codes_to_half_spread_zp(word_at<KB>(wv[0][u], i), hw, zlo, zhi);
          else codes_to_half_spread(word_at<KB>(wv[0][u], i), hw);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], as_half8(hw), d, 0, 0, 0);
        }
        acc[0][0] += half_bits_to_float((uint16_t)sraw[0][u]) * d;
      }
    }
  } else {
    // Activation fragments straight from global memory (L2 hits), natural
    // order, in batches of XB K-blocks to bound register use.
    const _Float16* xp[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int r = 16 * t + col < M ? 16 * t + col : M - 1;
      xp[t] = x + (int64_t)r * K + h * (KB / 4) + wave * KB;
    }
    load_w();
    half8_t xa[MT][XB][DW];
    auto load_x = [&](int b) {
#pragma unroll
      for (int v = 0; v < XB; ++v)
        if (b + v < U && wave + (b + v) * WAVES < nkb)
#pragma unroll
          for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < DW; ++i)
              xa[t][v][i] = *reinterpret_cast<const half8_t*>(xp[t] + (b + v) * (WAVES * KB) + 8 * i);
    };
#pragma unroll
    for (int b = 0; b < U; b += XB) {
      load_x(b);
#pragma unroll
      for (int v = 0; v < XB; ++v) {
        const int u = b + v;
        if (u < U && wave + u * WAVES < nkb) {
#pragma unroll
          for (int r = 0; r < RG; ++r) {
            float4_t d[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) d[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            const uint32_t zb = AFF ? zp_bias_natural(zraw[r][u]) : 0u;
#pragma unroll
            for (int i = 0; i < DW; ++i) {
              half2_t hw[4];
              if constexpr (AFF) codes_to_half_natural_zp(word_at<KB>(wv[r][u], i), hw, zb);
              else codes_to_half_natural(word_at<KB>(wv[r][u], i), hw);
              const half8_t bw = as_half8(hw);
#pragma unroll
              for (int t = 0; t < MT; ++t)
                d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[t][v][i], bw, d[t], 0, 0, 0);
            }
            const float sc = half_bits_to_float((uint16_t)sraw[r][u]);
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[r][t] += sc * d[t];
          }
        }
      }
    }
  }

  // Sum the waves' 16x16 partial tiles. Lane l holds rows 4*(l/16) + i of column l%16.
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t)
      *reinterpret_cast<float4_t*>(red + (((wave * RG + r) * MT + t) * 64 + lane) * 4) = acc[r][t];
  __syncthreads();
  for (int t = tid; t < 16 * M * RG; t += WAVES * 64) {
    const int r = t / (16 * M), rem = t - r * 16 * M;
    const int m = rem >> 4, nn = rem & 15;
    const int tm = m >> 4, mm = m & 15;                       // row tile, row inside it
    const int src = ((mm >> 2) * 16 + nn) * 4 + (mm & 3);
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += red[((w * RG + r) * MT + tm) * 256 + src];
    const int n = n0 + 16 * r + nn;
    if (n < N) ep.store(y, (int64_t)m * N + n, s, n);
  }
}

// KB for a group size, or 0 if the skinny kernel does not take it
// (group / KB must be a power of two: the scale index is a shift).
static int skinny_kb(int64_t group) {
  if (group == 32 || group == 64) return (int)group;
  if (group % 128 == 0 && ((group / 128) & (group / 128 - 1)) == 0) return 128;
  return 0;
}

// Largest K-block count one launch handles (16 waves x 8 K-blocks).
constexpr int kSkinnyMaxKB = 16 * 8;

const char* matmul_skinny_unsupported(int x_dtype, int64_t M, const void* x,
                                      const uint8_t* packed, int64_t N, int64_t K,
                                      int64_t group) {
  if (x_dtype != 1) return "skinny kernel takes binary16 activations only";
  if (M > 64) return "skinny kernel takes M <= 64";
  const int KB = skinny_kb(group);
  if (KB == 0) return "skinny kernel takes group 32, 64 or 128 times a power of two";
  if (K % KB != 0) return "skinny kernel needs K to be a multiple of min(group, 128)";
  if (K / KB > kSkinnyMaxKB) return "skinny kernel takes K <= 128 * min(group, 128)";
  // (four row tiles and eight K-blocks per wave do not fit 16 wavefronts' registers)
  if (M > 32 && K / KB > 16 * 6) return "skinny kernel takes M <= 32 when K > 96 * min(group, 128)";
  if (N >= (1ll << 30)) return "skinny kernel needs N below 2^30";
  if ((uintptr_t)x % 16 || (uintptr_t)packed % 16) return "skinny kernel needs 16-byte aligned x and packed";
  return nullptr;
}

// Whether the skinny kernel should take a shape it supports. Up to 16 rows
// always. For 17-64 rows its time grows with N times the number of 16-row
// tiles, while the tiled kernel's (32 x 128 tiles there) is about flat;
// measured on MI355X, the skinny kernel is the faster one while
// N * ceil(M / 16) <= 12288: [4096,4096] M = 32 11.6 us, M = 48 17.0 us
// (tiled about 20), but M = 64 20.1 against 20.5, [4096,11008] M = 64 59.8
// against 48.9, [11008,4096] M = 64 42.1 against 21.8.
bool matmul_skinny_preferred(int64_t M, int64_t N) {
  return M <= 16 || N * ((M + 15) / 16) <= 12288;
}

// Bytes of LDS a launch uses: the reduction buffer, plus the wave-private x
// slices of MR rows when they are staged.
static size_t skinny_lds(int waves, int U, int KB, int MR, int RG = 1, int MT = 1) {
  return (size_t)waves * RG * MT * 64 * 4 * sizeof(float) + (size_t)waves * MR * U * KB * 2;
}
constexpr size_t kSkinnyLdsMax = 64 * 1024;

template <int KB, int WAVES, int U, int MR, int RG, bool AFF, int MT = 1>
static void launch_mr(const _Float16* x, int M, const uint8_t* packed, const uint16_t* scales,
                      const uint8_t* zeros, int N, int K, int G, int kbs, void* y, Epilogue ep,
                      hipStream_t stream) {
  hipLaunchKernelGGL((matmul_skinny_kernel<KB, WAVES, U, MR, RG, AFF, MT>),
                     dim3((unsigned)((N + 16 * RG - 1) / (16 * RG))), dim3(WAVES * 64),
                     skinny_lds(WAVES, U, KB, MR, RG, MT), stream, x, M, packed, scales, zeros, N, K, G,
                     kbs, y, ep);
}

// 17 <= M <= 64: MT = 2 or 4 row tiles, direct x loads. Every block re-reads
// its rows' share of x (M/(4 RG) bytes of x per byte of weights), so the
// block takes as many row groups as its registers allow while the grid keeps
// about one block per CU.
template <int KB, int WAVES, int U, bool AFF, int MT>
static void launch_tiles(const _Float16* x, int M, const uint8_t* packed, const uint16_t* scales,
                         const uint8_t* zeros, int N, int K, int G, int kbs, void* y, Epilogue ep,
                         hipStream_t stream) {
  constexpr bool rg2 = WAVES <= 8;
  if constexpr (rg2) {
    if (N >= 256 * 16 * 2) {
      launch_mr<KB, WAVES, U, 0, 2, AFF, MT>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
      return;
    }
  }
  launch_mr<KB, WAVES, U, 0, 1, AFF, MT>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
}

template <int KB, int WAVES, int U, bool AFF>
static void launch_one(const _Float16* x, int M, const uint8_t* packed, const uint16_t* scales,
                       const uint8_t* zeros, int N, int K, int G, int kbs, void* y, Epilogue ep,
                       hipStream_t stream) {
  if constexpr (WAVES < 16 || U <= 6) {           // refused by matmul_skinny_unsupported otherwise
    if (M > 32) {
      launch_tiles<KB, WAVES, U, AFF, 4>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
      return;
    }
  }
  if (M > 16) {
    launch_tiles<KB, WAVES, U, AFF, 2>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
    return;
  }
  const int MR = M == 1 ? 1 : (M == 2 ? 2 : 4);
  // Direct x loads: as many row groups per block as keep about one block per
  // CU (x is re-read by every block, so fewer, wider blocks move less of it).
  // (Only where the weight registers of RG groups fit without spilling: 16
  // waves per block leave 128 VGPRs per lane.)
  constexpr bool rg4 = WAVES <= 8, rg2 = WAVES <= 8 || U <= 6;
  if constexpr (rg4) {
    if (M > 4 && N >= 256 * 16 * 4) {
      launch_mr<KB, WAVES, U, 0, 4, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
      return;
    }
  }
  if constexpr (rg2) {
    if (M > 4 && N >= 256 * 16 * 2) {
      launch_mr<KB, WAVES, U, 0, 2, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
      return;
    }
  }
  if (M > 4 || skinny_lds(WAVES, U, KB, MR) > kSkinnyLdsMax)
    launch_mr<KB, WAVES, U, 0, 1, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
  else if (MR == 1)
    launch_mr<KB, WAVES, U, 1, 1, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
  else if (MR == 2)
    launch_mr<KB, WAVES, U, 2, 1, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
  else
    launch_mr<KB, WAVES, U, 4, 1, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
}

// Waves per block and K-blocks per wave for nkb K-blocks: the fewest waves
// (<= 16) that cover K with at most 4 K-blocks each, else 16 waves with up to 8.
template <int KB, bool AFF>
static void launch_kb(const _Float16* x, int M, const uint8_t* packed, const uint16_t* scales,
                      const uint8_t* zeros, int N, int K, int G, int kbs, void* y, Epilogue ep,
                      hipStream_t stream) {
  const int nkb = K / KB;
  if (nkb <= 4 * 2) launch_one<KB, 4, 2, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
  else if (nkb <= 4 * 4) launch_one<KB, 4, 4, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
  else if (nkb <= 8 * 4) launch_one<KB, 8, 4, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
  else if (nkb <= 16 * 4) launch_one<KB, 16, 4, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
  else if (nkb <= 16 * 6) launch_one<KB, 16, 6, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
  else launch_one<KB, 16, 8, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream);
}

template <bool AFF>
static void launch_skinny_t(const _Float16* xh, int M, const uint8_t* packed,
                            const uint16_t* scales, const uint8_t* zeros, int N, int K, int G,
                            int KB, int kbs, void* y, Epilogue ep, hipStream_t stream) {
  switch (KB) {
    case 128: launch_kb<128, AFF>(xh, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream); break;
    case 64: launch_kb<64, AFF>(xh, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream); break;
    default: launch_kb<32, AFF>(xh, M, packed, scales, zeros, N, K, G, kbs, y, ep, stream); break;
  }
}

hipError_t launch_matmul_skinny(const void* x, int64_t M, const uint8_t* packed,
                                const uint16_t* scales, const uint8_t* zeros, int64_t N,
                                int64_t K, int64_t group, void* y, Epilogue ep,
                                hipStream_t stream) {
  const int KB = skinny_kb(group);
  const int G = (int)((K + group - 1) / group);
  if (M > 32 && K / KB > 16 * 6) return hipErrorInvalidValue;   // refused by matmul_skinny_unsupported
  int kbs = 0;
  while ((KB << kbs) < group) ++kbs;                  // group = KB << kbs
  const _Float16* xh = static_cast<const _Float16*>(x);
  if (zeros)
    launch_skinny_t<true>(xh, (int)M, packed, scales, zeros, (int)N, (int)K, G, KB, kbs, y, ep, stream);
  else
    launch_skinny_t<false>(xh, (int)M, packed, scales, zeros, (int)N, (int)K, G, KB, kbs, y, ep, stream);
  return hipGetLastError();
}

}  // namespace int4dq
