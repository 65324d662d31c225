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
// sp.S > 1: the block takes share blockIdx.y of K (K-blocks kb0 .. kb0 +
// sp.kb_per_share - 1, kb0 = blockIdx.y * sp.kb_per_share, a whole number of
// groups) and writes its partial [M, 16 RG] tile to sp.part instead of y.
// GPK = 2 or 4 (MR = 0 only): each K-block holds GPK groups of KB / GPK
// codes (two of 32 or 64, four of 32), whose integer sums are kept apart (an
// MFMA per group, the other groups' codes zeroed) and multiplied by their own
// scales; the scales (zero points) of a K-block are one 4- or 8-byte (2- or
// 4-byte) load. K-blocks of several groups cut the loads and K-block steps
// at 5 or more rows of x.
template <int KB, int WAVES, int U, int MR, int RG, bool AFF, int MT = 1, int GPK = 1>
__global__ __launch_bounds__(WAVES * 64) void matmul_skinny_kernel(
    const _Float16* __restrict__ x, int M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N, int K, int G,
    int kb_shift, void* __restrict__ y, Epilogue ep, SkinnySplit sp) {
  typedef typename WLoad<KB>::T wvec_t;
  constexpr int DW = KB / 32;                 // code words per lane per K-block = MFMAs
  constexpr int XB = (RG > 1 || MT > 1) ? 1 : (U < 4 ? U : 4);   // K-blocks per batch of direct x loads
  static_assert(MR == 0 || (RG == 1 && MT == 1), "row groups and row tiles with direct x loads only");
  static_assert(GPK == 1 || ((GPK == 2 || GPK == 4) && KB / GPK >= 32 && MR == 0),
                "several groups per K-block: groups of 32 codes or more, direct x loads");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* red = reinterpret_cast<float*>(lds);                  // [WAVES][RG][MT][64][4]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int col = lane & 15, h = lane >> 4;
  // GPK > 1: lane group h holds codes h KB/4 .. (h+1) KB/4 - 1 of a K-block,
  // all in the K-block's group (h GPK) / 4
  const int lgrp = (h * GPK) >> 2;
  const int n0 = blockIdx.x * 16 * RG;
  const int q = blockIdx.y;                    // share of K (0 without a split)
  const int kb0 = q * sp.kb_per_share;                  // its first K-block
  const int nkb = sp.S > 1 ? min(sp.kb_per_share, K / KB - kb0) : K / KB;   // K-blocks of the share
  x += (int64_t)kb0 * KB;                      // every x address below is x + m K + j KB + ...
  const uint8_t* prow[RG];
  const uint16_t* srow[RG];
  const uint8_t* zrow[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int nrow = (n0 + 16 * r + col < N) ? n0 + 16 * r + col : N - 1;   // tail rows: read, discard
    prow[r] = packed + (int64_t)nrow * (K >> 1) + (int64_t)kb0 * (KB / 2) + h * (KB / 8);
    const int g0 = GPK > 1 ? GPK * kb0 : kb0 >> kb_shift;   // first group of the share
    srow[r] = scales + (int64_t)nrow * G + g0;
    zrow[r] = AFF ? zeros + (int64_t)nrow * G + g0 : nullptr;
  }

  // Weight and scale loads of the wave's share, K-block by K-block. They are
  // issued after the (smaller) x staging loads, so that each K-block's
  // compute waits only for its own weights (loads return in order).
  wvec_t wv[RG][U];
  uint32_t sraw[RG][U][GPK == 4 ? 2 : 1], zraw[RG][U];   // scale bits (two per word), zero points
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
        if constexpr (GPK == 4) {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(srow[r] + 4 * j);
          sraw[r][u][0] = v.x;
          sraw[r][u][GPK == 4 ? 1 : 0] = v.y;
        } else if constexpr (GPK == 2) {
          sraw[r][u][0] = *reinterpret_cast<const uint32_t*>(srow[r] + 2 * j);
        } else {
          sraw[r][u][0] = srow[r][j >> kb_shift];
        }
      }
    if constexpr (AFF) {
#pragma unroll
      for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = wave + u * WAVES < nkb ? wave + u * WAVES : nkb - 1;
          if constexpr (GPK == 4) zraw[r][u] = *reinterpret_cast<const uint32_t*>(zrow[r] + 4 * j);
          else if constexpr (GPK == 2) zraw[r][u] = *reinterpret_cast<const uint16_t*>(zrow[r] + 2 * j);
          else zraw[r][u] = zrow[r][j >> kb_shift];
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
        acc[0][0] += half_bits_to_float((uint16_t)sraw[0][u][0]) * d;
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
            float4_t d[GPK][MT];               // integer sums, one per group of the K-block
#pragma unroll
            for (int q = 0; q < GPK; ++q)
#pragma unroll
              for (int t = 0; t < MT; ++t) d[q][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < DW; ++i) {
              half2_t hw[4];
              if constexpr (AFF) {
                // (GPK > 1: the zero point of the lane's own group)
                const uint32_t zb = zp_bias_natural(GPK > 1 ? (zraw[r][u] >> (8 * lgrp)) & 0xFFu : zraw[r][u]);
                codes_to_half_natural_zp(word_at<KB>(wv[r][u], i), hw, zb);
              } else {
                codes_to_half_natural(word_at<KB>(wv[r][u], i), hw);
              }
              if constexpr (GPK > 1) {
                // An MFMA adds the products of all four lane groups, and lane
                // group h holds codes of the K-block's group (h GPK) / 4 only:
                // each group's sum is an MFMA in which the other groups'
                // lanes give zeros.
#pragma unroll
                for (int g = 0; g < GPK; ++g) {
                  const uint32_t keep = lgrp == g ? 0xFFFFFFFFu : 0u;
                  half2_t hg[4];
#pragma unroll
                  for (int k = 0; k < 4; ++k)
                    hg[k] = __builtin_bit_cast(half2_t, __builtin_bit_cast(uint32_t, hw[k]) & keep);
                  const half8_t bg = as_half8(hg);
#pragma unroll
                  for (int t = 0; t < MT; ++t)
                    d[g][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[t][v][i], bg, d[g][t], 0, 0, 0);
                }
              } else {
                const half8_t bw = as_half8(hw);
#pragma unroll
                for (int t = 0; t < MT; ++t)
                  d[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[t][v][i], bw, d[0][t], 0, 0, 0);
              }
            }
            // each group's integer sum times its scale, groups in order
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              float4_t part = half_bits_to_float((uint16_t)sraw[r][u][0]) * d[0][t];
#pragma unroll
              for (int g = 1; g < GPK; ++g)
                part += half_bits_to_float((uint16_t)(sraw[r][u][g >> 1] >> (16 * (g & 1)))) * d[g][t];
              acc[r][t] += part;
            }
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
    if (n < N) {
      if (sp.S > 1) sp.part[((int64_t)q * M + m) * N + n] = s;
      else ep.store(y, (int64_t)m * N + n, s, n);
    }
  }
}

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left free (gfx9 encoding).
template <int NW>
__device__ __forceinline__ void wait_vmcnt_skinny() {
  static_assert(NW >= 0 && NW < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((NW & 0xF) | ((NW >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16 bytes per lane from x (a buffer of nbytes bytes) at byte voff + soff to
// LDS at lds + 16 * lane, by DMA. (A device function rather than a lambda
// body: the buffer resource type exists only on the device side.)
__device__ __forceinline__ void x_to_lds(const _Float16* x, int nbytes, uint8_t* lds, uint32_t voff,
                                         int soff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<_Float16*>(x), (short)0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff,
                                           0, 0);
}

// 16 bytes per lane from p (a buffer of nbytes bytes) at byte voff + soff to
// LDS at lds + 16 * lane, by DMA; bytes past nbytes read as zero.
template <typename T>
__device__ __forceinline__ void lds_dma_16(const T* p, int nbytes, uint8_t* lds, uint32_t voff, int soff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(p), (short)0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff,
                                           0, 0);
}

// v of lane i ^ 8 in each row of 16 lanes (DPP row_ror:8).
__device__ __forceinline__ uint32_t swap8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
}

// Pipelined form for 5 to 16 rows of x with K a multiple of 256 and group
// sizes 128 * 2^p. A block of 4 wavefronts (8, with one pair-block in flight
// each, for one row group and long rows) owns RG (1 to 4) groups of 16 weight rows;
// the wavefronts split K into pair-blocks of 256 codes (two K-blocks;
// wavefront w takes pair-blocks w, w + 4, ...), and each walks its share with
// the loads of the next P pair-blocks in flight.
//
//  * Weights: a pair-block is 128 bytes -- one whole cache line -- of each of
//    16 rows, read by two loads of 8 rows x 128 bytes (load A: rows 0-7,
//    load B: rows 8-15; lane (n, g) = (lane % 16, lane / 16) reads piece
//    g + 4 (n / 8) of row n % 8 in A and piece g + 4 (1 - n / 8) of row
//    8 + n % 8 in B). Loads of 16 rows x 64 bytes touch each line twice and
//    ran a quarter slower in a read-only test. The MFMA wants row n in lane
//    (n, g): pieces g and 4 + g of row n are the lane's own half of one load
//    and the other half of lane (n ^ 8, g)'s, fetched by one DPP row rotate.
//    Piece g holds codes 32 g .. 32 g + 31 of the first K-block, piece 4 + g
//    those of the second, so MFMAs 0-3 (first K-block, first group) and 4-7
//    (second) each stay inside one group.
//  * x: the pair-block of x (XR rows x 512 bytes, XR = 8 or 16) goes into a
//    slot of the wavefront's own LDS ring by DMA (2 rows per load); 16-byte
//    chunk c of row r sits at position c ^ r, so sixteen rows' reads of one
//    chunk fall in distinct banks.
//  * Scales (and zero points): the block's rows hold them contiguously, so
//    they are copied to LDS once, at the start, by whole-line DMA (per-step
//    loads touched one line per row for 4 bytes and cost as much request
//    traffic as the weights). A step reads both K-blocks' scales of a row
//    with one 32-bit LDS read when the group is 128 (GP), else one 16-bit
//    read that serves both.
// The MFMA arithmetic is the direct-load form of the kernel above (natural
// code order, the group's scale on each partial; rows of x >= M repeat a
// lower row and are discarded). The four wavefronts' partial tiles are added
// through LDS at the end.
template <int RG, int P, bool AFF, int XR, bool GP, int WAVES_ = 4>
__global__ __launch_bounds__(64 * WAVES_) void matmul_skinny_pipe_kernel(
    const _Float16* __restrict__ x, int M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N, int K, int G,
    int kb_shift, void* __restrict__ y, Epilogue ep) {
  // Dynamic LDS: the block's scales (16 RG G binary16, rounded up to 1 KB),
  // then its zero points (16 RG G bytes, rounded up to 1 KB).
  extern __shared__ __attribute__((aligned(16))) uint8_t sz_lds[];
  constexpr int PB = 256, WAVES = WAVES_;      // codes per pair-block; wavefronts (4 or 8)
  static_assert(WAVES == 4 || WAVES == 8, "wavefronts per block");
  static_assert(XR == 8 || XR == 16, "x rows staged");
  constexpr int XI = XR / 2;                   // x DMA loads per pair-block (2 rows each)
  constexpr int SLOT = XR * 2 * PB;            // bytes of one pair-block of x
  constexpr int RING = WAVES * P * SLOT;
  constexpr int RED = WAVES * RG * 64 * 16;    // the partial tiles at the end
  __shared__ __attribute__((aligned(1024))) uint8_t lds[RING > RED ? RING : RED];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const bool lo = col < 8;
  const int n0 = blockIdx.x * 16 * RG;
  const int npb = K / PB;
  const int nj = (npb - wave + WAVES - 1) / WAVES;   // pair-blocks of this wavefront (>= 1: npb >= 4)
  const int nrows = N - n0 < 16 * RG ? N - n0 : 16 * RG;   // rows of the block below N
  const uint8_t* wa[RG];
  const uint8_t* wb[RG];
  int srow[RG];                                // LDS scale index of the lane's row
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    // rows past N: read row N - 1, discard
    const int ra = n0 + 16 * r + (col & 7), rb = ra + 8, rl = 16 * r + col;
    wa[r] = packed + (int64_t)(ra < N ? ra : N - 1) * (K >> 1) + 16 * (g + 4 * (col >> 3));
    wb[r] = packed + (int64_t)(rb < N ? rb : N - 1) * (K >> 1) + 16 * (g + 4 * ((col >> 3) ^ 1));
    srow[r] = (rl < nrows ? rl : nrows - 1) * G;
  }
  const int sbytes = (16 * RG * G * 2 + 1023) & ~1023;
  const uint16_t* const ssh = reinterpret_cast<const uint16_t*>(sz_lds);
  const uint8_t* const zsh = sz_lds + sbytes;
  {
    // 1 KB per DMA load (lane l: bytes 16 l); bytes past the block's rows
    // (range-checked by the buffer load) read as zero and are not used
    const int su = sbytes >> 10;
    for (int u = wave; u < su; u += WAVES)
      lds_dma_16(scales + (int64_t)n0 * G, nrows * G * 2, sz_lds + u * 1024, (uint32_t)(u * 1024 + 16 * lane), 0);
    if constexpr (AFF) {
      const int zu = (16 * RG * G + 1023) >> 10;
      for (int u = wave; u < zu; u += WAVES)
        lds_dma_16(zeros + (int64_t)n0 * G, nrows * G, sz_lds + sbytes + u * 1024,
                   (uint32_t)(u * 1024 + 16 * lane), 0);
    }
  }
  // DMA source of lane l in x load t: row 2t + l/32 (rows >= M: row M-1),
  // chunk (l % 32) ^ row, so that position l % 32 of the row holds that chunk
  // (byte offsets into x; M * K * 2 < 2^31 is checked by the launcher). The
  // loads are buffer loads: the compiler's wait counting treats a pending
  // global-to-LDS load of the flat kind as possibly out of order and would
  // wait for every load at the loop top.
  const int xbytes = M * K * 2;
  uint32_t xoff[XI];
#pragma unroll
  for (int t = 0; t < XI; ++t) {
    const int r = 2 * t + (lane >> 5);
    const int rr = r < M ? r : M - 1;
    xoff[t] = (uint32_t)(rr * K * 2 + 16 * ((lane & 31) ^ r));
  }
  uint8_t* const ring = lds + wave * (P * SLOT);
  // A operand of lane (col, g) for MFMA i: chunk (i < 4 ? 0 : 16) + 4g +
  // i % 4 of row col (row col % XR: rows past XR are past M and discarded).
  const int xr = col & (XR - 1);
  int aoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) aoff[i] = xr * (2 * PB) + 16 * ((((i >> 2) << 4) + 4 * g + (i & 3)) ^ xr);

  // Ring of P in-flight pair-blocks. Slot q holds the wavefront's pair-block
  // j with j % P == q; an index past the share is clamped to its last one
  // (loaded, not used), so every step issues the same loads.
  u32x4_t wva[P][RG], wvb[P][RG];
  // A step past the wavefront's share (the ring's last round) still issues
  // its loads, so that the load counts the waits rely on stay fixed, but
  // every lane of them reads the first 16 bytes of x and of the codes: one
  // cache line each, not a pair-block's worth of traffic.
  auto issue = [&](int j, int q) __attribute__((always_inline)) {
    const bool live = j < nj;
    const int pb = wave + WAVES * (live ? j : nj - 1);
#pragma unroll
    for (int t = 0; t < XI; ++t)
      x_to_lds(x, xbytes, ring + q * SLOT + t * 1024, live ? xoff[t] : 0u, live ? pb * (2 * PB) : 0);
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const uint8_t* pa = live ? wa[r] + pb * (PB / 2) : packed;
      const uint8_t* pbb = live ? wb[r] + pb * (PB / 2) : packed;
      wva[q][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pa));
      wvb[q][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pbb));
    }
  };

  float4_t acc[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) acc[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // Step j past the share (the last round of the ring) repeats the last
  // pair-block with a zero scale factor: no branch in the loop, and its
  // (finite) partial contributes nothing.
  auto compute = [&](int q, int j) __attribute__((always_inline)) {
    const bool live = j < nj;
    const int pb = wave + WAVES * (live ? j : nj - 1);
    const int si = GP ? 2 * pb : (2 * pb) >> kb_shift;
    half8_t xf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xf[i] = *reinterpret_cast<const half8_t*>(ring + q * SLOT + aoff[i]);
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      uint32_t w[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t a = wva[q][r][k], b = wvb[q][r][k];
        w[k] = lo ? a : b;                     // own row, piece g
        w[4 + k] = swap8(lo ? b : a);          // own row, piece 4 + g (from lane n ^ 8)
      }
      const uint32_t s2 = GP ? *reinterpret_cast<const uint32_t*>(ssh + srow[r] + si) : ssh[srow[r] + si];
      const float s0 = half_bits_to_float((uint16_t)s2);
      const float s1 = half_bits_to_float((uint16_t)(GP ? s2 >> 16 : s2));
      uint32_t zb0 = 0u, zb1 = 0u;
      if constexpr (AFF) {
        zb0 = zp_bias_natural(zsh[srow[r] + si]);
        zb1 = zp_bias_natural(zsh[srow[r] + si + (GP ? 1 : 0)]);
      }
      float4_t d0 = {0.0f, 0.0f, 0.0f, 0.0f}, d1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        half2_t hw[4];
        if constexpr (AFF) codes_to_half_natural_zp(w[i], hw, zb0);
        else codes_to_half_natural(w[i], hw);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xf[i], as_half8(hw), d0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        half2_t hw[4];
        if constexpr (AFF) codes_to_half_natural_zp(w[4 + i], hw, zb1);
        else codes_to_half_natural(w[4 + i], hw);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xf[4 + i], as_half8(hw), d1, 0, 0, 0);
      }
      acc[r] += (live ? s0 : 0.0f) * d0 + (live ? s1 : 0.0f) * d1;
    }
  };

  // Loads per step; step j waits only for its own (loads complete in order,
  // the x DMA included): the P - 1 steps issued after it may still be in
  // flight. Its slot is then read back and refilled by the step P later.
  constexpr int L = XI + 2 * RG;
  static_assert(P * L < 64, "vmcnt range");
  // The prologue keeps its issue order too, so the first round's waits are
  // the same as every later round's; the loop runs at least once (nj >= 1),
  // so no branch separates it from the prologue.
#pragma unroll
  for (int q = 0; q < P; ++q) {
    issue(q, q);
    __builtin_amdgcn_sched_barrier(0);
  }
  // every wavefront's scale and zero-point copies (older than the prologue's
  // loads) have landed. A bare barrier: __syncthreads would also wait for
  // the prologue's x copies, which only this wavefront reads.
  wait_vmcnt_skinny<P * L>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  int j0 = 0;
  do {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      wait_vmcnt_skinny<(P - 1) * L>();
      __builtin_amdgcn_sched_barrier(0);
      compute(q, j0 + q);
      __builtin_amdgcn_sched_barrier(0);
      issue(j0 + q + P, q);
      __builtin_amdgcn_sched_barrier(0);
    }
    j0 += P;
  } while (j0 < nj);
  wait_vmcnt_skinny<0>();

  // Sum the four wavefronts' 16x16 partial tiles (the ring's LDS is reused
  // once every wavefront is done with it). Lane l holds rows 4*(l/16) + i of
  // column l%16.
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);   // [WAVES][RG][64][4]
#pragma unroll
  for (int r = 0; r < RG; ++r) *reinterpret_cast<float4_t*>(red + ((wave * RG + r) * 64 + lane) * 4) = acc[r];
  __syncthreads();
  for (int t = tid; t < 16 * M * RG; t += 64 * WAVES) {
    const int r = t / (16 * M), rem = t - r * 16 * M;
    const int m = rem >> 4, nn = rem & 15;
    const int src = (m >> 2) * 16 + nn, i = m & 3;
    auto at = [&](int w) { return red[((w * RG + r) * 64 + src) * 4 + i]; };
    float v = (at(0) + at(1)) + (at(2) + at(3));
    if constexpr (WAVES == 8) v += (at(4) + at(5)) + (at(6) + at(7));
    const int n = n0 + 16 * r + nn;
    if (n < N) ep.store(y, (int64_t)m * N + n, v, n);
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
  // (up to 64 threads per weight row; a dispatch holds fewer than 2^32)
  if (N >= (1ll << 25)) return "skinny kernel needs N below 2^25";
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

template <int KB, int WAVES, int U, int MR, int RG, bool AFF, int MT = 1, int GPK = 1>
static void launch_mr(const _Float16* x, int M, const uint8_t* packed, const uint16_t* scales,
                      const uint8_t* zeros, int N, int K, int G, int kbs, void* y, Epilogue ep, const SkinnySplit& sp,
                      hipStream_t stream) {
  hipLaunchKernelGGL((matmul_skinny_kernel<KB, WAVES, U, MR, RG, AFF, MT, GPK>),
                     dim3((unsigned)((N + 16 * RG - 1) / (16 * RG)), (unsigned)sp.S), dim3(WAVES * 64),
                     skinny_lds(WAVES, U, KB, MR, RG, MT), stream, x, M, packed, scales, zeros, N, K, G,
                     kbs, y, ep, sp);
}

// 17 <= M <= 64: MT = 2 or 4 row tiles, direct x loads. Every block re-reads
// its rows' share of x (M/(4 RG) bytes of x per byte of weights), so the
// block takes as many row groups as its registers allow while the grid keeps
// about one block per CU.
template <int KB, int WAVES, int U, bool AFF, int MT, int GPK>
static void launch_tiles(const _Float16* x, int M, const uint8_t* packed, const uint16_t* scales,
                         const uint8_t* zeros, int N, int K, int G, int kbs, void* y, Epilogue ep, const SkinnySplit& sp,
                         hipStream_t stream) {
  constexpr bool rg2 = WAVES <= 8;
  if constexpr (rg2) {
    if (N >= 256 * 16 * 2) {
      launch_mr<KB, WAVES, U, 0, 2, AFF, MT, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
      return;
    }
  }
  launch_mr<KB, WAVES, U, 0, 1, AFF, MT, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
}

template <int KB, int WAVES, int U, bool AFF, int GPK>
static void launch_one(const _Float16* x, int M, const uint8_t* packed, const uint16_t* scales,
                       const uint8_t* zeros, int N, int K, int G, int kbs, void* y, Epilogue ep, const SkinnySplit& sp,
                       hipStream_t stream) {
  if constexpr ((WAVES < 16 || U <= 6) && GPK < 4) {   // refused by matmul_skinny_unsupported otherwise
    // (four groups per K-block are not taken for more than 32 rows of x: four
    // sums of four row tiles would spill)
    if (M > 32) {
      launch_tiles<KB, WAVES, U, AFF, 4, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
      return;
    }
  }
  if (M > 16) {
    launch_tiles<KB, WAVES, U, AFF, 2, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
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
      launch_mr<KB, WAVES, U, 0, 4, AFF, 1, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
      return;
    }
  }
  if constexpr (rg2) {
    if (M > 4 && N >= 256 * 16 * 2) {
      launch_mr<KB, WAVES, U, 0, 2, AFF, 1, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
      return;
    }
  }
  if (GPK > 1 || M > 4 || skinny_lds(WAVES, U, KB, MR) > kSkinnyLdsMax) {
    launch_mr<KB, WAVES, U, 0, 1, AFF, 1, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
    return;
  }
  if constexpr (GPK != 1) return;              // (several groups per K-block only with M > 4)
  else if (MR == 1)
    launch_mr<KB, WAVES, U, 1, 1, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
  else if (MR == 2)
    launch_mr<KB, WAVES, U, 2, 1, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
  else
    launch_mr<KB, WAVES, U, 4, 1, AFF>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
}

// Waves per block and K-blocks per wave for nkb K-blocks: the fewest waves
// (<= 16) that cover K with at most 4 K-blocks each, else 16 waves with up to 8.
template <int KB, bool AFF, int GPK>
static void launch_kb(const _Float16* x, int M, const uint8_t* packed, const uint16_t* scales,
                      const uint8_t* zeros, int N, int K, int G, int kbs, void* y, Epilogue ep, const SkinnySplit& sp,
                      hipStream_t stream) {
  const int nkb = sp.S > 1 ? sp.kb_per_share : K / KB;   // K-blocks of one block (of its share)
  if (nkb <= 4 * 2) launch_one<KB, 4, 2, AFF, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
  else if (nkb <= 4 * 4) launch_one<KB, 4, 4, AFF, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
  else if (nkb <= 8 * 4) launch_one<KB, 8, 4, AFF, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
  // (K-blocks of two groups number at most 64, of four at most 32: K <= 128
  // groups; the longer forms are not built for them)
  else if constexpr (GPK <= 2) {
    if (nkb <= 16 * 4) launch_one<KB, 16, 4, AFF, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
    else if constexpr (GPK == 1) {
      if (nkb <= 16 * 6) launch_one<KB, 16, 6, AFF, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
      else launch_one<KB, 16, 8, AFF, GPK>(x, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream);
    }
  }
}

// KB: codes per group-sized K-block (skinny_kb). gpk = 2 or 4: K-blocks of
// gpk groups (gpk KB codes) instead.
template <bool AFF>
static void launch_skinny_t(const _Float16* xh, int M, const uint8_t* packed,
                            const uint16_t* scales, const uint8_t* zeros, int N, int K, int G,
                            int KB, int kbs, int gpk, void* y, Epilogue ep, const SkinnySplit& sp,
                            hipStream_t stream) {
  if (gpk == 4) {                              // K-blocks of four groups of 32
    launch_kb<128, AFF, 4>(xh, M, packed, scales, zeros, N, K, G, 0, y, ep, sp, stream);
    return;
  }
  if (gpk == 2) {                              // K-blocks of two groups (32 or 64 codes)
    if (KB == 32) launch_kb<64, AFF, 2>(xh, M, packed, scales, zeros, N, K, G, 0, y, ep, sp, stream);
    else launch_kb<128, AFF, 2>(xh, M, packed, scales, zeros, N, K, G, 0, y, ep, sp, stream);
    return;
  }
  switch (KB) {
    case 128: launch_kb<128, AFF, 1>(xh, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream); break;
    case 64: launch_kb<64, AFF, 1>(xh, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream); break;
    default: launch_kb<32, AFF, 1>(xh, M, packed, scales, zeros, N, K, G, kbs, y, ep, sp, stream); break;
  }
}

// Split of K (only with a workspace), for 5 to 64 rows of x against small
// matrices with long rows: with fewer than 128 groups of 16 weight rows the
// grid leaves at least half the CUs idle, and each block walks all of K for
// its rows alone. K is then cut into S = 2, 4 or 8 shares (the most that keep
// the grid within two blocks per CU), each at least 6 K-blocks and a whole
// number of groups; the shares' partial tiles meet in the workspace and a
// second kernel adds them in share order, as for the tiled kernel. That
// second kernel and the boundary between the two cost about 4 us, so the
// split is taken only where a block's work is long enough to lose more than
// that: at least 48 K-blocks (of skinny_rows_kb codes) times 16-row tiles of
// x per row group, and not where the pipelined form runs (5 to 16 rows,
// groups of 128 2^p). Measured (graph replays over a >= 1 GiB pool, split
// against unsplit): [1024, 8192] M = 64 17.1 / 36.4 us, [1000, 4096] M = 33
// 9.3 / 13.4, [768, 3072] group 128 M = 32 7.7 / 9.5, group 64 M = 32 8.2 /
// 9.8 and M = 40 9.0 / 12.5, group 32 M = 32 9.7 / 11.7, [100, 4096] group 32
// M = 17 7.8 / 10.2 and M = 5 6.8 / 7.7; at the threshold group 32 M = 16
// 8.84 / 8.86; below it the split lost: [768, 3072] group 64 M = 16 7.5 /
// 7.4 and M = 8 7.0 / 6.5, [300, 2048] group 64 M = 24 7.4 / 6.7.
struct SkinnyPlan {
  int S, kb_per_share;
  int64_t ws_bytes;
};
static bool skinny_pipe_takes(int64_t M, int KB, int64_t K) {
  return M > 4 && M <= 16 && KB == 128 && K % 256 == 0 && K >= 4 * 256 && M * K * 2 < ((int64_t)1 << 31);
}
// Codes per K-block of the older form for 5 or more rows of x: groups 32 and
// 64 run as K-blocks of 128 codes (four or two groups) where K allows, group
// 32 else as 64-code K-blocks of two groups (see the kernel).
static int skinny_rows_kb(int64_t M, int64_t K, int64_t group) {
  if ((group == 32 || group == 64) && M > 4 && K % 128 == 0) return 128;
  if (group == 32 && M > 4 && K % 64 == 0) return 64;
  return skinny_kb(group);
}
// (kb_per_share counts K-blocks of skinny_rows_kb(M, K, group) codes)
static SkinnyPlan skinny_plan(int64_t M, int64_t N, int64_t K, int64_t group) {
  SkinnyPlan pl{1, 0, 0};
  const int KB = skinny_rows_kb(M, K, group);
  if (KB == 0 || M <= 4 || K % KB != 0 || skinny_pipe_takes(M, skinny_kb(group), K)) return pl;
  const int64_t per_group = group > KB ? group / KB : 1;   // K-blocks per group (a power of two)
  const int64_t nkb = K / KB, rgroups = (N + 15) / 16, tiles = (M + 15) / 16;
  if (rgroups >= 128 || nkb * tiles < 48) return pl;
  for (int S = 8; S >= 2; S /= 2) {
    if (rgroups * S > 512) continue;
    int64_t kbps = (nkb + S - 1) / S;
    kbps = (kbps + per_group - 1) / per_group * per_group;
    const int64_t shares = (nkb + kbps - 1) / kbps;
    if (kbps < 6 || shares < 2) continue;
    pl.S = (int)shares;
    pl.kb_per_share = (int)kbps;
    break;
  }
  if (pl.S > 1) pl.ws_bytes = (int64_t)pl.S * M * N * 4;
  return pl;
}

int64_t matmul_skinny_workspace(int64_t M, int64_t N, int64_t K, int64_t group) {
  if (M < 1 || M > 64 || N >= (1ll << 25)) return 0;
  return skinny_plan(M, N, K, group).ws_bytes;
}

hipError_t launch_matmul_skinny(const void* x, int64_t M, const uint8_t* packed,
                                const uint16_t* scales, const uint8_t* zeros, int64_t N,
                                int64_t K, int64_t group, void* y, Epilogue ep, void* workspace,
                                int64_t workspace_bytes, hipStream_t stream) {
  const int KB = skinny_kb(group);
  const int G = (int)((K + group - 1) / group);
  if (M > 32 && K / KB > 16 * 6) return hipErrorInvalidValue;   // refused by matmul_skinny_unsupported
  int kbs = 0;
  while ((KB << kbs) < group) ++kbs;                  // group = KB << kbs
  const _Float16* xh = static_cast<const _Float16*>(x);
  // Groups per K-block (1, 2 or 4): a K-block's scales (zero points) are read
  // as one 2 gpk-byte (gpk-byte) word, so the arrays must be aligned to that;
  // else fewer groups per K-block.
  int gpk = skinny_rows_kb(M, K, group) / KB;
  if (gpk == 4 && M > 32) gpk = 2;             // (four sums of four row tiles would spill)
  while (gpk > 1 && (((uintptr_t)scales & (2 * gpk - 1)) != 0 || ((uintptr_t)zeros & (gpk - 1)) != 0 ||
                     K % (gpk * group) != 0))
    gpk >>= 1;
  if (K > 128 * group) gpk = 1;                // (refused by matmul_skinny_unsupported)
  const SkinnyPlan pl = skinny_plan(M, N, K, group);
  SkinnySplit sp{nullptr, 1, 0};
  if (pl.S > 1 && workspace && workspace_bytes >= pl.ws_bytes) {
    // the plan counts K-blocks of skinny_rows_kb codes; with fewer groups per
    // K-block (unaligned scales) a share is proportionally more K-blocks
    const int kbps = pl.kb_per_share * (skinny_rows_kb(M, K, group) / (gpk * KB));
    sp = SkinnySplit{static_cast<float*>(workspace), pl.S, kbps};
    if (zeros)
      launch_skinny_t<true>(xh, (int)M, packed, scales, zeros, (int)N, (int)K, G, KB, kbs, gpk, y, ep, sp, stream);
    else
      launch_skinny_t<false>(xh, (int)M, packed, scales, zeros, (int)N, (int)K, G, KB, kbs, gpk, y, ep, sp, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_reduce(sp.part, sp.S, M, N, y, ep, stream);
  }
  if (skinny_pipe_takes(M, KB, K)) {
    // the pipelined form: 4 row groups per block on wide matrices (x is
    // re-read once per 64 weight rows); below 1024 row groups, the count of
    // 1, 2 or 3 that gives the busiest CU the fewest rows (blocks spread
    // evenly over 256 CUs; ties to more rows per block, which re-read x less):
    // 688 row groups take 3 (230 blocks, 48 rows per CU, against 64 with 2).
    // The scale and zero-point copies want 16-byte aligned arrays and at
    // most 32 KB of LDS.
    const int64_t rgroups = (N + 15) / 16;
    int RG = 4;
    if (rgroups < 4 * 256) {
      int64_t best = -1;
      for (int rg = 1; rg <= 3; ++rg) {
        const int64_t rows = ((rgroups + rg - 1) / rg + 255) / 256 * rg;
        if (best < 0 || rows <= best) best = rows, RG = rg;
      }
    }
    const bool gp = kbs == 0;
    const int lds_sz = ((16 * RG * G * 2 + 1023) & ~1023) + (zeros ? (16 * RG * G + 1023) & ~1023 : 0);
    if (((uintptr_t)scales & 15) == 0 && ((uintptr_t)zeros & 15) == 0 && lds_sz <= 32 * 1024) {
      // One row group per block and rows of 32 pair-blocks or more: eight
      // wavefronts with one pair-block in flight each (the same loads in
      // flight per CU, half as many steps per wavefront). Measured on
      // [4096, 11008] (graph replays over a >= 1 GiB pool): M = 16 11.66 ->
      // 11.25 us, M = 8 10.04 -> 9.64; on [4096, 4096] (16 pair-blocks) and
      // with several row groups per block it was slower.
      const bool eight = RG == 1 && K / 256 >= 32;
      const dim3 grid((unsigned)((rgroups + RG - 1) / RG)), block(eight ? 512 : 256);
#define INT4DQ_PIPE(RGV, A, XRV, GPV)                                                                  \
  do {                                                                                                 \
    if (RGV == 1 && eight)                                                                             \
      hipLaunchKernelGGL((matmul_skinny_pipe_kernel<1, 1, A, XRV, GPV, 8>), grid, block, lds_sz, stream, \
                         xh, (int)M, packed, scales, zeros, (int)N, (int)K, G, kbs, y, ep);              \
    else                                                                                               \
      hipLaunchKernelGGL((matmul_skinny_pipe_kernel<RGV, 2, A, XRV, GPV>), grid, block, lds_sz, stream,  \
                         xh, (int)M, packed, scales, zeros, (int)N, (int)K, G, kbs, y, ep);              \
  } while (0)
#define INT4DQ_PIPE_RG(A, XRV, GPV)                                                                    \
  do {                                                                                                 \
    if (RG == 4) INT4DQ_PIPE(4, A, XRV, GPV);                                                          \
    else if (RG == 3) INT4DQ_PIPE(3, A, XRV, GPV);                                                     \
    else if (RG == 2) INT4DQ_PIPE(2, A, XRV, GPV);                                                     \
    else INT4DQ_PIPE(1, A, XRV, GPV);                                                                  \
  } while (0)
#define INT4DQ_PIPE_X(A, GPV)                                                                          \
  do {                                                                                                 \
    if (M <= 8) INT4DQ_PIPE_RG(A, 8, GPV); else INT4DQ_PIPE_RG(A, 16, GPV);                            \
  } while (0)
      if (zeros) {
        if (gp) INT4DQ_PIPE_X(true, true); else INT4DQ_PIPE_X(true, false);
      } else {
        if (gp) INT4DQ_PIPE_X(false, true); else INT4DQ_PIPE_X(false, false);
      }
#undef INT4DQ_PIPE_X
#undef INT4DQ_PIPE_RG
#undef INT4DQ_PIPE
      return hipGetLastError();
    }
  }
  if (zeros)
    launch_skinny_t<true>(xh, (int)M, packed, scales, zeros, (int)N, (int)K, G, KB, kbs, gpk, y, ep, sp, stream);
  else
    launch_skinny_t<false>(xh, (int)M, packed, scales, zeros, (int)N, (int)K, G, KB, kbs, gpk, y, ep, sp, stream);
  return hipGetLastError();
}

}  // namespace int4dq
