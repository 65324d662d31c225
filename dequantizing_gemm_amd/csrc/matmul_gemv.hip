// matmul_gemv.hip -- dequantizing matrix-vector product (one to four
// activation rows, binary16 x) on gfx950: weight-streaming kernels bound by
// HBM bandwidth.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, int4_matmul): y = x @ dequantize(W).T,
// one group at a time -- x times the group's integer codes, then the group's
// scale. ("Build a Blockwise INT4 Inference Engine", architecture overview and
// takeaways: full-precision weights never reach memory; the bottleneck is
// memory bandwidth.)
//
// With one activation row every packed byte is used for two flops, so the
// kernels here are pure streams of the packed weights, and the way they read
// them decides their speed. Three variants, chosen by the launcher:
//
//  * large matrices (packed weights >= 48 MB, K <= 16384; K <= 14336 for
//    affine codes): whole rows per wavefront, 1 KB of one row per load,
//    4x4x4 MFMAs used on their diagonal (matmul_gemv_rows_kernel, below);
//  * K <= 12288 with group = 32 << p: 4 rows x 256 bytes per load, which is
//    directly the B operand of v_mfma_f32_4x4x4f16 (matmul_gemv_mfma_kernel);
//    this variant alone also takes 2 to 4 activation rows, as the four rows
//    of the MFMA's A operand (the loads, code expansions and MFMAs are those
//    of one row);
//  * everything else (K <= 32768, group a multiple of 32): the VALU kernel
//    that follows, where a wavefront load covers 1 KB of one weight row
//    (lane l: bytes c*1024 + 16 l):
//
//  * Block = C wavefronts x RW weight rows, C = ceil(row bytes / 1 KB).
//    Wavefront c owns byte chunk c of each of the block's rows; its lane l
//    owns 16 bytes = 32 consecutive codes, which lie inside one group (the
//    group size is a multiple of 32).
//  * The lane's 32 activations are loaded once and permuted to the "spread"
//    order (x0,x4),(x1,x5),(x2,x6),(x3,x7) per 8, matching
//    codes_to_half_spread (9 VALU ops per 8 exact fp16 codes). Each word is
//    then four v_dot2_f32_f16: exact products, fp32 sums.
//  * The lane's integer dot product is multiplied by its group's scale
//    (integer-first), summed over the wavefront (DPP and lane-read
//    butterfly) and over the block's wavefronts in a fixed order through
//    LDS: deterministic, no atomics.
//  * Lanes past the end of a row (last chunk) read the row's last 16 bytes
//    and contribute zero; rows past N are read as row N-1 and not written.
//
// Affine codes ("Build a Blockwise INT4 Inference Engine", step 2): every
// variant has an AFF form that also loads the group's zero point next to its
// scale and expands codes to u - zp (codes_to_half_spread_zp, same op count).
#include "device_common.h"
#include "kernels.h"

#include <type_traits>

namespace int4dq {
// Launch choices: the matrix-core variant where it applies, with 4
// wavefronts (16 rows) per block (measured best of 1, 2, 4 on the
// 7B-class and large-FFN shapes).
constexpr bool g_gemv_mfma = true;
constexpr int g_gemv_waves = 4;

namespace {
constexpr int kGemvMaxChunks = 16;             // wavefronts per block (1024 threads)

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left free (gfx9 encoding).
template <int NW>
__device__ __forceinline__ void wait_vmcnt_gemv() {
  static_assert(NW >= 0 && NW < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((NW & 0xF) | ((NW >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes, as a wave-uniform value: inside each 16-lane row a
// butterfly of lane pairs (DPP: lanes i^1, i^2, then i <-> 7-i, i <-> 15-i)
// leaves the row sum in every lane of the row; the four row sums are then
// read from lanes 0, 16, 32, 48 and added in a fixed order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);                         // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);                         // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);                        // row_half_mirror
  v += dpp_f<0x140>(v);                        // row_mirror
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}
}  // namespace

template <int RW, bool AFF>
__global__ __launch_bounds__(64 * kGemvMaxChunks) void matmul_gemv_kernel(
    const _Float16* __restrict__ x, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N, int K, int G,
    int group, int gsh, void* __restrict__ y, Epilogue ep) {
  __shared__ float red[kGemvMaxChunks][RW];
  const int lane = threadIdx.x & 63;
  const int c = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunks = blockDim.x >> 6;
  const int RB = K >> 1;                                       // bytes per packed row
  int o = c * 1024 + lane * 16;
  const bool active = o < RB;
  if (!active) o = RB - 16;                                    // valid address, zero contribution
  const int k0 = 2 * o;                                        // first code of the lane
  // group of the lane's codes: a shift when group / 32 is a power of two
  const uint32_t gi = gsh >= 0 ? (uint32_t)(o >> 4) >> gsh : (uint32_t)(k0 / group);
  const int n0 = blockIdx.x * RW;
  // Rows of the block (uniform; rows past N read row N-1 and are not written)
  // with 32-bit unsigned lane offsets from them, so the loads use a scalar base.
  auto row_of = [&](int r) { return n0 + r < N ? n0 + r : N - 1; };

  // Loads in the order they are consumed (loads complete in order): the
  // lane's activations, the RW scales, then the RW weight rows, so the
  // work on row r waits only for row r's weights.
  u32x4_t xv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    xv[i] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(x) + (uint32_t)(2 * k0 + 16 * i));
  // (scheduling barriers keep the three groups in this order: the compiler
  // would otherwise sink a load below the first use of an earlier one)
  __builtin_amdgcn_sched_barrier(0);
  uint32_t s[RW], z[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) s[r] = (scales + (int64_t)row_of(r) * G)[gi];
  if constexpr (AFF) {
#pragma unroll
    for (int r = 0; r < RW; ++r) z[r] = (zeros + (int64_t)row_of(r) * G)[gi];
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4_t w[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r)
    w[r] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(packed + (int64_t)row_of(r) * RB + (uint32_t)o));
  __builtin_amdgcn_sched_barrier(0);
  // spread order per 8 activations: (x0,x4), (x1,x5), (x2,x6), (x3,x7)
  uint32_t xs[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xs[i][0] = __builtin_amdgcn_perm(xv[i].z, xv[i].x, 0x05040100u);
    xs[i][1] = __builtin_amdgcn_perm(xv[i].z, xv[i].x, 0x07060302u);
    xs[i][2] = __builtin_amdgcn_perm(xv[i].w, xv[i].y, 0x05040100u);
    xs[i][3] = __builtin_amdgcn_perm(xv[i].w, xv[i].y, 0x07060302u);
  }

  // Lanes past the row end contribute 0 through a multiply by an opaque 0/1
  // mask (their data is a valid clamped copy, finite for finite inputs): with a
  // visible condition the compiler would put the row work in a branch and
  // sink loads into it.
  float keep = active ? 1.0f : 0.0f;
  asm volatile("" : "+v"(keep));
  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t hw[4];
      if constexpr (AFF) codes_to_half_spread_zp(w[r][i], hw, zp_bias_lo(z[r]), zp_bias_hi(z[r]));
      else codes_to_half_spread(w[r][i], hw);
#pragma unroll
      for (int j = 0; j < 4; ++j) p = __builtin_amdgcn_fdot2(hw[j], __builtin_bit_cast(half2_t, xs[i][j]), p, false);
    }
    acc[r] = half_bits_to_float((uint16_t)s[r]) * p * keep;
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0)
#pragma unroll
    for (int r = 0; r < RW; ++r) red[c][r] = acc[r];
  __syncthreads();
  if ((int)threadIdx.x < RW && n0 + (int)threadIdx.x < N) {
    float sum = 0.0f;
    for (int cc = 0; cc < nchunks; ++cc) sum += red[cc][threadIdx.x];
    ep.store(y, n0 + threadIdx.x, sum, n0 + threadIdx.x);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core variant for rows of up to 24 column blocks (K <= 12288).
//
// v_mfma_f32_4x4x4f16 computes 16 independent 4x4x4 products: lane 4b+i
// holds row i of block b's A, lane 4b+j holds column j of its B, and lane
// 4b+j receives column j of its D. So a wavefront load in which lane 4b+j
// reads 16 bytes of weight row j at byte 256c + 16b covers 4 rows x 256
// contiguous bytes (two full lines per row), and its B operands are
// already in place: block b is the 32-code slice b of column block c of the
// wave's 4 rows, and eight MFMAs (4 codes each, A = the matching
// activations) leave in D the lane's integer dot product -- one group slice,
// since the group is a multiple of 32 -- which the lane multiplies by its
// scale. The dot products cost 8 MFMAs instead of 16 v_dot2 per 32 codes.
//
// Block = W groups of 4 rows, each taken by KSP wavefronts that split the
// rows' column blocks (KSP = 2 for long rows). The activation row (permuted
// to the spread order, zero past K) and the block's scales are staged once in LDS;
// every weight load of a lane (one per column block) is issued before the
// first wait, and column c waits only for its own load. Used for group sizes
// 32 << p and K <= 12288; other shapes take the VALU kernel above.
// CM: column blocks (256 bytes) per row, >= ceil(K / 512). GS: min(gsh, 3)
// (group = 32 << gsh), which bounds the groups per row and so the scale
// entries each thread stages.
// KSP: wavefronts per group of 4 rows, each taking CM / KSP of the column
// blocks; their partial sums are added through LDS in a fixed order.
// MR: rows of x staged (1, or 4 for M = 2 .. 4). Lane 4b+i supplies row i of
// block b's A, so with MR = 4 the A rows are x rows 0 .. 3 (rows >= M are
// zeros) and D[i][j] -- register i of lane 4b+j -- is x row i times weight
// row j: the same loads, expansions and MFMAs give up to four outputs per
// weight row.
template <int CM, int GS, int W, bool AFF, int KSP = 1, int MR = 1>
__global__ __launch_bounds__(64 * W * KSP) void matmul_gemv_mfma_kernel(
    const _Float16* __restrict__ x, int M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N, int K, int G,
    int group, int gsh, void* __restrict__ y, Epilogue ep) {
  typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
  static_assert(CM % KSP == 0, "column split");
  constexpr int CMP = CM / KSP;                // column blocks per wavefront
  constexpr int NT = 64 * W * KSP, ROWS = 4 * W;   // threads, rows per block
  constexpr int XU = CM * 64;                  // 16-byte x units per staged row (x row <= CM KB)
  constexpr int XPT = (MR * XU + NT - 1) / NT; // x units per thread
  constexpr int GMAX = (CM * 16 + (1 << GS) - 1) >> GS;           // groups per row, at most
  constexpr int SPT = (ROWS * GMAX + NT - 1) / NT;                 // scale entries per thread
  // Sized so that every thread's staging store is in bounds (no branch: a
  // branch here would make the compiler wait for every load at its join).
  __shared__ __attribute__((aligned(16))) uint32_t xsp[XPT * NT * 4];   // x, spread order
  __shared__ uint16_t ssh[SPT * NT];                                  // scales of the block's rows
  __shared__ uint8_t zsh[AFF ? SPT * NT : 1];                         // their zero points
  __shared__ float part_sum[KSP > 1 ? KSP * ROWS * MR : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave = wid / KSP, part = wid % KSP;  // group of 4 rows, share of the columns
  const int b = lane >> 2, j = lane & 3;
  const int RB = K >> 1;
  const int n0 = blockIdx.x * ROWS;
  const int xunits = K >> 3;                   // 8 activations per unit

  // Phase 1: activations and scales (older than every weight load).
  // unit u of the staging: row u / XU, unit u % XU of that row (past the row
  // end or past row M-1: unit 0 of x, stored as zeros below)
  u32x4_t xv[XPT];
#pragma unroll
  for (int t = 0; t < XPT; ++t) {
    const int u = t * NT + tid;
    const int m = u / XU, uu = u - m * XU;
    const int src = m < M && uu < xunits ? m * xunits + uu : 0;
    xv[t] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(x) + 16u * (uint32_t)src);
  }
  // the block's rows' scales are contiguous from row n0 (rows past N: clamped)
  const uint16_t* sblk = scales + (int64_t)n0 * G;
  const int slast = (N - n0 < ROWS ? N - n0 : ROWS) * G - 1;
  uint32_t sv[SPT], zv[SPT];
#pragma unroll
  for (int t = 0; t < SPT; ++t) {
    const int e = t * NT + tid;
    sv[t] = sblk[(uint32_t)(e < slast ? e : slast)];
  }
  if constexpr (AFF) {
    const uint8_t* zblk = zeros + (int64_t)n0 * G;
#pragma unroll
    for (int t = 0; t < SPT; ++t) {
      const int e = t * NT + tid;
      zv[t] = zblk[(uint32_t)(e < slast ? e : slast)];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // Phase 2: the lane's 16 bytes of each column block of its row.
  const int n = n0 + 4 * wave + j < N ? n0 + 4 * wave + j : N - 1;
  const uint8_t* prow = packed + (int64_t)n * RB;
  u32x4_t w[CMP];
#pragma unroll
  for (int c = 0; c < CMP; ++c) {
    int o = (part * CMP + c) * 256 + b * 16;
    o = o < RB ? o : RB - 16;                  // past the row end: valid, masked below
    w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(prow + (uint32_t)o));
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt_gemv<CMP>();                      // phase 1 landed
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < XPT; ++t) {
    const int u = t * NT + tid;
    const int m = u / XU, uu = u - m * XU;
    // units past the end of x (or of its M rows) are stored as zeros: lanes
    // past a row's end then contribute exactly 0 without a mask
    const uint32_t z = m < M && uu < xunits ? 0xFFFFFFFFu : 0u;
    u32x4_t sp;
    sp.x = __builtin_amdgcn_perm(xv[t].z, xv[t].x, 0x05040100u) & z;
    sp.y = __builtin_amdgcn_perm(xv[t].z, xv[t].x, 0x07060302u) & z;
    sp.z = __builtin_amdgcn_perm(xv[t].w, xv[t].y, 0x05040100u) & z;
    sp.w = __builtin_amdgcn_perm(xv[t].w, xv[t].y, 0x07060302u) & z;
    *reinterpret_cast<u32x4_t*>(xsp + 4 * u) = sp;
  }
#pragma unroll
  for (int t = 0; t < SPT; ++t) {
    ssh[t * NT + tid] = (uint16_t)sv[t];
    if constexpr (AFF) zsh[t * NT + tid] = (uint8_t)zv[t];
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // Column c of lane (b, j): codes 512 c + 32 b of row j, x units 64 c + 4 b
  // .. +3 (LDS dwords 4 per unit), group (16 c + b) >> gsh (exactly
  // (16 c >> gsh) + (b >> gsh), since 16 c is a multiple of 2^gsh when
  // gsh < 4 and b < 16 adds nothing when gsh >= 4). Lanes whose slice lies
  // past the row end read x units past K, which are zero.
  const uint16_t* srow = ssh + (4 * wave + j) * G + (b >> gsh);
  const uint8_t* zrow = zsh + (AFF ? (4 * wave + j) * G + (b >> gsh) : 0);
  const uint32_t* xl = xsp + 16 * b + (MR > 1 ? j * XU * 4 : 0);   // x row j of A (row 0 if MR = 1)
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
  static_for<0, CMP>([&](auto C_) {
    constexpr int c = decltype(C_)::value;
    const int cg = part * CMP + c;             // column block in the row
    const float sc = half_bits_to_float(srow[(16 * cg) >> gsh]);
    const uint32_t zp = AFF ? (uint32_t)zrow[(16 * cg) >> gsh] : 0u;
    u32x4_t xa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const u32x4_t*>(xl + 256 * cg + 4 * i);
    wait_vmcnt_gemv<CMP - 1 - c>();
    float4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t hw[4];
      if constexpr (AFF) codes_to_half_spread_zp(w[c][i], hw, zp_bias_lo(zp), zp_bias_hi(zp));
      else codes_to_half_spread(w[c][i], hw);
      const half4_t b0 = __builtin_bit_cast(half4_t, u32x2v_t{__builtin_bit_cast(uint32_t, hw[0]), __builtin_bit_cast(uint32_t, hw[1])});
      const half4_t b1 = __builtin_bit_cast(half4_t, u32x2v_t{__builtin_bit_cast(uint32_t, hw[2]), __builtin_bit_cast(uint32_t, hw[3])});
      const half4_t a0 = __builtin_bit_cast(half4_t, u32x2v_t{xa[i].x, xa[i].y});
      const half4_t a1 = __builtin_bit_cast(half4_t, u32x2v_t{xa[i].z, xa[i].w});
      d = __builtin_amdgcn_mfma_f32_4x4x4f16(a0, b0, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_4x4x4f16(a1, b1, d, 0, 0, 0);
    }
    // register m of D: x row m (row 0 of the block's A when MR = 1)
    acc[0] += sc * d.x;
    if constexpr (MR > 1) {
      acc[1] += sc * d.y;
      acc[2] += sc * d.z;
      acc[3] += sc * d.w;
    }
  });
  // Sum the 16 slices (lanes 4b+j, b = 0..15) of each of the 4 rows.
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) acc[m] += __shfl_xor(acc[m], off);
  if constexpr (KSP > 1) {
    if (b == 0) {
#pragma unroll
      for (int m = 0; m < MR; ++m) part_sum[(part * ROWS + 4 * wave + j) * MR + m] = acc[m];
    }
    __syncthreads();
    if (part != 0) return;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      acc[m] = part_sum[(4 * wave + j) * MR + m];
#pragma unroll
      for (int p = 1; p < KSP; ++p) acc[m] += part_sum[(p * ROWS + 4 * wave + j) * MR + m];
    }
  }
  const int nrow = n0 + 4 * wave + j;
  if (b == 0 && nrow < N) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
      if (m < M) ep.store(y, (int64_t)m * N + nrow, acc[m], nrow);
  }
}

// ---------------------------------------------------------------------------
// Row-streaming variant for large matrices (packed weights >= 48 MB, K <=
// 16384): on those the launch is long enough for the read pattern to decide
// the rate, and reading 1 KB of one row per load beats the 4-row layout above.
//
// Each wavefront owns whole rows r0, r0 + TW, r0 + 2 TW, ... (TW = all
// wavefronts of the grid, at most 64 rows each). Lane l reads bytes
// 1024 c + 16 l of every chunk c of a row, and holds the matching 32
// activations of every chunk in registers (spread order, staged once per
// block through LDS, zero past K). The dot products use v_mfma_f32_4x4x4f16
// "on the diagonal": lane 4b+i supplies row i of block b's A (its own
// activations) and column i of its B (its own codes), so D_b[i][i] -- register
// i of lane 4b+i -- is the lane's own 4-code dot product, accumulated over its
// 32 codes; the other D entries are unused. The lane scales its partial by its
// group's scale (integer-first), the wavefront sums the 64 partials of a row
// (DPP butterfly + four lane reads), and lane k keeps the row's result until
// one store at the end. Two rows are in flight per wavefront: row k+2 is
// issued as soon as row k has been consumed, with exact load counts.
constexpr int kRowWaves = 8;                   // wavefronts per block

template <int C, bool AFF>
__global__ __launch_bounds__(64 * kRowWaves) void matmul_gemv_rows_kernel(
    const _Float16* __restrict__ x, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N, int K, int G,
    int group, void* __restrict__ y, Epilogue ep) {
  typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
  constexpr int P = 2;                         // rows in flight per wavefront
  constexpr int NT = 64 * kRowWaves;
  constexpr int XPT = (C * 256 + NT - 1) / NT; // 16-byte x units staged per thread
  constexpr int LPR = (AFF ? 3 : 2) * C;       // loads per row: C scales, (C zero points,) C weight chunks
  __shared__ __attribute__((aligned(16))) uint32_t xsp[XPT * NT * 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int RB = K >> 1;
  const int xunits = K >> 3;

  // Per lane and chunk: byte offset in a row (past the row end: the row's
  // last 16 bytes, multiplied by zero activations) and group index.
  int off[C], sidx[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int o = 1024 * c + 16 * lane;
    off[c] = o < RB - 16 ? o : RB - 16;
    const int gi = (2 * o) / group;
    sidx[c] = gi < G ? gi : G - 1;
  }
  const int TW = gridDim.x * kRowWaves;
  const int r0 = blockIdx.x * kRowWaves + wave;
  const int R = r0 < N ? (N - 1 - r0) / TW + 1 : 0;   // rows of this wavefront (<= 64)

  u32x4_t w[P][C];
  uint32_t sc[P][C], zc[P][C];
  // Loads of the wavefront's k-th row into slot `slot` (a constant at every
  // call); rows past the end read row N-1 and are not stored.
  auto issue = [&](int k, int slot) __attribute__((always_inline)) {
    const int r = r0 + k * TW < N ? r0 + k * TW : N - 1;
    const uint8_t* prow = packed + (int64_t)r * RB;
    const uint16_t* srow = scales + (int64_t)r * G;
#pragma unroll
    for (int c = 0; c < C; ++c) sc[slot][c] = srow[sidx[c]];
    if constexpr (AFF) {
      const uint8_t* zrow = zeros + (int64_t)r * G;
#pragma unroll
      for (int c = 0; c < C; ++c) zc[slot][c] = zrow[sidx[c]];
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
      w[slot][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(prow + (uint32_t)off[c]));
  };

  // x loads, then the first P rows, then stage x (the row loads stay in flight).
  u32x4_t xv[XPT];
#pragma unroll
  for (int t = 0; t < XPT; ++t) {
    const int u = t * NT + tid < xunits ? t * NT + tid : xunits - 1;
    xv[t] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(x) + 16u * (uint32_t)u);
  }
  __builtin_amdgcn_sched_barrier(0);
  static_for<0, P>([&](auto S) {
    issue(decltype(S)::value, decltype(S)::value);
    __builtin_amdgcn_sched_barrier(0);
  });
  wait_vmcnt_gemv<P * LPR>();                  // x landed
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < XPT; ++t) {
    const int u = t * NT + tid;
    const uint32_t z = u < xunits ? 0xFFFFFFFFu : 0u;
    u32x4_t sp;
    sp.x = __builtin_amdgcn_perm(xv[t].z, xv[t].x, 0x05040100u) & z;
    sp.y = __builtin_amdgcn_perm(xv[t].z, xv[t].x, 0x07060302u) & z;
    sp.z = __builtin_amdgcn_perm(xv[t].w, xv[t].y, 0x05040100u) & z;
    sp.w = __builtin_amdgcn_perm(xv[t].w, xv[t].y, 0x07060302u) & z;
    *reinterpret_cast<u32x4_t*>(xsp + 4 * u) = sp;
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  u32x4_t xa[C][4];                            // lane's activations: units 256 c + 4 l .. +3
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) xa[c][i] = *reinterpret_cast<const u32x4_t*>(xsp + 4 * (256 * c + 4 * lane + i));

  const int jsel = lane & 3;
  float yv = 0.0f;
  // At least one pass (a wavefront without rows computes a clamped row and
  // stores nothing): a guarded loop would let the compiler sink the first row
  // loads below the barrier into the guard.
  int k0 = 0;
  do {
    static_for<0, P>([&](auto S) __attribute__((always_inline)) {
      constexpr int sl = decltype(S)::value;
      const int k = k0 + sl;
      wait_vmcnt_gemv<(P - 1) * LPR>();        // row k landed
      __builtin_amdgcn_sched_barrier(0);
      float part = 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
        const uint32_t zlo = AFF ? zp_bias_lo(zc[sl][c]) : 0u, zhi = AFF ? zp_bias_hi(zc[sl][c]) : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          half2_t hw[4];
          if constexpr (AFF) codes_to_half_spread_zp(w[sl][c][i], hw, zlo, zhi);
          else codes_to_half_spread(w[sl][c][i], hw);
          const half4_t b0 = __builtin_bit_cast(half4_t, u32x2v_t{__builtin_bit_cast(uint32_t, hw[0]), __builtin_bit_cast(uint32_t, hw[1])});
          const half4_t b1 = __builtin_bit_cast(half4_t, u32x2v_t{__builtin_bit_cast(uint32_t, hw[2]), __builtin_bit_cast(uint32_t, hw[3])});
          const half4_t a0 = __builtin_bit_cast(half4_t, u32x2v_t{xa[c][i].x, xa[c][i].y});
          const half4_t a1 = __builtin_bit_cast(half4_t, u32x2v_t{xa[c][i].z, xa[c][i].w});
          d = __builtin_amdgcn_mfma_f32_4x4x4f16(a0, b0, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_4x4x4f16(a1, b1, d, 0, 0, 0);
        }
        // the lane's own dot product is register (lane & 3); selects, not branches
        const float d01 = (jsel & 1) ? d.y : d.x;
        const float d23 = (jsel & 1) ? d.w : d.z;
        part += half_bits_to_float((uint16_t)sc[sl][c]) * ((jsel & 2) ? d23 : d01);
      }
      const float tot = wave_sum(part);
      yv = lane == k ? tot : yv;
      __builtin_amdgcn_sched_barrier(0);
      issue(k + P, sl);
      __builtin_amdgcn_sched_barrier(0);
    });
    k0 += P;
  } while (k0 < R);
  wait_vmcnt_gemv<0>();
  if (lane < R) ep.store(y, r0 + lane * TW, yv, r0 + lane * TW);
}

const char* matmul_gemv_unsupported(int x_dtype, int64_t M, const void* x,
                                    const uint8_t* packed, int64_t N, int64_t K,
                                    int64_t group) {
  if (x_dtype != 1) return "gemv kernel takes binary16 activations only";
  if (M < 1 || M > 4) return "gemv kernel takes 1 <= M <= 4";
  if (M > 1 && (K > 12288 || group % 32 != 0 || ((group / 32) & (group / 32 - 1)) != 0))
    return "gemv kernel takes M = 2 .. 4 only with K <= 12288 and group = 32 * 2^p";
  if (group % 32 != 0) return "gemv kernel needs group to be a multiple of 32";
  if (K % 32 != 0) return "gemv kernel needs K to be a multiple of 32";
  if (K / 2 > 1024 * kGemvMaxChunks) return "gemv kernel takes K <= 32768";
  // (its widest grids launch up to 128 threads per weight row, and a
  // dispatch holds fewer than 2^32)
  if (N >= (1ll << 25)) return "gemv kernel needs N below 2^25";
  if ((uintptr_t)x % 16 || (uintptr_t)packed % 16) return "gemv kernel needs 16-byte aligned x and packed";
  return nullptr;
}

template <bool AFF>
static void launch_gemv_t(const _Float16* xh0, int64_t M, const uint8_t* packed, const uint16_t* scales,
                          const uint8_t* zeros, int64_t N, int64_t K, int64_t group, void* y,
                          Epilogue ep, hipStream_t stream) {
  const int G = (int)((K + group - 1) / group);
  int gsh = 0;                                                 // log2(group / 32), or -1
  while ((32ll << gsh) < group) ++gsh;
  if ((32ll << gsh) != group) gsh = -1;
  const int chunks = (int)((K / 2 + 1023) / 1024);            // 1 KB chunks per row
  const int cols = (int)((K / 2 + 255) / 256);                // 256-byte column blocks per row
  if (M > 1) {
    // M = 2 .. 4 (K <= 12288, group 32 << gsh): the matrix-core variant with
    // four x rows in A. Blocks of 4 groups of 4 rows (x, up to 96 KB of it in
    // LDS, is staged once for 16 rows), column blocks split over two
    // wavefronts for rows of 16 or more.
#define INT4DQ_GEMV_MFMA4(CMV)                                                                   \
  do {                                                                                          \
    constexpr int KS = CMV >= 16 ? 2 : 1, W = 4;                                                \
    const dim3 grid((unsigned)((N + 4 * W - 1) / (4 * W))), block(64 * W * KS);                \
    const auto kern = gsh == 0 ? matmul_gemv_mfma_kernel<CMV, 0, W, AFF, KS, 4>                 \
                    : gsh == 1 ? matmul_gemv_mfma_kernel<CMV, 1, W, AFF, KS, 4>                 \
                    : gsh == 2 ? matmul_gemv_mfma_kernel<CMV, 2, W, AFF, KS, 4>                 \
                               : matmul_gemv_mfma_kernel<CMV, 3, W, AFF, KS, 4>;                \
    hipLaunchKernelGGL(kern, grid, block, 0, stream, xh0, (int)M, packed, scales, zeros, (int)N, \
                       (int)K, G, (int)group, gsh, y, ep);                                      \
  } while (0)
    if (N <= 1024 && cols > 4 && cols <= 6) {
      // Small matrices (64 blocks of 16 rows or fewer) with rows of 5 or 6
      // column blocks: 4 rows per block, their columns split over 3
      // wavefronts, so that four times as many CUs stream the weights.
      // Measured (graph replays over a >= 1 GiB pool): [768, 3072] M = 4
      // 4.04 -> 3.62 us, M = 2 3.72 -> 3.29; [2048, 3072] M = 4 4.02 -> 4.43
      // (not taken there).
      const dim3 grid((unsigned)((N + 3) / 4)), block(64 * 3);
      const auto kern = gsh == 0 ? matmul_gemv_mfma_kernel<6, 0, 1, AFF, 3, 4>
                      : gsh == 1 ? matmul_gemv_mfma_kernel<6, 1, 1, AFF, 3, 4>
                      : gsh == 2 ? matmul_gemv_mfma_kernel<6, 2, 1, AFF, 3, 4>
                                 : matmul_gemv_mfma_kernel<6, 3, 1, AFF, 3, 4>;
      hipLaunchKernelGGL(kern, grid, block, 0, stream, xh0, (int)M, packed, scales, zeros, (int)N,
                         (int)K, G, (int)group, gsh, y, ep);
      return;
    }
    if (cols <= 2) INT4DQ_GEMV_MFMA4(2);
    else if (cols <= 4) INT4DQ_GEMV_MFMA4(4);
    else if (cols <= 6) INT4DQ_GEMV_MFMA4(6);
    else if (cols <= 8) INT4DQ_GEMV_MFMA4(8);
    else if (cols <= 12) INT4DQ_GEMV_MFMA4(12);
    else if (cols <= 16) INT4DQ_GEMV_MFMA4(16);
    else if (cols <= 22) INT4DQ_GEMV_MFMA4(22);
    else INT4DQ_GEMV_MFMA4(24);
#undef INT4DQ_GEMV_MFMA4
    return;
  }
  // (the AFF form with 8 chunks would exceed 256 VGPRs and spill: it takes the
  // variants below)
  if (N * (K / 2) >= (48ll << 20) && chunks <= (AFF ? 7 : 8)) {
    // Large matrix: row streaming. 256 blocks of 8 wavefronts (more if a
    // wavefront would own over 64 rows).
    int64_t blocks = 256;
    while ((N + blocks * kRowWaves - 1) / (blocks * kRowWaves) > 64) blocks *= 2;
    const dim3 grid((unsigned)blocks), block(64 * kRowWaves);
#define INT4DQ_GEMV_ROWS(CC)                                                                      \
  hipLaunchKernelGGL((matmul_gemv_rows_kernel<CC, AFF>), grid, block, 0, stream, xh0, packed,    \
                     scales, zeros, (int)N, (int)K, G, (int)group, y, ep)
    switch (chunks) {
      case 1: INT4DQ_GEMV_ROWS(1); break;
      case 2: INT4DQ_GEMV_ROWS(2); break;
      case 3: INT4DQ_GEMV_ROWS(3); break;
      case 4: INT4DQ_GEMV_ROWS(4); break;
      case 5: INT4DQ_GEMV_ROWS(5); break;
      case 6: INT4DQ_GEMV_ROWS(6); break;
      case 7: INT4DQ_GEMV_ROWS(7); break;
      default:
        if constexpr (!AFF) INT4DQ_GEMV_ROWS(8);
        break;
    }
#undef INT4DQ_GEMV_ROWS
    return;
  }
  if (gsh >= 0 && g_gemv_mfma && cols > 4 && cols <= 12 && (N <= 1024 || (N <= 2048 && cols > 8))) {
    // Small matrices (64 blocks of 16 rows or fewer; 128 for rows of 9-12
    // column blocks) with rows of 5 to 12 column blocks: 4 rows per block,
    // their columns split over 3 (rows of 6) or 4 wavefronts, so that four
    // times as many CUs stream the weights. Measured (graph replays over a
    // >= 1 GiB pool), against 4 wavefronts of whole rows: [768, 3072] 3.26 ->
    // 2.79 us, [512, 3072] 3.15 -> 2.76, [768, 4096] 3.37 -> 2.86, [1024, 6144]
    // 4.37 -> 3.22, [2048, 6144] 4.59 -> 4.00; [4096, 3072] 3.60 -> 4.05 (not
    // taken there); rows of 2 column blocks gained nothing.
#define INT4DQ_GEMV_SPLITCOL(CMV, KSV)                                                            \
  do {                                                                                          \
    const dim3 grid((unsigned)((N + 3) / 4)), block(64 * KSV);                                  \
    const auto kern = gsh == 0 ? matmul_gemv_mfma_kernel<CMV, 0, 1, AFF, KSV>                   \
                    : gsh == 1 ? matmul_gemv_mfma_kernel<CMV, 1, 1, AFF, KSV>                   \
                    : gsh == 2 ? matmul_gemv_mfma_kernel<CMV, 2, 1, AFF, KSV>                   \
                               : matmul_gemv_mfma_kernel<CMV, 3, 1, AFF, KSV>;                  \
    hipLaunchKernelGGL(kern, grid, block, 0, stream, xh0, 1, packed, scales, zeros, (int)N,     \
                       (int)K, G, (int)group, gsh, y, ep);                                      \
  } while (0)
    if (cols <= 6) INT4DQ_GEMV_SPLITCOL(6, 3);
    else if (cols <= 8) INT4DQ_GEMV_SPLITCOL(8, 4);
    else INT4DQ_GEMV_SPLITCOL(12, 4);
#undef INT4DQ_GEMV_SPLITCOL
    return;
  }
  if (cols <= 24 && gsh >= 0 && g_gemv_mfma) {
    // Rows of 16 or more column blocks (K >= 7680) split each row's columns
    // over two wavefronts (blocks of 2 x 2 wavefronts, 8 rows): their chains
    // of expansions and MFMAs after the loads land are half as long. Measured
    // (1 GiB rotation pool): [4096,8192] 6.41 -> 5.65 us, [4096,11008] 7.91 ->
    // 6.98 us; rows of 12 column blocks or fewer were slower split ([4096,6144]
    // 4.65 -> 4.94 us), so they keep 4 wavefronts of whole rows per block.
#define INT4DQ_GEMV_MFMA(CMV)                                                                    \
  do {                                                                                          \
    constexpr int KS = CMV >= 16 ? 2 : 1, W = CMV >= 16 ? 2 : g_gemv_waves;                     \
    const dim3 grid((unsigned)((N + 4 * W - 1) / (4 * W))), block(64 * W * KS);                \
    const auto kern = gsh == 0 ? matmul_gemv_mfma_kernel<CMV, 0, W, AFF, KS>                    \
                    : gsh == 1 ? matmul_gemv_mfma_kernel<CMV, 1, W, AFF, KS>                    \
                    : gsh == 2 ? matmul_gemv_mfma_kernel<CMV, 2, W, AFF, KS>                    \
                               : matmul_gemv_mfma_kernel<CMV, 3, W, AFF, KS>;                   \
    hipLaunchKernelGGL(kern, grid, block, 0, stream, xh0, 1, packed, scales, zeros, (int)N,     \
                       (int)K, G, (int)group, gsh, y, ep);                                      \
  } while (0)
    if (cols <= 2) INT4DQ_GEMV_MFMA(2);
    else if (cols <= 4) INT4DQ_GEMV_MFMA(4);
    else if (cols <= 6) INT4DQ_GEMV_MFMA(6);
    else if (cols <= 8) INT4DQ_GEMV_MFMA(8);
    else if (cols <= 12) INT4DQ_GEMV_MFMA(12);
    else if (cols <= 16) INT4DQ_GEMV_MFMA(16);
    else if (cols <= 22) INT4DQ_GEMV_MFMA(22);
    else INT4DQ_GEMV_MFMA(24);
#undef INT4DQ_GEMV_MFMA
    return;
  }
  // Rows per block: enough wavefronts in flight (about 4096) to keep every
  // memory channel busy, up to 4 rows per wavefront.
  const int64_t want = (int64_t)chunks * N / 4096;
  const int rw = want >= 8 ? 8 : want >= 4 ? 4 : want >= 2 ? 2 : 1;
  const int64_t blocks = (N + rw - 1) / rw;
  const dim3 grid((unsigned)blocks), block(64 * chunks);
  const auto kern = rw == 8 ? matmul_gemv_kernel<8, AFF> : rw == 4 ? matmul_gemv_kernel<4, AFF>
                  : rw == 2 ? matmul_gemv_kernel<2, AFF> : matmul_gemv_kernel<1, AFF>;
  hipLaunchKernelGGL(kern, grid, block, 0, stream, xh0, packed, scales, zeros, (int)N, (int)K, G,
                     (int)group, gsh, y, ep);
}

hipError_t launch_matmul_gemv(const void* x, int64_t M, const uint8_t* packed, const uint16_t* scales,
                              const uint8_t* zeros, int64_t N, int64_t K, int64_t group, void* y,
                              Epilogue ep, hipStream_t stream) {
  const _Float16* xh = static_cast<const _Float16*>(x);
  if (zeros) launch_gemv_t<true>(xh, M, packed, scales, zeros, N, K, group, y, ep, stream);
  else launch_gemv_t<false>(xh, M, packed, scales, zeros, N, K, group, y, ep, stream);
  return hipGetLastError();
}

}  // namespace int4dq
