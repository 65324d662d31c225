// matmul_tiled.hip -- dequantizing matmul for many activation rows (binary16
// x) on gfx950: an MFMA kernel bound by matrix-core throughput.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, int4_matmul): y = x @ dequantize(W).T,
// one group at a time -- x times the group's integer codes first, then the
// group's scale on each output column. Full-precision weights never reach
// memory ("Build a Blockwise INT4 Inference Engine", architecture overview:
// the fusion boundary); here they exist only as exact fp16 integer codes in
// LDS, one sub-step at a time.
//
// Block tile 256 (rows of x) x 128 (weight rows), 512 threads = 4 x 2
// wavefronts (two per SIMD), each owning 64 x 64 outputs as 2 x 2 tiles of
// v_mfma_f32_32x32x16_f16 (fp32 accumulation in VGPRs). K advances in
// sub-steps of BK = min(group, 64) codes:
//  * x tiles [256 x BK] fp16 go global -> LDS by DMA (global_load_lds, 16 B
//    per lane, no VGPRs) into a 4-stage ring, three sub-steps ahead.
//  * The block's packed weights [128 x BK/2 bytes] are loaded to registers
//    four sub-steps ahead; one sub-step ahead each thread expands its words
//    to exact fp16 codes (codes_to_half_natural) into a 2-stage LDS ring, so
//    each code is expanded once per block, not once per wave.
//  * Both LDS tiles use rows of BK halves made of 16-byte pieces; logical
//    piece c of row r is stored at c ^ ((r / (16 / pieces)) % pieces). The 16
//    rows one pass of an MFMA operand read touches then cover all 64 banks;
//    each expansion store writes 1 KB contiguously (conflict-free for
//    ds_write_b128, which the row pattern is not).
//  * The k order inside a sub-step is a fixed permutation shared by A and B
//    (lane half h, k-step s: piece (BK / 16) h + s), which leaves the dot
//    product unchanged.
//  * Integer-first scaling with one accumulator set: the accumulator holds
//    (sum of finished groups' scaled partials) / (scale of the current group);
//    at each group boundary it is multiplied by s_prev / s_new for its column,
//    the group's integer products are accumulated by the MFMAs, and the final
//    value is multiplied by the last scale. A zero scale (a group of zero
//    codes) leaves the running scale unchanged. Mathematically this is
//    sum_g s_g * (x . q_g); the ratio multiply adds one fp32 rounding per group.
//    Which sub-steps open a group is a template parameter, so every sub-step is
//    one branch-free block.
//  * Each sub-step waits for exactly the group of loads issued D sub-steps
//    earlier (counts known at compile time), then one LDS-only barrier.
#include "device_common.h"
#include "kernels.h"

#include <type_traits>

namespace int4dq {

namespace {
typedef float float16_t __attribute__((ext_vector_type(16)));

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace

// Tile configuration: block tile BM x BN, WM x WN wavefronts (each owning a
// (BM/WM) x (BN/WN) tile of 32x32 MFMA tiles), BK codes per sub-step, NXS
// stages in the x ring (2 or 4; loads run NXS-1 sub-steps ahead), SPG
// sub-steps per group (1, 2 or 4, dividing NXS or equal to it), or 0: any
// power of two 2^gshift, decided at run time.
template <int BM, int BN, int WM, int WN, int BK, int NXS, int SPG>
__global__ __launch_bounds__(64 * WM * WN) void matmul_tiled_kernel(
    const _Float16* __restrict__ x, int M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, int N, int K, int G, int gshift,
    float* __restrict__ y) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int WMT = BM / WM, WNT = BN / WN;  // wave tile
  constexpr int TM = WMT / 32, TN = WNT / 32;  // 32x32 MFMA tiles per wave
  constexpr int KS = BK / 16;                  // MFMA k-steps per sub-step
  constexpr int PIECES = BK / 8;               // 16-byte pieces per row per sub-step
  constexpr int RPB = 16 / PIECES;             // rows per 256-byte LDS bank period
  constexpr int A_HALVES = BM * BK;            // one x stage
  constexpr int B_HALVES = BN * BK;            // one expanded-weight stage
  constexpr int XDMA = BM * PIECES / (64 * NW);// x DMA instructions per wave per stage
  constexpr int RPI = 64 / PIECES;             // rows per DMA instruction
  constexpr int WPT = BN * BK / 8 / NT;        // packed 32-bit words per thread per sub-step
  constexpr int D = NXS - 1;                   // x / scale prefetch distance (sub-steps)
  constexpr int U = NXS;                       // sub-steps per unrolled loop body
  static_assert(NXS == 2 || NXS == 4, "x ring depth");
  static_assert(SPG == 0 || (U % SPG == 0), "sub-steps per group");
  static_assert(XDMA >= 1 && BM * PIECES % (64 * NW) == 0, "x DMA split");
  static_assert(WPT >= 1 && BN * BK / 8 == WPT * NT, "weight words per thread");
  static_assert(WMT % 32 == 0 && WNT % 32 == 0, "wave tile");
  // Sub-step t issues one group of loads: x(t+D) (XDMA), w(t+D+1) (WPT) and,
  // when sub-step t+D opens a group, s(t+D) (TN). Sizes by t % U.
  constexpr auto s_used = [](int j) { return SPG == 0 || ((j + D) % U) % SPG == 0; };
  constexpr auto group_loads = [s_used](int j) {
    return XDMA + WPT + (s_used(((j % U) + U) % U) ? TN : 0);
  };
  // Loads pending that are newer than the group sub-step t needs: the groups of
  // sub-steps t-D+1 .. t-1 (main loop), or those issued before the tail.
  constexpr auto newer_loads = [group_loads](int j, bool tail) {
    int n = 0;
    if (!tail) {
      for (int i = 1; i < D; ++i) n += group_loads(j - i);
    } else {
      for (int i = 1; i <= D - 1 - j; ++i) n += group_loads(U - i);
    }
    return n;
  };

  // One array for both rings: with x stages and B stages at offsets the
  // compiler can tell apart, it does not wait for the x DMA before every read.
  __shared__ __attribute__((aligned(1024))) _Float16 lds[NXS * A_HALVES + 2 * B_HALVES];
  _Float16* const as = lds;
  _Float16* const bs = lds + NXS * A_HALVES;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int c32 = lane & 31, h = lane >> 5;

  // Tile assignment: consecutive block ids walk down the M tiles first. The
  // hardware deals block ids round-robin to the 8 XCDs, so with a multiple of
  // 8 M tiles each XCD keeps its x row-tiles in its own L2.
  const int mtiles = (M + BM - 1) / BM;
  const int bm = blockIdx.x % mtiles, bn = blockIdx.x / mtiles;
  const int m0 = bm * BM, n0 = bn * BN;

  auto swz = [](int r, int c) { return c ^ ((r / RPB) & (PIECES - 1)); };

  // --- x: DMA, wave instruction i writes 1 KB: rows xr0 + i*RPI, physical piece lane%PIECES.
  // Byte offsets from the tile's first row fit 32 bits (BM <= 256 rows, K < 2^23).
  const int xr0 = wave * XDMA * RPI + lane / PIECES;
  const char* xtile = reinterpret_cast<const char*>(x + (int64_t)m0 * K);
  uint32_t xoff[XDMA];
#pragma unroll
  for (int i = 0; i < XDMA; ++i) {
    const int r = xr0 + i * RPI;
    const int rr = m0 + r < M ? r : M - 1 - m0;                // rows past M: read row M-1, discarded
    xoff[i] = 2u * ((uint32_t)rr * (uint32_t)K + 8u * (uint32_t)swz(r, lane % PIECES));
  }

  // --- weights: write i of a wave stores 1 KB of the B stage contiguously
  // (piece P = (wave*WPT + i)*64 + lane, row P / PIECES, physical piece
  // P % PIECES): ds_write_b128 has no bank conflicts on contiguous addresses.
  // The thread loads the packed word of that row's logical piece.
  const uint8_t* wsrc[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int P = (wave * WPT + i) * 64 + lane;
    const int row = P / PIECES, c = swz(row, P % PIECES);
    int n = n0 + row;
    n = n < N ? n : N - 1;                                     // tail rows: read, discarded
    wsrc[i] = packed + (int64_t)n * (K >> 1) + 4 * c;
  }
  // scales of the lane's output columns
  const uint16_t* ssrc[TN];
#pragma unroll
  for (int b = 0; b < TN; ++b) {
    int n = n0 + wn * WNT + b * 32 + c32;
    n = n < N ? n : N - 1;
    ssrc[b] = scales + (int64_t)n * G;
  }
  const int T = K / BK;
  const int spg_log = SPG == 0 ? gshift : SPG == 4 ? 2 : SPG == 2 ? 1 : 0;
  uint32_t wr[NXS][WPT];                                       // w(t) in slot t % NXS
  uint32_t sr[NXS][TN];                                        // s(t) in slot t % NXS

  // Loads of sub-step t's operands (an index past the end is clamped to the
  // last sub-step; such data is never used).
  auto load_w = [&](int t, int slot) {
    const int tc = t < T ? t : T - 1;
#pragma unroll
    for (int i = 0; i < WPT; ++i)
      wr[slot][i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(wsrc[i] + tc * (BK / 2)));
  };
  auto load_sx = [&](int t, int slot, bool with_s) {
    const int tc = t < T ? t : T - 1;
    if (with_s) {
      // Sub-steps of one group load the same scales; the opaque index keeps
      // the compiler from merging such loads, which would change the load
      // counts the waits rely on.
      int gi = tc >> spg_log;
      asm volatile("" : "+s"(gi));
#pragma unroll
      for (int b = 0; b < TN; ++b) sr[slot][b] = ssrc[b][gi];
    }
    const char* base = xtile + (int64_t)tc * (2 * BK);
#pragma unroll
    for (int i = 0; i < XDMA; ++i)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(base + xoff[i]),
          reinterpret_cast<void*>(as + slot * A_HALVES + (wave * XDMA + i) * 512), 16, 0, 0);
  };
  auto expand = [&](int slot, int bstage) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      half2_t hw[4];
      codes_to_half_natural(wr[slot][i], hw);
      *reinterpret_cast<half8_t*>(bs + bstage * B_HALVES + ((wave * WPT + i) * 64 + lane) * 8) = as_half8(hw);
    }
  };

  float16_t acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  float srun[TN];
#pragma unroll
  for (int b = 0; b < TN; ++b) srun[b] = 0.0f;

  // Operand LDS offsets (halves) for k-step s; m-tile a adds a*32 rows, n-tile b
  // adds b*32 rows (whole swizzle periods, so the piece is unchanged).
  int aoff[KS], boff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int c = (BK / 16) * h + s;
    const int ra = wm * WMT + c32, rb = wn * WNT + c32;
    aoff[s] = ra * BK + 8 * swz(ra, c);
    boff[s] = rb * BK + 8 * swz(rb, c);
  }

  // The loads of one group may be issued in any order. Sub-step t needs s(t),
  // x(t) and w(t+1) -- exactly the group that sub-step t-D issued -- so it
  // waits until only the newer groups are pending. x(t+D) goes to the stage
  // sub-step t-1 read, w(t+D+1) to the slot of w(t), which sub-step t-1
  // expanded. Every load issued is used, so none is dropped by the compiler.
  // Prologue: w0, then the groups of sub-steps -D .. -1, then expand w0
  // (scheduling barriers keep the groups apart, as the waits assume).
  load_w(0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < D; ++g) {
    load_sx(g, g, s_used(g + U - D));
    load_w(g + 1, g + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  constexpr auto prologue_loads = [group_loads]() {
    int n = 0;
    for (int g = 0; g < D; ++g) n += group_loads(g - D);
    return n;
  };
  wait_vmcnt<prologue_loads()>();                              // w(0)
  __builtin_amdgcn_sched_barrier(0);
  expand(0, 0);

  // Sub-step t = t0 + j with t0 a multiple of U: x stage, scale slot and
  // weight slot j, B stage j % 2, all compile-time. In the tail (after the
  // last whole block of U) no loads are issued.
  auto substep = [&](auto J, auto Tail, int t) {
    constexpr int j = decltype(J)::value;
    constexpr bool tail = decltype(Tail)::value;
    constexpr int p = j & 1;
    wait_vmcnt<newer_loads(j, tail)>();                        // group of t-D landed
    lds_barrier();                                             // x(t), B(t) visible; stages of t-1 free
    // Keep every use of the awaited registers below the wait: a use hoisted
    // above it makes the compiler add a wait of its own, and with LDS DMA in
    // flight that wait is for every load.
    __builtin_amdgcn_sched_barrier(0);
    bool gstart;
    if constexpr (SPG == 0) gstart = (t & ((1 << gshift) - 1)) == 0;
    else gstart = j % SPG == 0;
    float ratio[TN];
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const float sn = half_bits_to_float((uint16_t)sr[j][b]);
      const bool live = gstart && sn != 0.0f;                  // zero scale: keep the running one
      // srun / sn to within an ulp (a uniform relative error of the finished
      // groups' part, far inside the tolerance); srun = 0 gives 0.
      ratio[b] = live ? srun[b] * __builtin_amdgcn_rcpf(sn) : 1.0f;
      srun[b] = live ? sn : srun[b];
    }
    expand((j + 1) % U, p ^ 1);                                // w(t+1) -> B stage of t+1
    if constexpr (!tail) {
      load_sx(t + D, (j + D) % U, s_used(j));
      load_w(t + D + 1, j);
    }
    const _Float16* sa = as + j * A_HALVES;
    const _Float16* sb = bs + p * B_HALVES;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      half8_t af[TM], bf[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a) af[a] = *reinterpret_cast<const half8_t*>(sa + aoff[s] + a * 32 * BK);
#pragma unroll
      for (int b = 0; b < TN; ++b) bf[b] = *reinterpret_cast<const half8_t*>(sb + boff[s] + b * 32 * BK);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          if (s == 0 && (SPG == 0 || gstart)) acc[a][b] *= ratio[b];
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
        }
    }
  };

  using body = std::false_type;
  using tail = std::true_type;
  int t0 = 0;
  for (; t0 + U <= T; t0 += U) {
    substep(std::integral_constant<int, 0>(), body(), t0);
    substep(std::integral_constant<int, 1>(), body(), t0 + 1);
    if constexpr (U == 4) {
      substep(std::integral_constant<int, 2>(), body(), t0 + 2);
      substep(std::integral_constant<int, 3>(), body(), t0 + 3);
    }
  }
  if (t0 < T) substep(std::integral_constant<int, 0>(), tail(), t0);
  if constexpr (U == 4) {
    if (t0 + 1 < T) substep(std::integral_constant<int, 1>(), tail(), t0 + 1);
    if (t0 + 2 < T) substep(std::integral_constant<int, 2>(), tail(), t0 + 2);
  }
  wait_vmcnt<0>();                                             // no LDS DMA in flight at exit

  // Epilogue: apply the last running scale; lane l holds column l%32 and rows
  // 8*(i/4) + 4*(l/32) + (i%4) of each 32x32 tile (register i).
#pragma unroll
  for (int b = 0; b < TN; ++b) {
    const int n = n0 + wn * WNT + b * 32 + c32;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * WMT + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (m < M && n < N) y[(int64_t)m * N + n] = acc[a][b][i] * srun[b];
      }
  }
}

// Launch one tiled configuration for group = BK << gs. Sub-steps per group
// are a template parameter when they divide the unroll (NXS), else read at
// run time.
#define INT4DQ_TILED_LAUNCH(BM, BN, WM, WN, BK, NXS)                                          \
  do {                                                                                        \
    int gs = 0;                                                                               \
    while ((int64_t(BK) << gs) < group) ++gs;                                                 \
    auto kernel = matmul_tiled_kernel<BM, BN, WM, WN, BK, NXS, 0>;                            \
    if (gs == 0) kernel = matmul_tiled_kernel<BM, BN, WM, WN, BK, NXS, 1>;                    \
    else if (gs == 1) kernel = matmul_tiled_kernel<BM, BN, WM, WN, BK, NXS, 2>;               \
    else if (gs == 2 && NXS == 4) kernel = matmul_tiled_kernel<BM, BN, WM, WN, BK, NXS, (NXS == 4 ? 4 : 0)>; \
    const int64_t blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);                         \
    if (blocks >= (1ll << 31)) return hipErrorInvalidValue;                                   \
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(64 * WM * WN), 0, stream, xh,      \
                       (int)M, packed, scales, (int)N, (int)K, G, gs, y);                     \
  } while (0)

// BK for a group size, or 0 if the kernel does not take it (group / BK must be
// a power of two: the group index of a sub-step is a shift).
static int tiled_bk(int64_t group) {
  if (group == 32) return 32;
  if (group % 64 == 0 && ((group / 64) & (group / 64 - 1)) == 0) return 64;
  return 0;
}

const char* matmul_tiled_unsupported(int x_dtype, const void* x, const uint8_t* packed,
                                     int64_t K, int64_t group) {
  if (x_dtype != 1) return "tiled kernel takes binary16 activations only";
  const int BK = tiled_bk(group);
  if (BK == 0) return "tiled kernel takes group 32 or 64 times a power of two";
  if (K % BK != 0) return "tiled kernel needs K to be a multiple of min(group, 64)";
  if (K >= (1ll << 23)) return "tiled kernel needs K below 2^23";
  if ((uintptr_t)x % 16 || (uintptr_t)packed % 16) return "tiled kernel needs 16-byte aligned x and packed";
  return nullptr;
}

hipError_t launch_matmul_tiled(const void* x, int64_t M, const uint8_t* packed,
                               const uint16_t* scales, int64_t N, int64_t K, int64_t group,
                               float* y, hipStream_t stream) {
  const int BK = tiled_bk(group);
  const int G = (int)((K + group - 1) / group);
  if (M >= (1ll << 31) || N >= (1ll << 31)) return hipErrorInvalidValue;
  const _Float16* xh = static_cast<const _Float16*>(x);
  if (BK == 32) INT4DQ_TILED_LAUNCH(256, 128, 4, 2, 32, 4);
  else INT4DQ_TILED_LAUNCH(256, 128, 4, 2, 64, 4);
  return hipGetLastError();
}

}  // namespace int4dq
