// matmul_tiled.hip -- dequantizing matmul for many activation rows (binary16
// x) on gfx950: an MFMA kernel bound by matrix-core throughput.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, int4_matmul): y = x @ dequantize(W).T
// with dequantize(W) = q * scale per group. Full-precision weights never reach
// memory ("Build a Blockwise INT4 Inference Engine", architecture overview:
// the fusion boundary); here they exist only in registers, one MFMA k-step at
// a time, as binary16 products q * scale of the exact integer codes and their
// group's scale (one rounding each, at most 2^-11 relative).
//
// Block tile 128 (rows of x) x 256 (weight rows), 256 threads = 4 wavefronts
// side by side along N, one per SIMD, each owning 128 x 64 outputs as 4 x 2
// tiles of v_mfma_f32_32x32x16_f16 (fp32 accumulation in 128 AGPRs). The
// global -> LDS bytes per sub-step are 16 KB of x and 8 KB of packed weights
// (a 256 x 128 tile moves 32 KB + 4 KB for the same flops). For fewer rows of
// x the block is 128 x 128, 64 x 128 or 32 x 128 with wave tiles one MFMA
// tile wide (4, 2 or 1 tiles of 32 rows), so that the grid still covers the
// CUs and every code is expanded once per block. Wave tiles larger than
// 64 x 64 halve the LDS bytes read per MFMA.
// K advances in sub-steps of BK = min(group, 64) codes:
//  * x tiles [BM x BK] fp16 go global -> LDS by DMA (global_load_lds, 16 B
//    per lane, no VGPRs) into a 4-stage ring, three sub-steps ahead.
//  * Packed weights go global -> LDS by DMA too, in "super-tiles" of 128 B
//    (256 codes) of each of the block's weight rows: eight lanes cover a full
//    128-byte line, and a 2-slot ring loads super-tile j+1 while j is used.
//  * Each wavefront reads its own packed words (one 16-byte read per 32-column
//    tile per sub-step), expands them to exact fp16 codes in registers
//    (codes_to_half_natural) and multiplies each pair by its group's scale
//    (one packed fp16 multiply) right before the MFMAs that use them.
//  * The k order inside a sub-step is a fixed permutation shared by A and B
//    (lane half h, k-step s: codes (BK/2) h + 8 s .. +7), so each lane's
//    packed bytes for a sub-step are contiguous and the dot product is
//    unchanged.
//  * LDS rows are made of 16-byte pieces; logical piece c of row r is stored
//    at c ^ f(r), which makes every 16-lane pass of an operand read cover all
//    64 banks. DMA writes stay contiguous (the swizzle is applied to the
//    global source address).
//  * Sub-step t's A fragments for k-step 0 and its packed words are read at
//    the end of sub-step t-1, so the MFMA pipe does not wait for LDS after the
//    barrier; the barrier of sub-step t therefore makes the data of t+1
//    visible (it waits for the loads issued two sub-steps earlier).
//  * The scale enters with the codes, so the accumulators are never read or
//    rescaled inside the loop (they stay in AGPRs); a group boundary only
//    switches the scale word of each column. A scale too large for the
//    binary16 product (above 8188) sends the block through two more passes
//    with the exponent shifted, described at the passes below.
//  * Each sub-step waits for exactly the loads issued two sub-steps earlier
//    (counts known at compile time; the loop is unrolled over two super-tiles
//    so every stage and slot index is a constant), then one LDS-only barrier.
//    Scheduling groups interleave LDS reads, code expansion and MFMAs.
//  * Affine codes ("Build a Blockwise INT4 Inference Engine", step 2; the AFF
//    form): each group's zero point is loaded with its scale, and its bias
//    word (codes_to_half_natural_zp) is switched at the group boundary
//    together with the scale, so the codes expand to u - zp exactly before
//    the multiply.
#include "device_common.h"
#include "kernels.h"

#include <algorithm>
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

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    unroll<B + 1, E>(f);
  }
}

constexpr int kThreads = 256;
}  // namespace

// BK: codes per sub-step (32 or 64). SPG: sub-steps per group (1, 2, 4 or 8),
// or 0: any power of two 2^gshift, decided at run time. TM, TN: 32 x 32 MFMA
// tiles per wavefront in M and N. WN: wavefronts side by side along N (4, or
// 2 for 2 x 2 wavefronts). Block tile (32 TM * 4 / WN) x (32 TN * WN). The
// launcher uses WN = 4 with (TM, TN) = (4, 2), (4, 1), (2, 1) and (1, 1).
template <int BK, int SPG, int TM, bool AFF, int WN, int TN, int NXS_ = 4, int WS_ = 2>
__global__ __launch_bounds__(kThreads) void matmul_tiled_kernel(
    const _Float16* __restrict__ x, int M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N, int K, int G,
    int gshift, void* __restrict__ y, Epilogue ep, TiledSplit sp) {
  constexpr int WMT = 32 * TM, WNT = 32 * TN;         // wave tile; TM x TN 32x32 MFMA tiles
  constexpr int NW = 4, BM = WMT * (NW / WN), BN = WNT * WN;
  static_assert(WN == 2 || WN == 4, "wave layout");
  static_assert(TN == 1 || TN == 2, "wave tile columns");
  constexpr int KS = BK / 16;                  // MFMA k-steps per sub-step
  constexpr int PIECES = BK / 8;               // 16-byte pieces per x row per stage
  constexpr int RPB = 16 / PIECES;             // x rows per 256-byte bank period
  // x ring stages and prefetch distance; packed super-tile slots. (Deeper
  // rings for the small tiles -- 8 stages, 4 slots -- measured no faster: with
  // 64-row tiles a block is bound by its own instruction stream, not latency.)
  constexpr int NXS = NXS_, D = NXS - 1;
  constexpr int WS = WS_;
  constexpr int A_BYTES = BM * BK * 2;         // one x stage
  constexpr int XDMA = BM * PIECES / (64 * NW);// x DMA instructions per wave per sub-step
  constexpr int RPI = 64 / PIECES;             // x rows per DMA instruction
  constexpr int SUB = 256 / BK;                // sub-steps per packed super-tile
  constexpr int U = WS * SUB;                  // sub-steps per unrolled body
  constexpr int W_BYTES = BN * 128;            // one packed super-tile
  constexpr int WDMA = W_BYTES / 1024 / NW;    // W DMA instructions per wave per super-tile
  static_assert(BK == 32 || BK == 64, "sub-step");
  static_assert(TM == 1 || TM == 2 || TM == 4, "wave tile");
  static_assert(XDMA >= 1 && XDMA * 64 * NW == BM * PIECES, "x DMA split");
  static_assert(SPG == 0 || U % SPG == 0, "sub-steps per group");
  static_assert(NXS * A_BYTES + WS * W_BYTES <= 160 * 1024, "LDS");
  static_assert(U % NXS == 0 && SUB * (WS - 1) >= D && D % SUB != 0, "ring indices and weight lead");
  // Sub-step t issues x(t+D), s(t+D) when t+D opens a group (every sub-step
  // when SPG is decided at run time), and super-tile t/SUB + WS - 1 when t is
  // the first sub-step of a super-tile. Sizes by position in the unrolled body.
  constexpr auto s_used = [](int j) { return SPG == 0 || (((j % U) + U) % U) % SPG == 0; };
  constexpr auto group_loads = [s_used](int j) {
    const int jj = ((j % U) + U) % U;
    return XDMA + (s_used(jj + D) ? (AFF ? 2 : 1) * TN : 0) + (jj % SUB == 0 ? WDMA : 0);
  };
  // Sub-step t needs x(t+1) and s(t+1) (loaded by the group of t+1-D; the
  // super-tile of t+1 was loaded earlier still): the groups of t+2-D .. t-1 may
  // still be in flight.
  constexpr auto newer_loads = [group_loads](int j) {
    int n = 0;
    for (int i = 0; i <= D - 2; ++i) n += group_loads(j - i);
    return n;
  };

  // One array for both rings: with stages and slots at constant offsets the
  // compiler can tell the DMA targets from the regions being read. Every LDS
  // address is written as an offset from the array itself (not from a pointer
  // variable into it), which keeps the DMA destinations scalar.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NXS * A_BYTES + WS * W_BYTES];
  constexpr int W_LDS = NXS * A_BYTES;         // offset of the packed-weight slots

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int c32 = lane & 31, h = lane >> 5;

  // Tile assignment: consecutive block ids walk down the M tiles first. With a
  // split of K (sp.S > 1) block id / tiles is the block's share of K:
  // sub-steps [split * sp.steps, +sp.steps), which start on a packed
  // super-tile and on a group boundary. The hardware deals block ids
  // round-robin to the 8 XCDs; without a split, and when the grid allows it,
  // the order below gives each XCD a compact rectangle of tiles instead.
  const int mtiles = (M + BM - 1) / BM, ntiles = (N + BN - 1) / BN;
  const int tiles = mtiles * ntiles;
  const int tile = blockIdx.x % tiles, split = blockIdx.x / tiles;
  int bm = tile % mtiles, bn = tile / mtiles;
  if (sp.S == 1 && tiles % 8 == 0 && mtiles % 4 == 0) {
    // XCD rectangles: XCD x takes tiles x T/8 .. (x+1) T/8 - 1 of an order
    // that walks bands of 4 tile rows column by column, so the 32 blocks an
    // XCD runs at a time cover about 4 x 8 tiles and its L2 sees 4 x row
    // tiles and 8 weight column tiles, not 2 and 16. Measured at M = 2048 on
    // the 7B-class shapes: 15-21% fewer bytes fetched past the L2s, the same
    // time per launch.
    const int t = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
    const int band = t / (4 * ntiles), q = t % (4 * ntiles);
    bm = 4 * band + (q & 3);
    bn = q >> 2;
  }
  const int m0 = bm * BM, n0 = bn * BN;
  const int t_begin = split * sp.steps;        // first sub-step of the block's share of K
  const int T = min(K / BK - t_begin, sp.steps);   // sub-steps of the share
  const int RB = K >> 1;                       // bytes per packed row
  const int RBl = RB - t_begin * (BK / 2);     // bytes of a row from the share's start

  auto swz = [](int r, int c) { return c ^ ((r / RPB) & (PIECES - 1)); };

  // --- x DMA: wave instruction i writes 1 KB: rows xr0 + i*RPI, physical
  // piece lane % PIECES. Byte offsets from the tile's first row fit 32 bits
  // (BM rows, K < 2^23). Rows past M read row M-1 (discarded).
  const int xr0 = wave * XDMA * RPI + lane / PIECES;
  const char* xtile = reinterpret_cast<const char*>(x + (int64_t)m0 * K + (int64_t)t_begin * BK);
  uint32_t xoff[XDMA];
#pragma unroll
  for (int i = 0; i < XDMA; ++i) {
    const int r = xr0 + i * RPI;
    const int rr = m0 + r < M ? r : M - 1 - m0;
    xoff[i] = 2u * ((uint32_t)rr * (uint32_t)K + 8u * (uint32_t)swz(r, lane % PIECES));
  }
  // --- W DMA: chunk c = wave*WDMA + i holds block rows 8c .. 8c+7 (128 B of
  // each); lane l writes row 8c + l/8 at physical piece l % 8, which holds
  // logical piece (l % 8) ^ ((row >> 1) & 7). Rows past N read row N-1.
  const uint8_t* wsrc[WDMA];
  int wpiece[WDMA];
#pragma unroll
  for (int i = 0; i < WDMA; ++i) {
    const int R = 8 * (wave * WDMA + i) + lane / 8;
    const int n = n0 + R < N ? n0 + R : N - 1;
    wsrc[i] = packed + (int64_t)n * RB + (int64_t)t_begin * (BK / 2);
    wpiece[i] = 16 * ((lane % 8) ^ ((R >> 1) & 7));
  }
  // --- scales of the lane's two output columns
  const uint16_t* ssrc[TN];
  const uint8_t* zsrc[TN];
#pragma unroll
  for (int b = 0; b < TN; ++b) {
    const int n = n0 + wn * WNT + b * 32 + c32;
    ssrc[b] = scales + (int64_t)(n < N ? n : N - 1) * G;
    zsrc[b] = AFF ? zeros + (int64_t)(n < N ? n : N - 1) * G : nullptr;
  }
  const int spg_log = SPG == 0 ? gshift : SPG == 8 ? 3 : SPG == 4 ? 2 : SPG == 2 ? 1 : 0;
#pragma unroll
  for (int b = 0; b < TN; ++b) {
    ssrc[b] += t_begin >> spg_log;
    if constexpr (AFF) zsrc[b] += t_begin >> spg_log;
  }

  // Loads (an index past the end is clamped to a valid address; such data is
  // never used).
  uint32_t sr[NXS][TN];                        // s(t) in slot t % NXS
  uint32_t zr[NXS][TN];                        // zero points alike (AFF)
  auto issue_x = [&](int t, int stage) {
    const int tc = t < T ? t : T - 1;
    const char* base = xtile + (int64_t)tc * (2 * BK);
#pragma unroll
    for (int i = 0; i < XDMA; ++i)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + xoff[i]),
                                       reinterpret_cast<void*>(lds + stage * A_BYTES + (wave * XDMA + i) * 1024),
                                       16, 0, 0);
  };
  auto issue_s = [&](int t, int slot) {
    const int tc = t < T ? t : T - 1;
    // Sub-steps of one group load the same scales; the opaque index keeps the
    // compiler from merging such loads, which would change the load counts the
    // waits rely on.
    int gi = tc >> spg_log;
    asm volatile("" : "+s"(gi));
#pragma unroll
    for (int b = 0; b < TN; ++b) sr[slot][b] = ssrc[b][gi];
    if constexpr (AFF) {
#pragma unroll
      for (int b = 0; b < TN; ++b) zr[slot][b] = zsrc[b][gi];
    }
  };
  auto issue_w = [&](int st, int slot) {
#pragma unroll
    for (int i = 0; i < WDMA; ++i) {
      int o = 128 * st + wpiece[i];
      o = o < RBl - 16 ? o : RBl - 16;         // past the row end: valid, unused
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(wsrc[i] + (uint32_t)o),
                                       reinterpret_cast<void*>(lds + W_LDS + slot * W_BYTES + (wave * WDMA + i) * 1024),
                                       16, 0, 0);
    }
  };

  // Operand LDS offsets. A, k-step s: row wm*128 + c32 (+ 32 a), logical
  // piece KS*h + s. Packed W of lane (n = c32, h), tile b, sub-step u of a
  // super-tile: bytes (BK/2) u + (BK/4) h of row wn*64 + 32 b + n, whose
  // swizzle term (row >> 1) & 7 is (n >> 1) & 7.
  int aoff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int ra = wm * WMT + c32;
    aoff[s] = 2 * (ra * BK + 8 * swz(ra, KS * h + s));
  }
  const int wsw = (c32 >> 1) & 7;
  auto woff = [&](int u, int b) {
    const int byte = (BK / 2) * u + (BK / 4) * h;
    return (wn * WNT + b * 32 + c32) * 128 + 16 * ((byte >> 4) ^ wsw) + (byte & 15);
  };

  // Each code is multiplied by its group's binary16 scale as it is expanded:
  // w_hat = q * scale rounded once to binary16 (exact whenever the product
  // fits 11 significant bits; a relative error of at most 2^-11 otherwise,
  // subnormal products included), so the MFMAs accumulate x . w_hat directly
  // and no accumulator is touched at a group boundary. A zero scale makes its
  // group contribute nothing, whatever its codes.
  // That needs |q * scale| <= 65504: every scale at most 8188 (4094 for affine
  // codes, whose integer weights reach 15). A block that meets a larger (or
  // non-finite) scale in its columns discards its first pass and makes two
  // more over K: one with only the large-scale groups, their scales
  // multiplied by 2^-16 (an exponent shift: exact, and normal since the scale
  // is at least 4096), whose sums are then multiplied by 2^16, and one adding
  // the other groups at their own scales. Every product keeps its single
  // binary16 rounding; only the sum order changes.
  // Pass modes: 0 every group as is; 1 the groups with small scales only; 2
  // the groups with large scales only, scaled by 2^-16.
  constexpr uint32_t kSafe = AFF ? 0x6BFFu : 0x6FFFu;   // largest scale bits without overflow

  float16_t acc[TM][TN];
  uint32_t big = 0;                            // a scale above kSafe was seen (mode 0)

  // Scale word (the group's factor twice, binary16) of a column whose scale
  // has bits sb, in pass mode `mode`.
  auto scale_word = [&](uint32_t sb, int mode) {
    const bool large = (sb & 0x7FFFu) > kSafe;
    const bool keep = mode == 0 || (mode == 1) != large;
    const uint32_t f = sb - (mode == 2 ? 0x4000u : 0u);   // 2^-16: exponent - 16
    return keep ? f | (f << 16) : 0u;
  };

  // The usual pass (mode 0), operands staged through the LDS rings.
  auto run = [&]() __attribute__((always_inline)) {
    uint32_t s2[TN];                           // the group's scale factor twice, binary16
    uint32_t zb[TN];                           // bias word of the current group (AFF)
    half8_t af[TM];                            // A fragments of the next k-step
    uint32_t wp[TN][KS];                       // packed words of the current sub-step
    auto read_a = [&](int stage, int s, half8_t* dst) {
#pragma unroll
      for (int a = 0; a < TM; ++a)
        dst[a] = *reinterpret_cast<const half8_t*>(lds + stage * A_BYTES + aoff[s] + a * 32 * BK * 2);
    };
    auto read_w = [&](int slot, int u, uint32_t (*dst)[KS]) {
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const uint8_t* p = lds + W_LDS + slot * W_BYTES + woff(u, b);
        if constexpr (BK == 64) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
          dst[b][0] = v.x; dst[b][1] = v.y; dst[b][2] = v.z; dst[b][3] = v.w;
        } else {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(p);
          dst[b][0] = v.x; dst[b][1] = v.y;
        }
      }
    };
    auto expand_b = [&](const uint32_t (*w)[KS], int s, half8_t* bf) {
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        half2_t hw[4];
        if constexpr (AFF) codes_to_half_natural_zp(w[b][s], hw, zb[b]);
        else codes_to_half_natural(w[b][s], hw);
        const half2_t sc = __builtin_bit_cast(half2_t, s2[b]);
#pragma unroll
        for (int i = 0; i < 4; ++i) hw[i] *= sc;
        bf[b] = as_half8(hw);
      }
    };
    // State of the group that opens at the sub-step whose scale (and zero
    // point) slot is `slot`.
    auto open_group = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const uint32_t sb = sr[slot][b] & 0xFFFFu;
        big |= (sb & 0x7FFFu) > kSafe ? 1u : 0u;
        s2[b] = scale_word(sb, 0);
        if constexpr (AFF) zb[b] = zp_bias_natural(zr[slot][b]);
      }
    };

    // Prologue: the load groups of the virtual sub-steps -D .. -1, built like
    // the steady state's (x(t+D), s(t+D), super-tile t/SUB + WS - 1 where t is
    // a multiple of SUB), the first one also carrying the super-tiles that the
    // steady state would have loaded before it. Then wait for that first group
    // and read sub-step 0's k-step-0 fragments and packed words.
    constexpr int catch_up = WS - (D + SUB - 1) / SUB;   // super-tiles 0 .. catch_up-1
    unroll<0, D>([&](auto I_) {
      constexpr int t = decltype(I_)::value - D;
      issue_x(t + D, (t + D) % NXS);
      if constexpr (t == -D) {
        issue_s(0, 0);
#pragma unroll
        for (int st = 0; st < catch_up; ++st) issue_w(st, st % WS);
      } else {
        if constexpr (s_used(t + D)) issue_s(t + D, (t + D) % NXS);
        if constexpr (t % SUB == 0) issue_w(t / SUB + WS - 1, (t / SUB + WS - 1) % WS);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    constexpr auto prologue_newer = [group_loads]() {
      int n = 0;
      for (int i = 1; i <= D - 1; ++i) n += group_loads(-i);
      return n;
    };
    wait_vmcnt<prologue_newer()>();
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_a(0, 0, af);
    read_w(0, 0, wp);
    open_group(0);                             // sub-step 0 opens the first group

    // Sub-step t = t0 + J, t0 a multiple of U: x stage J % NXS, W slot
    // (J / SUB) % WS, scale slot J % NXS, all compile-time.
    // (always inlined: an outlined sub-step would take the DMA destinations and
    // the register arrays by reference, i.e. through scratch memory)
    auto substep = [&](auto J_, int t) __attribute__((always_inline)) {
      constexpr int J = decltype(J_)::value;
      constexpr int ws = (J / SUB) % WS, xs = J % NXS;
      constexpr int J1 = (J + 1) % U;
      constexpr int xs1 = J1 % NXS, ws1 = (J1 / SUB) % WS, u1 = J1 % SUB;
      __builtin_amdgcn_sched_barrier(0);
      issue_x(t + D, (J + D) % NXS);           // into the stage of t-1
      if constexpr (s_used(J + D)) issue_s(t + D, (J + D) % NXS);
      if constexpr (J % SUB == 0) issue_w(t / SUB + WS - 1, (ws + WS - 1) % WS);
      half8_t bcur[TN];
      expand_b(wp, 0, bcur);
      __builtin_amdgcn_sched_barrier(0);
      uint32_t wnext[TN][KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        half8_t cur[TM];
#pragma unroll
        for (int a = 0; a < TM; ++a) cur[a] = af[a];
        if (s + 1 < KS) {
          read_a(xs, s + 1, af);
        } else {                               // sub-step t+1: k-step 0 and its packed words
          wait_vmcnt<newer_loads(J)>();
          lds_barrier();                       // data of t+1 visible; stage of t free
          __builtin_amdgcn_sched_barrier(0);
          read_a(xs1, 0, af);
          read_w(ws1, u1, wnext);
        }
        half8_t bnext[TN];
        if (s + 1 < KS) expand_b(wp, s + 1, bnext);
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur[a], bcur[b], acc[a][b], 0, 0, 0);
        if (s + 1 < KS) {
          // one MFMA, four VALU (the next k-step's codes and scale), one LDS read
#pragma unroll
          for (int i = 0; i < TM * TN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            if (i < TM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        } else {
          // The scale (and zero-point) slot of t+1 holds t+1's group wherever
          // a group can open there (every sub-step when the group size is
          // decided at run time), so the group state is switched there without
          // a condition.
          if constexpr (SPG == 0 || (J + 1) % SPG == 0) open_group(xs1);
#pragma unroll
          for (int i = 0; i < TM * TN; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < TM + TN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < TN; ++b) bcur[b] = bnext[b];
      }
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int i = 0; i < KS; ++i) wp[b][i] = wnext[b][i];
    };

    // Main loop over whole bodies, then the last partial body with each
    // sub-step guarded (sub-steps skipped there are all at the end, so the
    // load counts of the ones that run are unchanged).
    int t0 = 0;
    for (; t0 + U <= T; t0 += U)
      unroll<0, U>([&](auto J) { substep(J, t0 + decltype(J)::value); });
    unroll<0, U>([&](auto J) {
      if (t0 + decltype(J)::value < T) substep(J, t0 + decltype(J)::value);
    });
    wait_vmcnt<0>();                           // no LDS DMA in flight at exit
  };

  // The rare passes (modes 2 and 1): each wavefront reads its A fragments and
  // packed words straight from global memory, with the same k order and
  // fragment layout as the usual pass. Slow, and kept apart from the LDS
  // rings so that it adds no LDS traffic the usual pass has to be ordered
  // against.
  auto run_direct = [&](int mode) {
    const int kb = RB;                         // bytes per packed row
    int rows[TM], cols[TN];
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int m = m0 + wm * WMT + a * 32 + c32;
      rows[a] = m < M ? m : M - 1;
    }
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int n = n0 + wn * WNT + b * 32 + c32;
      cols[b] = n < N ? n : N - 1;
    }
    for (int t = t_begin; t < t_begin + T; ++t) {
      const int gi = t >> spg_log;
      uint32_t s2[TN], zb[TN];
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        s2[b] = scale_word(scales[(int64_t)cols[b] * G + gi], mode);
        zb[b] = 0u;
        if constexpr (AFF) zb[b] = zp_bias_natural(zeros[(int64_t)cols[b] * G + gi]);
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int k = t * BK + (BK / 2) * h + 8 * s;   // first of the lane's 8 codes
        half8_t af[TM], bf[TN];
#pragma unroll
        for (int a = 0; a < TM; ++a)
          af[a] = *reinterpret_cast<const half8_t*>(x + (int64_t)rows[a] * K + k);
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const uint32_t d = *reinterpret_cast<const uint32_t*>(packed + (int64_t)cols[b] * kb + (k >> 1));
          half2_t hw[4];
          if constexpr (AFF) codes_to_half_natural_zp(d, hw, zb[b]);
          else codes_to_half_natural(d, hw);
          const half2_t sc = __builtin_bit_cast(half2_t, s2[b]);
#pragma unroll
          for (int i = 0; i < 4; ++i) hw[i] *= sc;
          bf[b] = as_half8(hw);
        }
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
      }
    }
  };

  auto zero_acc = [&]() {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  };
  zero_acc();
  run();
  // Block-wide OR of the waves' flags, through the ring array itself (every
  // DMA and LDS read of the pass has completed). (__syncthreads_or would add a
  // second LDS object, after which the compiler can no longer tell the DMA
  // targets from the operand reads and waits for every load in flight.)
  {
    const bool wave_big = __builtin_amdgcn_ballot_w64(big != 0u) != 0;
    lds_barrier();
    if (lane == 0) reinterpret_cast<volatile uint32_t*>(lds)[wave] = wave_big ? 1u : 0u;
    lds_barrier();
  }
  const uint32_t* flags = reinterpret_cast<const uint32_t*>(lds);
  if ((flags[0] | flags[1] | flags[2] | flags[3]) != 0u) {
    // a large scale somewhere in the block's columns: mode 2, times 2^16,
    // then mode 1 on top
    zero_acc();
    run_direct(2);
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b) acc[a][b] *= 65536.0f;
    run_direct(1);
  }

  // Split of K: the share's partial tile goes to the workspace; a second
  // kernel adds the shares in order and applies the output step.
  if (sp.S > 1) {
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int n = n0 + wn * WNT + b * 32 + c32;
          const int m = m0 + wm * WMT + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (m < M && n < N) sp.part[((int64_t)split * M + m) * N + n] = acc[a][b][i];
        }
    return;
  }

  // Store: lane l holds column l%32 and rows 8*(i/4) + 4*(l/32) + (i%4) of each
  // 32x32 tile (register i). A block tile inside y (every block but the last
  // row and column of tiles) stores without per-output bounds checks; the
  // output precision is one branch for the whole tile. The stores are
  // nontemporal (streamed past the caches): every block writes its whole
  // tile at the end, and on the one-round grids all blocks do so at once
  // (measured 0.8-2.8% faster per launch at M = 2048 on the 7B-class shapes).
  const bool full = m0 + BM <= M && n0 + BN <= N;
  auto store_all = [&](auto* yt) __attribute__((always_inline)) {
    typedef std::remove_pointer_t<decltype(yt)> T;
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int n = n0 + wn * WNT + b * 32 + c32;
      const float bn = ep.column(n < N ? n : N - 1);
      if (full) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = m0 + wm * WMT + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
            __builtin_nontemporal_store((T)ep.apply(acc[a][b][i], bn), yt + (int64_t)m * N + n);
          }
      } else {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = m0 + wm * WMT + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
            if (m < M && n < N) __builtin_nontemporal_store((T)ep.apply(acc[a][b][i], bn), yt + (int64_t)m * N + n);
          }
      }
    }
  };
  if (ep.half) store_all(static_cast<_Float16*>(y));
  else store_all(static_cast<float*>(y));
}

// BK for a group size, or 0 if the kernel does not take it (group / BK must be
// a power of two: the group index of a sub-step is a shift).
static int tiled_bk(int64_t group) {
  if (group == 32) return 32;
  if (group % 64 == 0 && ((group / 64) & (group / 64 - 1)) == 0) return 64;
  return 0;
}

// Second step of a split of K: y[m, n] = act(sum over shares q = 0 .. S-1,
// in that order, of part[q, m, n] + bias[n]) in y's precision. Four outputs
// per thread (N a multiple of 4), one per thread otherwise.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int S,
                                                           int64_t MN, int N, void* __restrict__ y,
                                                           Epilogue ep) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= MN) return;
  if ((N & 3) == 0) {                          // four outputs of one row
    float4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int q = 0; q < S; ++q) v += *reinterpret_cast<const float4_t*>(part + q * MN + i0);
    const int64_t n = i0 % N;
#pragma unroll
    for (int j = 0; j < 4; ++j) ep.store(y, i0 + j, v[j], n + j);
  } else {
    for (int64_t i = i0; i < i0 + 4 && i < MN; ++i) {
      float v = 0.0f;
      for (int q = 0; q < S; ++q) v += part[q * MN + i];
      ep.store(y, i, v, i % N);
    }
  }
}

// Tile configuration, group cadence and split of K for one call.
struct TiledPlan {
  int cfg;          // 0: 128 x 256, 1: 128 x 128, 2: 64 x 128, 3: 32 x 128 block tiles
  int BK, gs;       // codes per sub-step; group = BK << gs
  int64_t tiles;    // output tiles
  int S, steps;     // shares of K and sub-steps per share (S = 1: no split)
  int64_t ws_bytes; // workspace the split needs (0 without one)
};

// Block tile (rows of x x weight rows), always four wavefronts side by side
// along N: the first of 128 x 256, 128 x 128, 64 x 128 and 32 x 128 whose
// height fits M (rounded up to 32) and whose grid has 160 blocks or more,
// else 32 x 128. Measured on the 7B-class shapes: 128 x 256 is 7-8% faster
// than 256 x 128 (x is read from L2 half as often); a grid of about 170
// large tiles beats one of 340 smaller ones (M = 512 on [11008, 4096]: 60 us
// against 78), but 128 blocks on 256 CUs do not. For small M the narrow
// wave tiles (one 32-column MFMA tile each) expand every code once per
// block where 2 x 2 wavefronts expanded it twice: M = 128 on [4096, 11008]
// 70.4 -> 50.0 us with 32 x 128 tiles, [4096, 4096] 29.2 -> 21.5 us.
// Split of K (only with a workspace): a grid of 128 tiles or fewer leaves at
// least half the CUs idle while each block walks all of K alone, a chain of
// sub-steps bound by load latency. Then K is cut into S = 2, 4 or 8 shares
// (the most that keep the grid within two blocks per CU), each at least 16
// sub-steps and starting on a packed super-tile and a group boundary. The
// shares' partial tiles meet in the workspace and a second kernel adds them
// in share order (deterministic; the kernel boundary orders the partials'
// stores before their loads, where one kernel would need a device-wide cache
// write-back per block, which measured 4x slower). Measured (graph replays):
// M = 128 on [4096, 11008] 49.2 -> 31.4 us, on [4096, 4096] 21.0 -> 17.5 us;
// grids of 256 tiles were slower split (M = 256 on [4096, 4096] 23.0 -> 25.1
// us, M = 512 29.5 -> 35.0 us) and are not.
static TiledPlan tiled_plan(int64_t M, int64_t N, int64_t K, int64_t group) {
  TiledPlan pl{};
  pl.BK = tiled_bk(group);
  auto grid_of = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  const int64_t Mr = (M + 31) / 32 * 32;
  pl.cfg = (Mr >= 128 && grid_of(128, 256) >= 160) ? 0
         : (Mr >= 128 && grid_of(128, 128) >= 160) ? 1
         : (Mr >= 64 && grid_of(64, 128) >= 160) ? 2 : 3;
  // (a 32-row tile of 32-code sub-steps is 2 KB of x: less than one DMA
  // instruction per wavefront, so group 32 takes 64-row tiles at least)
  if (pl.BK == 32 && pl.cfg == 3) pl.cfg = 2;
  pl.tiles = pl.cfg == 0 ? grid_of(128, 256) : grid_of(128 >> (pl.cfg - 1), 128);
  pl.gs = 0;
  while ((int64_t(pl.BK) << pl.gs) < group) ++pl.gs;
  const int64_t T = K / pl.BK;
  pl.S = 1;
  pl.steps = (int)T;
  const int64_t align = std::max<int64_t>(256 / pl.BK, int64_t(1) << pl.gs);
  for (int S = 8; S >= 2 && pl.tiles <= 128; S /= 2) {
    if (pl.tiles * S > 512) continue;
    int64_t steps = (T + S - 1) / S;
    steps = (steps + align - 1) / align * align;
    const int64_t shares = (T + steps - 1) / steps;
    if (steps < 16 || shares < 2) continue;
    pl.S = (int)shares;
    pl.steps = (int)steps;
    break;
  }
  if (pl.S > 1) pl.ws_bytes = (int64_t)pl.S * M * N * 4;
  return pl;
}

int64_t matmul_tiled_workspace(int64_t M, int64_t N, int64_t K, int64_t group) {
  if (tiled_bk(group) == 0 || M < 1 || M >= (1ll << 31) || N >= (1ll << 31)) return 0;
  return tiled_plan(M, N, K, group).ws_bytes;
}

const char* matmul_tiled_unsupported(int x_dtype, int64_t M, const void* x, const uint8_t* packed,
                                     int64_t N, int64_t K, int64_t group) {
  if (x_dtype != 1) return "tiled kernel takes binary16 activations only";
  const int BK = tiled_bk(group);
  if (BK == 0) return "tiled kernel takes group 32 or 64 times a power of two";
  if (K % BK != 0) return "tiled kernel needs K to be a multiple of min(group, 64)";
  if (K >= (1ll << 23)) return "tiled kernel needs K below 2^23";
  if (M >= (1ll << 31) || N >= (1ll << 31)) return "tiled kernel needs M and N below 2^31";
  // one block of 256 threads per tile and share of K; a dispatch holds fewer
  // than 2^32 threads
  const TiledPlan pl = tiled_plan(M < 1 ? 1 : M, N, K, group);
  if (pl.tiles * pl.S >= (1ll << 24)) return "tiled kernel takes at most 2^24 blocks (M x N too large)";
  if ((uintptr_t)x % 16 || (uintptr_t)packed % 16) return "tiled kernel needs 16-byte aligned x and packed";
  return nullptr;
}

hipError_t launch_matmul_tiled(const void* x, int64_t M, const uint8_t* packed,
                               const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                               int64_t group, void* y, Epilogue ep, void* workspace,
                               int64_t workspace_bytes, hipStream_t stream) {
  const int G = (int)((K + group - 1) / group);
  if (M >= (1ll << 31) || N >= (1ll << 31)) return hipErrorInvalidValue;
  TiledPlan pl = tiled_plan(M, N, K, group);
  TiledSplit sp{nullptr, 1, pl.steps};
  if (pl.S > 1 && workspace && workspace_bytes >= pl.ws_bytes) {
    sp.part = static_cast<float*>(workspace);
    sp.S = pl.S;
  } else {
    sp.steps = (int)(K / pl.BK);
  }
  const int64_t blocks = pl.tiles * sp.S;
  if (blocks >= (1ll << 24)) return hipErrorInvalidValue;   // refused by matmul_tiled_unsupported
  const int BK = pl.BK, gs = pl.gs, cfg = pl.cfg;
#define INT4DQ_TILED_PICK(TMV, A, TNV)                                                                     \
  (BK == 32 ? matmul_tiled_kernel<32, 1, (TMV > 1 ? TMV : 2), A, 4, TNV>                                 \
   : gs == 0 ? matmul_tiled_kernel<64, 1, TMV, A, 4, TNV> : gs == 1 ? matmul_tiled_kernel<64, 2, TMV, A, 4, TNV> \
   : gs == 2 ? matmul_tiled_kernel<64, 4, TMV, A, 4, TNV> : gs == 3 ? matmul_tiled_kernel<64, 8, TMV, A, 4, TNV> \
             : matmul_tiled_kernel<64, 0, TMV, A, 4, TNV>)
#define INT4DQ_TILED_CFG(A)                                                                            \
  (cfg == 0 ? INT4DQ_TILED_PICK(4, A, 2) : cfg == 1 ? INT4DQ_TILED_PICK(4, A, 1)                      \
   : cfg == 2 ? INT4DQ_TILED_PICK(2, A, 1) : INT4DQ_TILED_PICK(1, A, 1))
  const auto kernel = zeros ? INT4DQ_TILED_CFG(true) : INT4DQ_TILED_CFG(false);
#undef INT4DQ_TILED_CFG
#undef INT4DQ_TILED_PICK
  hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const _Float16*>(x), (int)M, packed, scales, zeros, (int)N, (int)K, G,
                     gs, y, ep, sp);
  if (sp.S > 1) return launch_split_reduce(sp.part, sp.S, M, N, y, ep, stream);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const float* part, int S, int64_t M, int64_t N, void* y, Epilogue ep,
                               hipStream_t stream) {
  const int64_t MN = M * N;
  const int64_t rblocks = (MN + 1023) / 1024;
  if (rblocks >= (1ll << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)rblocks), dim3(256), 0, stream, part, S, MN,
                     (int)N, y, ep);
  return hipGetLastError();
}

}  // namespace int4dq
