// matmul_tiled.hip -- dequantizing matmul for many activation rows (binary16
// x) on gfx950: an MFMA kernel bound by matrix-core throughput.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, int4_matmul): y = x @ dequantize(W).T,
// one group at a time -- x times the group's integer codes first, then the
// group's scale on each output column. Full-precision weights never reach
// memory ("Build a Blockwise INT4 Inference Engine", architecture overview:
// the fusion boundary); here they exist only as exact fp16 integer codes in
// the registers that feed the matrix cores.
//
// Block tile 256 (rows of x) x 128 (weight rows), 256 threads = 2 x 2
// wavefronts, each owning 128 x 64 outputs as 4 x 2 tiles of
// v_mfma_f32_32x32x16_f16 (fp32 accumulation, 128 accumulator VGPRs).
// K advances in sub-steps of BK = min(group, 64) codes:
//  * x tiles [256 x BK] fp16 go global -> LDS by DMA (global_load_lds, 16 B
//    per lane, no VGPRs) into a 3-stage ring, two sub-steps ahead. Each 128-B
//    row holds 8 16-byte pieces stored at piece ^ (row & 7), so the 32 rows an
//    MFMA operand read touches fall in distinct banks.
//  * The weights never touch LDS: each lane loads the 16 packed bytes of its
//    weight row that its B fragments need (two sub-steps ahead, in registers)
//    and expands each 32-bit word to 8 exact fp16 codes right before the MFMA
//    (codes_to_half_natural). The k order inside a sub-step is a fixed
//    permutation shared by A and B (lane half h, k-step s: codes 32h + 8s ..),
//    which leaves the dot product unchanged.
//  * Integer-first scaling with one accumulator set: the accumulator holds
//    (sum of finished groups' scaled partials) / (scale of the current group);
//    at each group boundary it is multiplied by s_prev / s_new for its column,
//    the group's integer products are accumulated by the MFMAs, and the final
//    value is multiplied by the last scale. A zero scale (a group of zero
//    codes) leaves the running scale unchanged. Mathematically this is
//    sum_g s_g * (x . q_g); the ratio multiply adds one fp32 rounding per group.
#include "device_common.h"
#include "kernels.h"

#include <type_traits>

namespace int4dq {

namespace {
constexpr int kBM = 256, kBN = 128, kThreads = 256;
typedef float float16_t __attribute__((ext_vector_type(16)));

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
}  // namespace

// BK: codes per sub-step (32 or 64). Requires K % BK == 0 and group = BK << gshift.
template <int BK>
__global__ __launch_bounds__(kThreads) void matmul_tiled_kernel(
    const _Float16* __restrict__ x, int M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, int N, int K, int G, int gshift,
    float* __restrict__ y) {
  constexpr int KS = BK / 16;                 // MFMA k-steps per sub-step
  constexpr int PIECES = BK / 8;              // 16-byte pieces per x row per sub-step
  constexpr int STAGE_HALVES = kBM * BK;      // one x stage
  constexpr int XDMA = kBM * PIECES / 64 / 4; // DMA instructions per wave per stage
  typedef typename std::conditional<BK == 64, u32x4_t, u32x2_t>::type wvec_t;
  __shared__ __attribute__((aligned(1024))) _Float16 xs[3 * STAGE_HALVES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int c32 = lane & 31, h = lane >> 5;

  // Tile assignment: consecutive block ids walk down the M tiles first so the
  // blocks resident together share weight tiles.
  const int mtiles = (M + kBM - 1) / kBM;
  const int bm = blockIdx.x % mtiles, bn = blockIdx.x / mtiles;
  const int m0 = bm * kBM, n0 = bn * kBN;

  // --- x DMA addressing: wave instruction i writes LDS bytes [1 KB * (wave*XDMA+i), +1 KB):
  //     rows R + i * (64 / PIECES) with R = wave * XDMA * (64 / PIECES) + lane / PIECES, and
  //     physical piece lane % PIECES, which holds logical piece c = (lane % PIECES) ^ (row % PIECES)
  //     -- the same c for every i, since each instruction advances by whole swizzle periods.
  constexpr int RPI = 64 / PIECES;                            // rows per DMA instruction
  const int xr0 = wave * XDMA * RPI + lane / PIECES;
  const int xc = (lane % PIECES) ^ (xr0 & (PIECES - 1));
  const bool xfull = m0 + kBM <= M;                           // common case: no row clamping
  auto xrow_off = [&](int i) -> int64_t {                     // element offset of row i's piece
    int r = m0 + xr0 + i * RPI;
    if (!xfull) r = r < M ? r : M - 1;                        // rows past M: discarded
    return (int64_t)r * K + 8 * xc;
  };
  auto dma_x = [&](int t, int stage) {
#pragma unroll
    for (int i = 0; i < XDMA; ++i)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(x + xrow_off(i) + t * BK),
          reinterpret_cast<void*>(xs + stage * STAGE_HALVES + (wave * XDMA + i) * 512), 16, 0, 0);
  };

  // --- weights: lane (c32, h) of n-tile b reads row n, bytes [t*BK/2 + h*BK/4, +BK/4)
  const uint8_t* wsrc[2];
  const uint16_t* ssrc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    int n = n0 + wn * 64 + b * 32 + c32;
    n = n < N ? n : N - 1;                                     // tail rows: read, discard
    wsrc[b] = packed + (int64_t)n * (K >> 1) + h * (BK / 4);
    ssrc[b] = scales + (int64_t)n * G;
  }
  wvec_t wr[3][2];
  uint32_t sr[3][2];
  auto load_w = [&](int t, int slot) {
#pragma unroll
    for (int b = 0; b < 2; ++b) sr[slot][b] = ssrc[b][(t * BK) >> (gshift + (BK == 64 ? 6 : 5))];
#pragma unroll
    for (int b = 0; b < 2; ++b)
      wr[slot][b] = __builtin_nontemporal_load(reinterpret_cast<const wvec_t*>(wsrc[b] + t * (BK / 2)));
  };

  float16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  float srun[2] = {0.0f, 0.0f};

  const int T = K / BK;
  const int steps_per_group = 1 << gshift;
  // A-fragment LDS offsets (halves) for k-step s within a stage, for m-tile 0;
  // m-tile a adds a * 32 rows (a constant, and a whole number of swizzle periods).
  int aoff[KS];
  {
    const int r = wm * 128 + c32;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = (PIECES == 8 ? 4 * h : 2 * h) + s;         // logical piece of k = 32h/16h + 8s
      aoff[s] = r * BK + 8 * (c ^ (r & (PIECES - 1)));
    }
  }

  // Loads of sub-step t (x DMA + scales + weights), always issued: an index
  // past the end is clamped to the last sub-step (its data lands in a stage or
  // register slot that is never read again). With no branch around loads the
  // wait counts below stay exact.
  auto issue = [&](int t, int stage, int slot) {
    const int tc = t < T ? t : T - 1;
    dma_x(tc, stage);
    load_w(tc, slot);
  };
  issue(0, 0, 0);
  issue(1, 1, 1);

  auto substep = [&](int t, int stage, int slot, int slot2) {
    // Outstanding: loads of t and t+1 (XDMA + 4 each, in order); wait for t's.
    wait_vmcnt<XDMA + 4>();
    lds_barrier();                                             // x stage t visible; stage t+2 free
    issue(t + 2, (stage + 2) % 3, slot2);
    if ((t & (steps_per_group - 1)) == 0) {                    // first sub-step of a group
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float sn = half_bits_to_float((uint16_t)sr[slot][b]);
        const bool live = sn != 0.0f;                          // zero scale: keep the running one
        const float ratio = live ? (srun[b] == 0.0f ? 0.0f : srun[b] / sn) : 1.0f;
        srun[b] = live ? sn : srun[b];
#pragma unroll
        for (int a = 0; a < 4; ++a) acc[a][b] *= ratio;
      }
    }
    const _Float16* st = xs + stage * STAGE_HALVES;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      half8_t af[4], bf[2];
#pragma unroll
      for (int a = 0; a < 4; ++a) af[a] = *reinterpret_cast<const half8_t*>(st + aoff[s] + a * 32 * BK);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        half2_t hw[4];
        codes_to_half_natural(wr[slot][b][s], hw);
        bf[b] = as_half8(hw);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
  };

  // Main loop over whole triples (ring slots and stages are compile-time),
  // then the one or two remaining sub-steps.
  const int Tm = T - T % 3;
  for (int t = 0; t < Tm; t += 3) {
    substep(t, 0, 0, 2);
    substep(t + 1, 1, 1, 0);
    substep(t + 2, 2, 2, 1);
  }
  if (Tm < T) substep(Tm, 0, 0, 2);
  if (Tm + 1 < T) substep(Tm + 1, 1, 1, 0);
  wait_vmcnt<0>();                                             // no LDS DMA in flight at exit

  // Epilogue: apply the last running scale; lane l holds column l%32 and rows
  // 8*(i/4) + 4*(l/32) + (i%4) of each 32x32 tile (register i).
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int n = n0 + wn * 64 + b * 32 + c32;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * 128 + a * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (m < M && n < N) y[(int64_t)m * N + n] = acc[a][b][i] * srun[b];
      }
  }
}

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
  if (K >= (1ll << 30)) return "tiled kernel needs K below 2^30";
  if ((uintptr_t)x % 16 || (uintptr_t)packed % 16) return "tiled kernel needs 16-byte aligned x and packed";
  return nullptr;
}

hipError_t launch_matmul_tiled(const void* x, int64_t M, const uint8_t* packed,
                               const uint16_t* scales, int64_t N, int64_t K, int64_t group,
                               float* y, hipStream_t stream) {
  const int BK = tiled_bk(group);
  const int G = (int)((K + group - 1) / group);
  int gshift = 0;
  while ((BK << gshift) < group) ++gshift;
  const int64_t blocks = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (M >= (1ll << 31) || N >= (1ll << 31) || blocks >= (1ll << 31)) return hipErrorInvalidValue;
  const _Float16* xh = static_cast<const _Float16*>(x);
  if (BK == 64)
    hipLaunchKernelGGL(matmul_tiled_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, xh,
                       (int)M, packed, scales, (int)N, (int)K, G, gshift, y);
  else
    hipLaunchKernelGGL(matmul_tiled_kernel<32>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, xh,
                       (int)M, packed, scales, (int)N, (int)K, G, gshift, y);
  return hipGetLastError();
}

}  // namespace int4dq
