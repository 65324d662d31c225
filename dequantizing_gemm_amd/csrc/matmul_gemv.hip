// matmul_gemv.hip -- dequantizing matrix-vector product (one activation row,
// binary16 x) on gfx950: a weight-streaming kernel bound by HBM bandwidth.
//
// Definition (drill page "Implement INT4 group quantization, nibble packing
// and a dequantizing matmul", statement, int4_matmul): y = x @ dequantize(W).T,
// one group at a time -- x times the group's integer codes, then the group's
// scale. ("Build a Blockwise INT4 Inference Engine", architecture overview and
// takeaways: full-precision weights never reach memory; the bottleneck is
// memory bandwidth.)
//
// With one activation row every packed byte is used for two flops, so the
// kernel is a pure stream of the packed weights, and the way it reads them
// decides its speed. A wavefront load instruction here covers 1 KB of one
// weight row (lane l: bytes c*1024 + 16 l), i.e. eight full 128-byte lines:
// this streams at the rate of a plain contiguous copy, where a layout that
// feeds the matrix cores directly (16 rows x 64 bytes per instruction, half
// lines) measured 12-25% slower. So the contraction runs on the VALU:
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
//    (integer-first), summed over the wavefront (DPP and lane-swap
//    butterfly) and over the block's wavefronts in a fixed order through
//    LDS: deterministic, no atomics.
//  * Lanes past the end of a row (last chunk) read the row's last 16 bytes
//    and contribute zero; rows past N are read as row N-1 and not written.
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

template <int RW>
__global__ __launch_bounds__(64 * kGemvMaxChunks) void matmul_gemv_kernel(
    const _Float16* __restrict__ x, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, int N, int K, int G, int group, int gsh,
    float* __restrict__ y) {
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
  uint32_t s[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) s[r] = (scales + (int64_t)row_of(r) * G)[gi];
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
      codes_to_half_spread(w[r][i], hw);
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
    y[n0 + threadIdx.x] = sum;
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
// Block = W wavefronts of 4 rows each. The activation row (permuted to the
// spread order, zero past K) and the block's scales are staged once in LDS;
// every weight load of a lane (one per column block) is issued before the
// first wait, and column c waits only for its own load. Used for group sizes
// 32 << p and K <= 12288; other shapes take the VALU kernel above.
// CM: column blocks (256 bytes) per row, >= ceil(K / 512). GS: min(gsh, 3)
// (group = 32 << gsh), which bounds the groups per row and so the scale
// entries each thread stages.
template <int CM, int GS, int W>
__global__ __launch_bounds__(64 * W) void matmul_gemv_mfma_kernel(
    const _Float16* __restrict__ x, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, int N, int K, int G, int group, int gsh,
    float* __restrict__ y) {
  typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
  constexpr int NT = 64 * W, ROWS = 4 * W;     // threads, rows per block
  constexpr int XPT = (CM * 64 + NT - 1) / NT; // 16-byte x units per thread (x row <= CM KB)
  constexpr int GMAX = (CM * 16 + (1 << GS) - 1) >> GS;           // groups per row, at most
  constexpr int SPT = (ROWS * GMAX + NT - 1) / NT;                 // scale entries per thread
  // Sized so that every thread's staging store is in bounds (no branch: a
  // branch here would make the compiler wait for every load at its join).
  __shared__ __attribute__((aligned(16))) uint32_t xsp[XPT * NT * 4];   // x, spread order
  __shared__ uint16_t ssh[SPT * NT];                                  // scales of the block's rows

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = lane >> 2, j = lane & 3;
  const int RB = K >> 1;
  const int n0 = blockIdx.x * ROWS;
  const int xunits = K >> 3;                   // 8 activations per unit

  // Phase 1: activations and scales (older than every weight load).
  u32x4_t xv[XPT];
#pragma unroll
  for (int t = 0; t < XPT; ++t) {
    int u = t * NT + tid;
    u = u < xunits ? u : xunits - 1;
    xv[t] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(x) + 16u * (uint32_t)u);
  }
  // the block's rows' scales are contiguous from row n0 (rows past N: clamped)
  const uint16_t* sblk = scales + (int64_t)n0 * G;
  const int slast = (N - n0 < ROWS ? N - n0 : ROWS) * G - 1;
  uint32_t sv[SPT];
#pragma unroll
  for (int t = 0; t < SPT; ++t) {
    const int e = t * NT + tid;
    sv[t] = sblk[(uint32_t)(e < slast ? e : slast)];
  }
  __builtin_amdgcn_sched_barrier(0);
  // Phase 2: the lane's 16 bytes of each column block of its row.
  const int n = n0 + 4 * wave + j < N ? n0 + 4 * wave + j : N - 1;
  const uint8_t* prow = packed + (int64_t)n * RB;
  u32x4_t w[CM];
#pragma unroll
  for (int c = 0; c < CM; ++c) {
    int o = c * 256 + b * 16;
    o = o < RB ? o : RB - 16;                  // past the row end: valid, masked below
    w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(prow + (uint32_t)o));
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt_gemv<CM>();                       // phase 1 landed
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < XPT; ++t) {
    const int u = t * NT + tid;
    // units past the end of x are stored as zeros: lanes past a row's end
    // then contribute exactly 0 without a mask
    const uint32_t z = u < xunits ? 0xFFFFFFFFu : 0u;
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
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // Column c of lane (b, j): codes 512 c + 32 b of row j, x units 64 c + 4 b
  // .. +3 (LDS dwords 4 per unit), group (16 c + b) >> gsh (exactly
  // (16 c >> gsh) + (b >> gsh), since 16 c is a multiple of 2^gsh when
  // gsh < 4 and b < 16 adds nothing when gsh >= 4). Lanes whose slice lies
  // past the row end read x units past K, which are zero.
  const uint16_t* srow = ssh + (4 * wave + j) * G + (b >> gsh);
  const uint32_t* xl = xsp + 16 * b;
  float acc = 0.0f;
  static_for<0, CM>([&](auto C_) {
    constexpr int c = decltype(C_)::value;
    const float sc = half_bits_to_float(srow[(16 * c) >> gsh]);
    u32x4_t xa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const u32x4_t*>(xl + 256 * c + 4 * i);
    wait_vmcnt_gemv<CM - 1 - c>();
    float4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t hw[4];
      codes_to_half_spread(w[c][i], hw);
      const half4_t b0 = __builtin_bit_cast(half4_t, u32x2v_t{__builtin_bit_cast(uint32_t, hw[0]), __builtin_bit_cast(uint32_t, hw[1])});
      const half4_t b1 = __builtin_bit_cast(half4_t, u32x2v_t{__builtin_bit_cast(uint32_t, hw[2]), __builtin_bit_cast(uint32_t, hw[3])});
      const half4_t a0 = __builtin_bit_cast(half4_t, u32x2v_t{xa[i].x, xa[i].y});
      const half4_t a1 = __builtin_bit_cast(half4_t, u32x2v_t{xa[i].z, xa[i].w});
      d = __builtin_amdgcn_mfma_f32_4x4x4f16(a0, b0, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_4x4x4f16(a1, b1, d, 0, 0, 0);
    }
    acc += sc * d.x;                           // row 0 of the block: the activation row
  });
  // Sum the 16 slices (lanes 4b+j, b = 0..15) of each of the 4 rows.
#pragma unroll
  for (int off = 4; off < 64; off <<= 1) acc += __shfl_xor(acc, off);
  if (b == 0 && n0 + 4 * wave + j < N) y[n0 + 4 * wave + j] = acc;
}

const char* matmul_gemv_unsupported(int x_dtype, int64_t M, const void* x,
                                    const uint8_t* packed, int64_t N, int64_t K,
                                    int64_t group) {
  if (x_dtype != 1) return "gemv kernel takes binary16 activations only";
  if (M != 1) return "gemv kernel takes M = 1";
  if (group % 32 != 0) return "gemv kernel needs group to be a multiple of 32";
  if (K % 32 != 0) return "gemv kernel needs K to be a multiple of 32";
  if (K / 2 > 1024 * kGemvMaxChunks) return "gemv kernel takes K <= 32768";
  if (N >= (1ll << 31)) return "gemv kernel needs N below 2^31";
  if ((uintptr_t)x % 16 || (uintptr_t)packed % 16) return "gemv kernel needs 16-byte aligned x and packed";
  return nullptr;
}

hipError_t launch_matmul_gemv(const void* x, const uint8_t* packed, const uint16_t* scales,
                              int64_t N, int64_t K, int64_t group, float* y, hipStream_t stream) {
  const int G = (int)((K + group - 1) / group);
  int gsh = 0;                                                 // log2(group / 32), or -1
  while ((32ll << gsh) < group) ++gsh;
  if ((32ll << gsh) != group) gsh = -1;
  const _Float16* xh0 = static_cast<const _Float16*>(x);
  const int cols = (int)((K / 2 + 255) / 256);                // 256-byte column blocks per row
  if (cols <= 24 && gsh >= 0 && g_gemv_mfma) {
    constexpr int W = g_gemv_waves;                              // wavefronts (4 rows each) per block
    const dim3 g16((unsigned)((N + 4 * W - 1) / (4 * W))), b256(64 * W);
#define INT4DQ_GEMV_MFMA(CMV)                                                                    \
  do {                                                                                          \
    const auto kern = gsh == 0 ? matmul_gemv_mfma_kernel<CMV, 0, W> : gsh == 1 ? matmul_gemv_mfma_kernel<CMV, 1, W> \
                    : gsh == 2 ? matmul_gemv_mfma_kernel<CMV, 2, W> : matmul_gemv_mfma_kernel<CMV, 3, W>;       \
    hipLaunchKernelGGL(kern, g16, b256, 0, stream, xh0, packed, scales, (int)N, (int)K, G,     \
                       (int)group, gsh, y);                                                     \
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
    return hipGetLastError();
  }
  const int chunks = (int)((K / 2 + 1023) / 1024);
  // Rows per block: enough wavefronts in flight (about 4096) to keep every
  // memory channel busy, up to 4 rows per wavefront.
  const int64_t want = (int64_t)chunks * N / 4096;
  const int rw = want >= 8 ? 8 : want >= 4 ? 4 : want >= 2 ? 2 : 1;
  const int64_t blocks = (N + rw - 1) / rw;
  const _Float16* xh = static_cast<const _Float16*>(x);
  const dim3 grid((unsigned)blocks), block(64 * chunks);
  if (rw == 8)
    hipLaunchKernelGGL(matmul_gemv_kernel<8>, grid, block, 0, stream, xh, packed, scales, (int)N, (int)K, G, (int)group, gsh, y);
  else if (rw == 4)
    hipLaunchKernelGGL(matmul_gemv_kernel<4>, grid, block, 0, stream, xh, packed, scales, (int)N, (int)K, G, (int)group, gsh, y);
  else if (rw == 2)
    hipLaunchKernelGGL(matmul_gemv_kernel<2>, grid, block, 0, stream, xh, packed, scales, (int)N, (int)K, G, (int)group, gsh, y);
  else
    hipLaunchKernelGGL(matmul_gemv_kernel<1>, grid, block, 0, stream, xh, packed, scales, (int)N, (int)K, G, (int)group, gsh, y);
  return hipGetLastError();
}

}  // namespace int4dq
