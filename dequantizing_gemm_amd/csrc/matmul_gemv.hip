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

namespace int4dq {

namespace {
constexpr int kGemvMaxChunks = 16;             // wavefronts per block (1024 threads)

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
