// Entry side of the sequence-parallel region: RMSNorm of each rank's
// sequence slice, written straight into that slice's rows of the gathered
// [T x H] buffer -- the buffer every rank holds after the all-gather that
// feeds the next column linear.
//
// The norm runs on sequence slices because it is row-wise (2kiu.com blog post,
// section 4.3; "张量并行", Megatron-SP section), and RMSNorm needs only the
// mean of squares of the whole hidden vector (blog post, section 3.3).
//
//   Y[r*T/N + t, :] = X_r[t, :] * (1 / sqrt(mean(X_r[t, :]^2) + eps)) * g
//
// HBM-bound streaming kernel, one wave per token row:
//  * the row is read once into registers (U 16-byte pieces per lane, lane i
//    taking bytes 16i.. of every KB), so X leaves HBM exactly once;
//  * the sum of squares runs in fp32, per lane in piece order, then across
//    the wave by an xor butterfly -- every pair adds the same two values, so
//    all lanes end with the same bits and the result repeats run to run;
//  * the scale is the hardware reciprocal square root of mean + eps (about
//    one ulp in fp32, far below the bf16 output step);
//  * y = (x * scale) * g in fp32, one round-to-nearest-even cast, 16-byte
//    stores into the gathered buffer.
#include <type_traits>

#include "tp_device.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int kNormThreads = 256;  // 4 waves = 4 rows per workgroup

template <typename T>
struct Vec;
template <>
struct Vec<bf16> {
  using V = bf16x8;
  static constexpr int E = 8;
};
template <>
struct Vec<float> {
  using V = floatx4;
  static constexpr int E = 4;
};

template <typename T, int U>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_gather_kernel(NormParams p) {
  using V = typename Vec<T>::V;
  constexpr int E = Vec<T>::E;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kNormThreads / 64) + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int64_t per = p.slice_rows;
  const int64_t r = p.slice >= 0 ? p.slice : row / per;  // rank (slice) of this row
  const int64_t t = p.slice >= 0 ? row : row - r * per;  // row within the slice
  const T* const x = static_cast<const T*>(p.X) + r * p.slice_stride + t * p.ldx;
  T* const y = static_cast<T*>(p.Y) + (r * per + t) * p.ldy;
  const T* const g = static_cast<const T*>(p.gamma);

  V v[U];
  float ss = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = (u * 64 + lane) * E;  // first element of this piece
    if (c < p.H) {
      v[u] = *reinterpret_cast<const V*>(x + c);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) v[u][e] = static_cast<T>(0.0f);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float f = static_cast<float>(v[u][e]);
      ss = fmaf(f, f, ss);
    }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  const float scale = __builtin_amdgcn_rsqf(ss * p.inv_h + p.eps);

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = (u * 64 + lane) * E;
    if (c < p.H) {
      const V gv = *reinterpret_cast<const V*>(g + c);
      V o;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float f = static_cast<float>(v[u][e]) * scale * static_cast<float>(gv[e]);
        if constexpr (std::is_same<T, bf16>::value)
          o[e] = to_bf16(f);
        else
          o[e] = f;
      }
      *reinterpret_cast<V*>(y + c) = o;
    }
  }
}

template <typename T>
hipError_t launch_typed(const NormParams& p, hipStream_t s) {
  constexpr int per_piece = 64 * Vec<T>::E;
  const int64_t pieces = (p.H + per_piece - 1) / per_piece;
  const dim3 g((unsigned)((p.rows + kNormThreads / 64 - 1) / (kNormThreads / 64))), b(kNormThreads);
#define TP_NORM_CASE(UU)                                                        \
  if (pieces <= UU) {                                                           \
    launch_kernel((rmsnorm_gather_kernel<T, UU>), g, b, 0u, s, p);              \
    return hipGetLastError();                                                   \
  }
  TP_NORM_CASE(1)
  TP_NORM_CASE(2)
  TP_NORM_CASE(4)
  TP_NORM_CASE(8)
  TP_NORM_CASE(16)
  TP_NORM_CASE(24)
  TP_NORM_CASE(32)
#undef TP_NORM_CASE
  return hipErrorInvalidValue;
}

}  // namespace

int64_t rmsnorm_max_hidden(bool bf16_io) { return 32 * 64 * (bf16_io ? 8 : 4); }

hipError_t launch_rmsnorm_gather(const NormParams& p, bool bf16_io, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  return bf16_io ? launch_typed<bf16>(p, s) : launch_typed<float>(p, s);
}

}  // namespace tp
