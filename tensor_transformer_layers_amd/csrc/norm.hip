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
// HBM-bound streaming kernel, one to four waves per token row (wide rows are
// split so that each wave holds at most 8 KB of its row and enough waves stay
// resident to keep HBM busy):
//  * the row is read once into registers (U 16-byte pieces per lane, lane i
//    taking bytes 16i.. of every KB of its wave's part), so X leaves HBM
//    exactly once;
//  * the sum of squares runs in fp32, per lane in piece order, then across
//    the wave by an xor butterfly -- every pair adds the same two values, so
//    all lanes end with the same bits -- then, for split rows, over the
//    row's waves in wave order through LDS; the result repeats run to run;
//  * the scale is the hardware reciprocal square root of mean + eps (about
//    one ulp in fp32, far below the bf16 output step);
//  * y = (x * scale) * g in fp32, one round-to-nearest-even cast, 16-byte
//    stores into the gathered buffer.
#include <type_traits>

#include "tp_device.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {


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

template <typename T, int U, int WPR, int NT>
__global__ __launch_bounds__(NT) void rmsnorm_gather_kernel(NormParams p) {
  using V = typename Vec<T>::V;
  constexpr int E = Vec<T>::E;
  constexpr int kRows = NT / 64 / WPR;  // rows per workgroup
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int part = wv % WPR;  // which part of its row this wave holds
  const int64_t row = (int64_t)blockIdx.x * kRows + wv / WPR;
  if (WPR == 1 && row >= p.rows) return;  // split rows keep every wave for the barrier
  const bool live = row < p.rows;
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
    const int c = ((part * U + u) * 64 + lane) * E;  // first element of this piece
    if (live && c < p.H) {
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
  if constexpr (WPR > 1) {
    __shared__ float part_ss[NT / 64];
    if (lane == 0) part_ss[wv] = ss;
    __syncthreads();
    const int w0 = wv - part;
    ss = part_ss[w0];
#pragma unroll
    for (int k = 1; k < WPR; ++k) ss += part_ss[w0 + k];
  }
  const float scale = __builtin_amdgcn_rsqf(ss * p.inv_h + p.eps);

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = ((part * U + u) * 64 + lane) * E;
    if (live && c < p.H) {
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

template <typename T, int U, int WPR, int NT = 256>
hipError_t launch_shape(const NormParams& p, hipStream_t s) {
  constexpr int kRows = NT / 64 / WPR;
  const dim3 g((unsigned)((p.rows + kRows - 1) / kRows)), b(NT);
  launch_kernel((rmsnorm_gather_kernel<T, U, WPR, NT>), g, b, 0u, s, p);
  return hipGetLastError();
}

// pieces = 1 KB pieces of a row; rows of more than 2 pieces are split over
// 2 to 8 waves (at most 4 pieces, 16 registers of row data, per wave)
template <typename T>
hipError_t launch_typed(const NormParams& p, hipStream_t s) {
  constexpr int per_piece = 64 * Vec<T>::E;
  const int64_t pieces = (p.H + per_piece - 1) / per_piece;
  if (pieces <= 1) return launch_shape<T, 1, 1>(p, s);
  if (pieces <= 2) return launch_shape<T, 2, 1>(p, s);
  if (pieces <= 4) return launch_shape<T, 2, 2>(p, s);
  if (pieces <= 8) return launch_shape<T, 2, 4>(p, s);
  if (pieces <= 16) return launch_shape<T, 4, 4>(p, s);
  if (pieces <= 24) return launch_shape<T, 3, 8, 512>(p, s);
  if (pieces <= 32) return launch_shape<T, 4, 8, 512>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

int64_t rmsnorm_max_hidden(bool bf16_io) { return 32 * 64 * (bf16_io ? 8 : 4); }

hipError_t launch_rmsnorm_gather(const NormParams& p, bool bf16_io, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  return bf16_io ? launch_typed<bf16>(p, s) : launch_typed<float>(p, s);
}

}  // namespace tp
