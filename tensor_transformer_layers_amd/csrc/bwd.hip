// Layout kernels of the MLP pair's backward: a tiled transpose (optionally
// applying GELU to a stored pre-activation on the way) and a fixed-order row
// sum for the bias gradients.
//
// The backward's contractions over the token axis (weight gradients
// dA = X^T dZ and dB = H^T dY) and over the output axis of a weight (dH =
// dY B, dX = dZ A) need operands that are contiguous along the contraction.
// The GEMM kernel reads both operands K-contiguous, so each operand that is
// not is transposed once into the workspace: HBM-bound copies, a few percent
// of the backward's time at the large workloads.
//
// Both kernels are deterministic (no atomics, fixed summation order).
#include "tp_device.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;          // 64 x 64 elements per workgroup
constexpr int kPitch = kTile + 8;  // LDS row pitch in elements: rows stay 16-byte aligned

// Thread t moves 16-byte chunk (t & 7) of tile rows (t >> 3) and (t >> 3) + 32:
// 8 lanes cover one 128-byte row segment, in and out.  The tile is written
// to LDS transposed (element by element) and read back in 16-byte rows.
template <bool GELU>
__global__ __launch_bounds__(kThreads) void transpose_kernel(TransposeParams p, int tilesC) {
  __shared__ __attribute__((aligned(16))) bf16 tile[kTile * kPitch];
  const int tr = (int)blockIdx.x / tilesC, tc = (int)blockIdx.x % tilesC;
  const int64_t r0 = (int64_t)tr * kTile, c0 = (int64_t)tc * kTile;
  const int chunk = threadIdx.x & 7, rr = threadIdx.x >> 3;
  const bf16* const in = static_cast<const bf16*>(p.in);
  bf16x8 v[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // both loads in flight before any LDS write
    const int64_t gr = r0 + rr + 32 * j, gc = c0 + chunk * 8;
    v[j] = bf16x8{};
    if (gr < p.R && gc < p.C) v[j] = *reinterpret_cast<const bf16x8*>(in + gr * p.ld_in + gc);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16 x = v[j][e];
      if constexpr (GELU) x = to_bf16(gelu_bf16out(static_cast<float>(x)));
      tile[(chunk * 8 + e) * kPitch + rr + 32 * j] = x;
    }
  __syncthreads();
  bf16* const out = static_cast<bf16*>(p.out);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int oc = rr + 32 * j;  // output row c0 + oc = input column
    const int64_t go = c0 + oc, gi = r0 + chunk * 8;
    if (go < p.C && gi < p.R)
      *reinterpret_cast<bf16x8*>(out + go * p.ld_out + gi) =
          *reinterpret_cast<const bf16x8*>(&tile[oc * kPitch + chunk * 8]);
  }
}

// One wave per row: lane l adds elements 8l .. 8l+7 of each 512-element
// stretch, stretches in order, then an xor butterfly combines the lanes.
// The order is fixed, so the sums are bit-identical run to run.
constexpr int kRowsPerBlock = kThreads / kWave;

__global__ __launch_bounds__(kThreads) void rowsum_kernel(RowSumParams p) {
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= p.R) return;  // whole waves leave together
  const int lane = lane_id();
  const bf16* const row = static_cast<const bf16*>(p.in) + r * p.ld;
  float acc = 0.0f;
#pragma unroll 4
  for (int64_t c = lane * 8; c < p.C; c += 8 * kWave) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(row + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += static_cast<float>(v[e]);
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) p.out[r] = acc;
}

}  // namespace

hipError_t launch_transpose(const TransposeParams& p, bool gelu, hipStream_t s) {
  const int64_t tilesR = (p.R + kTile - 1) / kTile, tilesC = (p.C + kTile - 1) / kTile;
  const int64_t grid = tilesR * tilesC;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (gelu)
    launch_kernel(transpose_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s, p, (int)tilesC);
  else
    launch_kernel(transpose_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s, p, (int)tilesC);
  return hipGetLastError();
}

hipError_t launch_rowsum(const RowSumParams& p, hipStream_t s) {
  const int64_t grid = (p.R + kRowsPerBlock - 1) / kRowsPerBlock;
  if (grid <= 0) return hipSuccess;
  launch_kernel(rowsum_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace tp
