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

// Thread t moves 16-byte chunk (t % CH) of tile rows (t / CH) + (256 / CH) j,
// CH = the chunks per 64-element row (8 for bf16, 16 for fp32): the lanes of
// a row cover one contiguous row segment, in and out.  The tile is written to
// LDS transposed (element by element) and read back in 16-byte rows.  With
// GELU, the activation is applied on the way (fp32: erf form with the device
// erff; bf16: the 7.1.26 form, rounded to bf16).
template <typename E, bool GELU>
__global__ __launch_bounds__(kThreads) void transpose_kernel(TransposeParams p, int tilesC) {
  constexpr int VE = 16 / sizeof(E);                     // elements per 16-byte chunk
  constexpr int CH = kTile / VE;                         // chunks per tile row
  constexpr int PITCH = kTile + VE;                      // 16-byte aligned LDS rows
  constexpr int RSTEP = kThreads / CH, NJ = kTile / RSTEP;
  typedef E ev __attribute__((ext_vector_type(VE)));
  __shared__ __attribute__((aligned(16))) E tile[kTile * PITCH];
  const int tr = (int)blockIdx.x / tilesC, tc = (int)blockIdx.x % tilesC;
  const int64_t r0 = (int64_t)tr * kTile, c0 = (int64_t)tc * kTile;
  const int chunk = threadIdx.x % CH, rr = threadIdx.x / CH;
  const E* const in = static_cast<const E*>(p.in);
  ev v[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {  // every load in flight before any LDS write
    const int64_t gr = r0 + rr + RSTEP * j, gc = c0 + chunk * VE;
    v[j] = ev{};
    if (gr < p.R && gc < p.C) v[j] = *reinterpret_cast<const ev*>(in + gr * p.ld_in + gc);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      E x = v[j][e];
      if constexpr (GELU) {
        if constexpr (sizeof(E) == 4)
          x = gelu_erf(x);
        else
          x = to_bf16(gelu_bf16out(static_cast<float>(x)));
      }
      tile[(chunk * VE + e) * PITCH + rr + RSTEP * j] = x;
    }
  __syncthreads();
  E* const out = static_cast<E*>(p.out);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int oc = rr + RSTEP * j;  // output row c0 + oc = input column
    const int64_t go = c0 + oc, gi = r0 + chunk * VE;
    if (go < p.C && gi < p.R)
      *reinterpret_cast<ev*>(out + go * p.ld_out + gi) = *reinterpret_cast<const ev*>(&tile[oc * PITCH + chunk * VE]);
  }
}

// One wave per row: lane l adds elements 8l .. 8l+7 of each 512-element
// stretch, stretches in order, then an xor butterfly combines the lanes.
// The order is fixed, so the sums are bit-identical run to run.
constexpr int kRowsPerBlock = kThreads / kWave;

template <typename E>
__global__ __launch_bounds__(kThreads) void rowsum_kernel(RowSumParams p) {
  constexpr int VE = 16 / sizeof(E);
  typedef E ev __attribute__((ext_vector_type(VE)));
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= p.R) return;  // whole waves leave together
  const int lane = lane_id();
  const E* const row = static_cast<const E*>(p.in) + r * p.ld;
  float acc = 0.0f;
#pragma unroll 4
  for (int64_t c = lane * VE; c < p.C; c += VE * kWave) {
    const ev v = *reinterpret_cast<const ev*>(row + c);
#pragma unroll
    for (int e = 0; e < VE; ++e) acc += static_cast<float>(v[e]);
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) p.out[r] = acc;
}

}  // namespace

hipError_t launch_transpose(const TransposeParams& p, bool gelu, bool f32, hipStream_t s) {
  const int64_t tilesR = (p.R + kTile - 1) / kTile, tilesC = (p.C + kTile - 1) / kTile;
  const int64_t grid = tilesR * tilesC;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(kThreads);
  if (f32 && gelu)
    launch_kernel(transpose_kernel<float, true>, g, b, 0, s, p, (int)tilesC);
  else if (f32)
    launch_kernel(transpose_kernel<float, false>, g, b, 0, s, p, (int)tilesC);
  else if (gelu)
    launch_kernel(transpose_kernel<bf16, true>, g, b, 0, s, p, (int)tilesC);
  else
    launch_kernel(transpose_kernel<bf16, false>, g, b, 0, s, p, (int)tilesC);
  return hipGetLastError();
}

hipError_t launch_rowsum(const RowSumParams& p, bool f32, hipStream_t s) {
  const int64_t grid = (p.R + kRowsPerBlock - 1) / kRowsPerBlock;
  if (grid <= 0) return hipSuccess;
  if (f32)
    launch_kernel(rowsum_kernel<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  else
    launch_kernel(rowsum_kernel<bf16>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace tp
