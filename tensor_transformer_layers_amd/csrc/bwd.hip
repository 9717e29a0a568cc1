// Layout and reduction kernels of the MLP pair's backward: a tiled transpose
// (optionally applying GELU to a stored pre-activation on the way), a
// fixed-order row sum, and a fixed-order column sum for the bias gradients.
//
// The backward's contractions over the token axis (weight gradients
// dA = dZ^T X and dB = dY^T H) and over the output axis of a weight (dH =
// dY B, dX = dZ A) read operands that are not contiguous along the
// contraction.  The bf16 GEMM reads such operands as stored (K-outer, through
// the transposing LDS read); the fp32 path, and shapes the K-outer GEMM does
// not take, transpose them once into the workspace instead: HBM-bound copies.
// The bias gradients are then row sums of the transposed dZ and dY, or
// column sums of the untransposed ones.
//
// All kernels are deterministic (no atomics, fixed summation order).
#include <algorithm>

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
// erff; bf16: gelu_bf16out, rounded to bf16).
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

// Column sums: a workgroup sums a strip of 16*VE columns (VE elements per 16
// bytes) over one chunk of rows.  One launch serves up to two independent
// sums (the backward's two bias gradients): workgroups [0, j0.groups) take
// the first, the rest the second.  Lane l owns columns VE*(l % 16) .. +VE-1 of
// the strip; wave w takes rows 4w + l/16 + 16j of the chunk (each load
// instruction covers four 256-byte row segments), eight rows in flight per
// lane.  Lanes l, l^16, l^32, l^48 then fold by an xor butterfly and the four
// waves' sums add in wave order through LDS; the chunks' partials are folded
// by a second launch of the same kernel over the fp32 partial matrices.  Every
// order is fixed, so the sums are bit-identical run to run, and a sum's bits
// do not depend on whether it shares its launches with another.
constexpr int kColsumTargetGroups = 1024;  // ~4 per CU: enough loads in flight to stream from HBM
constexpr int kColsumMaxChunks = 128;      // bounds the fold's depth
constexpr int kColsumMinRows = 128;        // one full unrolled trip per wave

// One column sum of a launch: in [R x C] (row pitch ld), rows_per_chunk rows
// per chunk, strips strips of columns, groups = strips x chunks workgroups,
// chunk k's sums to dst + k C.
struct ColsumJob {
  const void* in;
  int64_t ld, R, C, rows_per_chunk;
  int strips, groups;
  float* dst;
};

template <typename E>
__global__ __launch_bounds__(kThreads) void colsum_kernel(ColsumJob j0, ColsumJob j1) {
  constexpr int VE = 16 / sizeof(E);
  constexpr int SW = 16 * VE;  // columns per strip
  constexpr int U = 8;         // rows in flight per lane
  typedef E ev __attribute__((ext_vector_type(VE)));
  __shared__ __attribute__((aligned(16))) float red[kThreads / kWave][SW];
  const bool second = (int)blockIdx.x >= j0.groups;
  const ColsumJob& j = second ? j1 : j0;
  const int bid = second ? (int)blockIdx.x - j0.groups : (int)blockIdx.x;
  const E* const in = static_cast<const E*>(j.in);
  const int64_t ld = j.ld, R = j.R, C = j.C, rows_per_chunk = j.rows_per_chunk;
  const int strips = j.strips;
  float* const dst = j.dst;
  const int strip = bid % strips, chunk = bid / strips;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int64_t c = (int64_t)strip * SW + (lane & 15) * VE;
  const int64_t r0 = (int64_t)chunk * rows_per_chunk;
  const int64_t r1 = min(R, r0 + rows_per_chunk);
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.0f;
  if (c < C) {
    const E* const col = in + c;
    int64_t r = r0 + 4 * w + (lane >> 4);
    for (; r + 16 * (U - 1) < r1; r += 16 * U) {
      ev v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const ev*>(col + (r + 16 * u) * ld);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] += static_cast<float>(v[u][e]);
    }
    for (; r < r1; r += 16) {
      const ev v = *reinterpret_cast<const ev*>(col + r * ld);
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] += static_cast<float>(v[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    acc[e] += __shfl_xor(acc[e], 16);
    acc[e] += __shfl_xor(acc[e], 32);
  }
  if (lane < 16)
#pragma unroll
    for (int e = 0; e < VE; ++e) red[w][(lane & 15) * VE + e] = acc[e];
  __syncthreads();
  if (w == 0 && lane < 16 && c < C) {
    float* const out = dst + (int64_t)chunk * C + c;
#pragma unroll
    for (int e0 = 0; e0 < VE; e0 += 4) {
      floatx4 s;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = (lane & 15) * VE + e0 + e;
        s[e] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
      }
      *reinterpret_cast<floatx4*>(out + e0) = s;
    }
  }
}

// Rows per chunk of the first column-sum pass over [R x C]: about
// kColsumTargetGroups workgroups, at most kColsumMaxChunks chunks of at least
// kColsumMinRows rows, a multiple of 16 rows.
int64_t colsum_rows_per_chunk(int64_t R, int64_t C) {
  const int64_t strips = (C + 127) / 128;
  int64_t chunks = (kColsumTargetGroups + strips - 1) / strips;
  chunks = std::min<int64_t>(chunks, kColsumMaxChunks);
  chunks = std::min<int64_t>(chunks, (R + kColsumMinRows - 1) / kColsumMinRows);
  chunks = std::max<int64_t>(chunks, 1);
  const int64_t rpc = (R + chunks - 1) / chunks;
  return (rpc + 15) / 16 * 16;
}

int64_t colsum_chunk_count(int64_t R, int64_t C) {
  const int64_t rpc = colsum_rows_per_chunk(R, C);
  return (R + rpc - 1) / rpc;
}

}  // namespace

size_t colsum_part_floats(int64_t R, int64_t C) {
  return R > 0 && C > 0 ? (size_t)colsum_chunk_count(R, C) * (size_t)C : 0;
}

namespace {

// The jobs of the two launches of up to two column sums: the chunk sums, and
// the fold of the chunks' partials (fp32 [chunks x C]) in chunk order (one
// chunk of all rows).  A job with no workgroups is never selected.
hipError_t colsum_jobs(const ColSumParams* ps, int n, ColsumJob (&sums)[2], ColsumJob (&folds)[2], int64_t& g1,
                       int64_t& g2) {
  if (n < 0 || n > 2) return hipErrorInvalidValue;
  sums[0] = sums[1] = folds[0] = folds[1] = ColsumJob{};
  g1 = g2 = 0;
  int k = 0;
  for (int i = 0; i < n; ++i) {
    const ColSumParams& p = ps[i];
    if (p.R <= 0 || p.C <= 0) continue;
    if (p.C % 8) return hipErrorInvalidValue;
    const int64_t rpc = colsum_rows_per_chunk(p.R, p.C), chunks = colsum_chunk_count(p.R, p.C);
    const int64_t strips1 = (p.C + 127) / 128, strips2 = (p.C + 63) / 64;
    if (strips1 * chunks > 0x3fffffff || strips2 > 0x3fffffff) return hipErrorInvalidValue;
    sums[k] = ColsumJob{p.in, p.ld, p.R, p.C, rpc, (int)strips1, (int)(strips1 * chunks), p.part};
    folds[k] = ColsumJob{p.part, p.C, chunks, p.C, chunks, (int)strips2, (int)strips2, p.out};
    g1 += strips1 * chunks;
    g2 += strips2;
    ++k;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_colsum_chunks(const ColSumParams* ps, int n, hipStream_t s) {
  ColsumJob sums[2], folds[2];
  int64_t g1, g2;
  const hipError_t e = colsum_jobs(ps, n, sums, folds, g1, g2);
  if (e != hipSuccess || g1 == 0) return e;
  launch_kernel(colsum_kernel<bf16>, dim3((unsigned)g1), dim3(kThreads), 0, s, sums[0], sums[1]);
  return hipGetLastError();
}

hipError_t launch_colsum_fold(const ColSumParams* ps, int n, hipStream_t s) {
  ColsumJob sums[2], folds[2];
  int64_t g1, g2;
  const hipError_t e = colsum_jobs(ps, n, sums, folds, g1, g2);
  if (e != hipSuccess || g2 == 0) return e;
  launch_kernel(colsum_kernel<float>, dim3((unsigned)g2), dim3(kThreads), 0, s, folds[0], folds[1]);
  return hipGetLastError();
}

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
