// The all-reduce stand-in: fixed-order fp32 fold of the N row partials, bias
// added once after the sum, one round-to-nearest-even cast.
//
// Row split, 2kiu.com blog post section 2.2 (the partials are summed
// elementwise) and "张量并行" (row-split equation XB = X1B1 + X2B2); bias once
// after the all-reduce: listing of "Tensor Parallelism基础：模型切分原理".
// Reduce-scatter along the sequence (one contiguous row block per rank):
// "张量并行", Megatron-SP section; blog post section 4.3.
//
// HBM-bound streaming kernel.  Thread t of a block owns 4 consecutive outputs
// in each of U consecutive 1024-float stretches, so every load and store
// instruction of a wave covers one contiguous span (1 KB of fp32 per load).
// All N*U partial loads are issued before the adds, which run strictly in
// shard order ((P0 + P1) + P2) + ... as plain fp32 adds (no FMA can form:
// there are no multiplies); then the bias, one RNE cast, and an 8-byte (bf16)
// or 16-byte (fp32) store per stretch.  The partials are read exactly once
// (non-temporal loads).  Grid-stride over the [rows x H] region; no atomics,
// so the result is bit-identical run to run.  Each thread owns U = 4 stretches,
// and the grid covers the region in one trip.
#include "tp_device.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ floatx4 ld_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
}

constexpr int kU = 4;  // 16-byte stretches per thread per trip

template <bool OUT_BF16, int NP, bool STRIDED = false>
__global__ __launch_bounds__(kThreads) void reduce_kernel(ReduceParams p, int64_t n4) {
  const int np = NP > 0 ? NP : p.n_parts;
  const float* const src0 = p.P + p.row0 * p.H;
  const int64_t step = (int64_t)gridDim.x * kThreads * kU;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kU + threadIdx.x; base < n4; base += step) {
    floatx4 acc[kU];
    bool ok[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      ok[u] = base + u * kThreads < n4;
      acc[u] = ok[u] ? ld_nt(src0 + (base + u * kThreads) * 4) : floatx4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (NP > 0) {
      floatx4 part[NP > 1 ? NP - 1 : 1][kU];
#pragma unroll
      for (int k = 1; k < NP; ++k)  // issue every load first ...
#pragma unroll
        for (int u = 0; u < kU; ++u)
          part[k - 1][u] = ok[u] ? ld_nt(src0 + k * p.part_stride + (base + u * kThreads) * 4)
                                 : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 1; k < NP; ++k)  // ... then add strictly in shard order
#pragma unroll
        for (int u = 0; u < kU; ++u) acc[u] += part[k - 1][u];
    } else {
      for (int k = 1; k < np; ++k)
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (ok[u]) acc[u] += ld_nt(src0 + k * p.part_stride + (base + u * kThreads) * 4);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (!ok[u]) continue;
      const int64_t e = (base + u * kThreads) * 4;
      if (p.bias) {
        const int64_t c = e % p.H;  // H is a multiple of 4: the 4 outputs share a row
        if constexpr (OUT_BF16) {
          const bf16x4 b = *reinterpret_cast<const bf16x4*>(static_cast<const bf16*>(p.bias) + c);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[u][j] += static_cast<float>(b[j]);
        } else {
          acc[u] += *reinterpret_cast<const floatx4*>(static_cast<const float*>(p.bias) + c);
        }
      }
      // output rows of width H at pitch ldy (the 4 outputs share a row)
      const int64_t eo = STRIDED ? (e / p.H) * p.ldy + e % p.H : e;
      if constexpr (OUT_BF16) {
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = to_bf16(acc[u][j]);
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.Y) + eo) = o;
      } else {
        *reinterpret_cast<floatx4*>(static_cast<float*>(p.Y) + eo) = acc[u];
      }
    }
  }
}

template <bool OUT_BF16>
hipError_t launch_typed(const ReduceParams& p, hipStream_t s) {
  const int64_t n4 = p.rows * p.H / 4;
  if (n4 <= 0) return hipSuccess;
  // one trip per workgroup: short-lived workgroups streaming 16 KB of each
  // partial keep more requests in flight than a capped grid-stride grid
  // (measured on the 8-partial workloads); the loop stays for grids at the cap
  const int64_t per_block = (int64_t)kThreads * kU;
  const int64_t blocks = std::min<int64_t>((n4 + per_block - 1) / per_block, int64_t(1) << 30);
  const dim3 g((unsigned)blocks), b(kThreads);
  if (p.ldy != p.H) {  // pitched output rows (a block of a wider matrix)
    if (p.n_parts == 16)
      launch_kernel((reduce_kernel<OUT_BF16, 16, true>), g, b, 0, s, p, n4);
    else
      launch_kernel((reduce_kernel<OUT_BF16, 0, true>), g, b, 0, s, p, n4);
    return hipGetLastError();
  }
  switch (p.n_parts) {
    case 1: launch_kernel((reduce_kernel<OUT_BF16, 1>), g, b, 0, s, p, n4); break;
    case 2: launch_kernel((reduce_kernel<OUT_BF16, 2>), g, b, 0, s, p, n4); break;
    case 4: launch_kernel((reduce_kernel<OUT_BF16, 4>), g, b, 0, s, p, n4); break;
    case 8: launch_kernel((reduce_kernel<OUT_BF16, 8>), g, b, 0, s, p, n4); break;
    case 16: launch_kernel((reduce_kernel<OUT_BF16, 16>), g, b, 0, s, p, n4); break;
    default: launch_kernel((reduce_kernel<OUT_BF16, 0>), g, b, 0, s, p, n4); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const ReduceParams& p, bool out_bf16, hipStream_t s) {
  return out_bf16 ? launch_typed<true>(p, s) : launch_typed<false>(p, s);
}

}  // namespace tp
