// The all-reduce stand-in: fixed-order fp32 fold of the N row partials, bias
// added once after the sum, one round-to-nearest-even cast.
//
// Row split, 2kiu.com blog post section 2.2 (the partials are summed
// elementwise) and "张量并行" (row-split equation XB = X1B1 + X2B2); bias once
// after the all-reduce: listing of "Tensor Parallelism基础：模型切分原理".
// Reduce-scatter along the sequence (one contiguous row block per rank):
// "张量并行", Megatron-SP section; blog post section 4.3.
//
// HBM-bound streaming kernel: every thread owns 8 consecutive outputs, reads
// them from each partial with two 16-byte non-temporal loads (the partials are
// read exactly once), adds the partials strictly in shard order
// ((P0 + P1) + P2) + ... with plain fp32 adds (no FMA can form: there are no
// multiplies), adds the bias, and writes 16 (bf16) or 32 (fp32) contiguous
// bytes.  Grid-stride over the [rows x H] region; no atomics, so the result is
// bit-identical run to run.
#include "tp_device.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ floatx4 ld_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
}

template <bool OUT_BF16, int NP>
__global__ __launch_bounds__(kThreads) void reduce_kernel(ReduceParams p, int64_t n8) {
  const int np = NP > 0 ? NP : p.n_parts;
  const float* const src0 = p.P + p.row0 * p.H;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < n8; g += stride) {
    const int64_t e = g * 8;
    const float* s = src0 + e;
    floatx4 lo = ld_nt(s), hi = ld_nt(s + 4);
    if constexpr (NP > 0) {
      floatx4 plo[NP > 1 ? NP - 1 : 1], phi[NP > 1 ? NP - 1 : 1];
#pragma unroll
      for (int k = 1; k < NP; ++k) {  // issue every load first ...
        plo[k - 1] = ld_nt(s + k * p.part_stride);
        phi[k - 1] = ld_nt(s + k * p.part_stride + 4);
      }
#pragma unroll
      for (int k = 1; k < NP; ++k) {  // ... then add strictly in shard order
        lo += plo[k - 1];
        hi += phi[k - 1];
      }
    } else {
      for (int k = 1; k < np; ++k) {
        lo += ld_nt(s + k * p.part_stride);
        hi += ld_nt(s + k * p.part_stride + 4);
      }
    }
    if (p.bias) {
      const int64_t c = e % p.H;  // H is a multiple of 8: the 8 outputs share a row
      if constexpr (OUT_BF16) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p.bias) + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo[j] += static_cast<float>(b[j]);
          hi[j] += static_cast<float>(b[j + 4]);
        }
      } else {
        const float* b = static_cast<const float*>(p.bias) + c;
        lo += *reinterpret_cast<const floatx4*>(b);
        hi += *reinterpret_cast<const floatx4*>(b + 4);
      }
    }
    if constexpr (OUT_BF16) {
      bf16x8 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[j] = to_bf16(lo[j]);
        o[j + 4] = to_bf16(hi[j]);
      }
      *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p.Y) + e) = o;
    } else {
      float* y = static_cast<float*>(p.Y) + e;
      *reinterpret_cast<floatx4*>(y) = lo;
      *reinterpret_cast<floatx4*>(y + 4) = hi;
    }
  }
}

template <bool OUT_BF16>
hipError_t launch_typed(const ReduceParams& p, hipStream_t s) {
  const int64_t n8 = p.rows * p.H / 8;
  if (n8 <= 0) return hipSuccess;
  // enough resident waves to keep ~8 x 32 bytes per lane in flight on every CU;
  // beyond that the grid-stride loop takes over
  const int64_t blocks = std::min<int64_t>((n8 + kThreads - 1) / kThreads, 256 * 16);
  const dim3 g((unsigned)blocks), b(kThreads);
  switch (p.n_parts) {
    case 1: hipLaunchKernelGGL((reduce_kernel<OUT_BF16, 1>), g, b, 0, s, p, n8); break;
    case 2: hipLaunchKernelGGL((reduce_kernel<OUT_BF16, 2>), g, b, 0, s, p, n8); break;
    case 4: hipLaunchKernelGGL((reduce_kernel<OUT_BF16, 4>), g, b, 0, s, p, n8); break;
    case 8: hipLaunchKernelGGL((reduce_kernel<OUT_BF16, 8>), g, b, 0, s, p, n8); break;
    default: hipLaunchKernelGGL((reduce_kernel<OUT_BF16, 0>), g, b, 0, s, p, n8); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const ReduceParams& p, bool out_bf16, hipStream_t s) {
  return out_bf16 ? launch_typed<true>(p, s) : launch_typed<false>(p, s);
}

}  // namespace tp
