// Vocab-parallel cross-entropy after the output head.  The logits never
// reach memory: the GEMM's EPI_CE_STATS epilogue reduces each shard's logits
// to statistics per (token, 64-column chunk) -- max, sum of exp(l - max), and
// the label's logit when the chunk holds the label.  Then:
//   ce_fold_kernel     per (shard, token): the fold of its chunks, in order
//   ce_combine_kernel  per token: the fold over shards in shard order,
//                      loss = log S + M - target
//   ce_mean_kernel     the mean over tokens, in a fixed order
//   embed_partial_kernel  the input side: each shard's masked lookup of the
//                      token ids it owns (zero rows elsewhere)
//   embed_fold_kernel  the fold of those partials in shard order
// The blog post at 2kiu.com, section 6.2: each shard computes only its own
// vocab partition's logits and its part of the loss, an all-reduce combines
// them, and the vocab padding is left out of the loss.
//
// All are deterministic (fixed orders, no atomics).
#include <math.h>

#include "tp_device.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int kThreads = 256;

// Input side: one wave per (shard, token) row of the partial slab.  The
// shard that owns the token's id copies its embedding row; every other shard
// writes a row of -0.0, the additive identity of IEEE arithmetic (x + -0 is
// x for every x, a stored -0.0 included, where +0 would turn -0.0 into
// +0.0).  The partials keep the table's type (each holds table entries and
// signed zeros, so the fold's sums are exact in any precision).  Lane l
// moves the 16-byte vector l of each 1 KiB stretch: every load and store
// instruction of the wave covers one contiguous KiB.  Non-temporal stores:
// the slab is read once, by the fold.
template <typename E>
__global__ __launch_bounds__(kThreads) void embed_partial_kernel(EmbedParams p) {
  constexpr int VE = 16 / sizeof(E);
  typedef E ev __attribute__((ext_vector_type(VE)));
  constexpr int kRows = kThreads / kWave;
  const int64_t row = (int64_t)blockIdx.x * kRows + (threadIdx.x >> 6);
  if (row >= (int64_t)p.shards * p.T) return;  // whole waves leave together
  const int lane = lane_id();
  const int s = (int)(row / p.T);
  const int64_t t = row - (int64_t)s * p.T;
  const int64_t lo = (int64_t)(p.shard0 + s) * p.Vs, hi = min(lo + p.Vs, p.V);
  const int64_t id = p.ids[t];
  const bool own = id >= lo && id < hi;
  const E* const src = static_cast<const E*>(p.E) + (own ? id : 0) * p.H;
  E* const dst = static_cast<E*>(p.P) + (int64_t)s * p.sP + t * p.H;
  ev nz;
#pragma unroll
  for (int e = 0; e < VE; ++e) nz[e] = static_cast<E>(-0.0f);
#pragma unroll 4
  for (int64_t c = (int64_t)lane * VE; c < p.H; c += (int64_t)VE * kWave) {
    ev v = nz;
    if (own) v = *reinterpret_cast<const ev*>(src + c);
    __builtin_nontemporal_store(v, reinterpret_cast<ev*>(dst + c));
  }
}

// The embedding's all-reduce stand-in: thread i folds 16-byte vectors
// i + u * 256 (u < kFoldU, within its workgroup's span) of the N partials in
// shard order ((-0 + P0) + P1) + ... in fp32, then casts back to the table's
// type (exact: at most one term per element is not -0.0, and starting from
// -0.0 keeps the sign of a stored zero).  All loads of a group of 8 shards
// are issued before its adds.
constexpr int kFoldU = 4;

template <typename E>
__global__ __launch_bounds__(kThreads) void embed_fold_kernel(EmbedFoldParams p) {
  constexpr int VE = 16 / sizeof(E);
  typedef E ev __attribute__((ext_vector_type(VE)));
  const int64_t nv = p.n / VE;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kFoldU + threadIdx.x;
  const E* const src = static_cast<const E*>(p.P);
  float acc[kFoldU][VE];
#pragma unroll
  for (int u = 0; u < kFoldU; ++u)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[u][e] = -0.0f;
  for (int k0 = 0; k0 < p.N; k0 += 8) {
    ev v[8][kFoldU];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int u = 0; u < kFoldU; ++u) {
        const int64_t i = base + u * kThreads;
        if (k0 + k < p.N && i < nv)
          v[k][u] = __builtin_nontemporal_load(reinterpret_cast<const ev*>(src + (k0 + k) * p.sP + i * VE));
      }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k0 + k < p.N)
#pragma unroll
        for (int u = 0; u < kFoldU; ++u)
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[u][e] += static_cast<float>(v[k][u][e]);
  }
#pragma unroll
  for (int u = 0; u < kFoldU; ++u) {
    const int64_t i = base + u * kThreads;
    if (i < nv) {
      ev o;
#pragma unroll
      for (int e = 0; e < VE; ++e) o[e] = static_cast<E>(acc[u][e]);
      *reinterpret_cast<ev*>(static_cast<E*>(p.Y) + i * VE) = o;
    }
  }
}

// One thread per (shard, token): the fold of the shard's 64-column chunk
// statistics in chunk order (consecutive threads read consecutive tokens).
__global__ __launch_bounds__(kThreads) void ce_fold_kernel(CeFoldParams p) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)p.shards * p.T) return;
  const int s = (int)(i / p.T);
  const int64_t t = i - (int64_t)s * p.T;
  const float* const m = p.stats + (int64_t)s * p.cps * p.T + t;
  MaxSum acc = {-INFINITY, 0.0f};
  float z = 0.0f;
#pragma unroll 4
  for (int k = 0; k < p.cps; ++k) {
    const int64_t o = (int64_t)k * p.T;
    acc = ms_merge(acc, {m[o], m[o + p.astride]});
    z += m[o + 2 * p.astride];
  }
  const int64_t slot = (int64_t)(p.shard0 + s) * p.T + t;
  p.m[slot] = acc.m;
  p.s[slot] = acc.s;
  p.z[slot] = z;
}

// One thread per token: the fold over the N shards' statistics in order.
__global__ __launch_bounds__(kThreads) void ce_combine_kernel(CeCombineParams p) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= p.T) return;
  MaxSum acc = {p.m[t], p.s[t]};
  float target = p.z[t];
  for (int i = 1; i < p.N; ++i) {
    const int64_t slot = (int64_t)i * p.T + t;
    acc = ms_merge(acc, {p.m[slot], p.s[slot]});
    target += p.z[slot];
  }
  p.loss[t] = logf(acc.s) + acc.m - target;
}

// One workgroup: thread j adds tokens j, j + 256, ... in order, then a fixed
// tree over the 256 partial sums.
__global__ __launch_bounds__(kThreads) void ce_mean_kernel(const float* loss, int64_t T, float* mean) {
  __shared__ float part[kThreads];
  float acc = 0.0f;
  for (int64_t t = threadIdx.x; t < T; t += kThreads) acc += loss[t];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kThreads / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *mean = part[0] / (float)T;
}

}  // namespace

hipError_t launch_embed_partial(const EmbedParams& p, bool f32, hipStream_t s) {
  constexpr int kRows = kThreads / kWave;
  const int64_t grid = ((int64_t)p.shards * p.T + kRows - 1) / kRows;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (f32)
    launch_kernel(embed_partial_kernel<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  else
    launch_kernel(embed_partial_kernel<bf16>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_embed_fold(const EmbedFoldParams& p, bool f32, hipStream_t s) {
  const int64_t vecs = p.n / (f32 ? 4 : 8);
  const int64_t grid = (vecs + kThreads * kFoldU - 1) / (kThreads * kFoldU);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (f32)
    launch_kernel(embed_fold_kernel<float>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  else
    launch_kernel(embed_fold_kernel<bf16>, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_ce_fold(const CeFoldParams& p, hipStream_t s) {
  const int64_t grid = ((int64_t)p.shards * p.T + kThreads - 1) / kThreads;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  launch_kernel(ce_fold_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_ce_combine(const CeCombineParams& p, hipStream_t s) {
  const int64_t grid = (p.T + kThreads - 1) / kThreads;
  if (grid <= 0) return hipSuccess;
  launch_kernel(ce_combine_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_ce_mean(const float* loss, int64_t T, float* mean, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  launch_kernel(ce_mean_kernel, dim3(1), dim3(kThreads), 0, s, loss, T, mean);
  return hipGetLastError();
}

}  // namespace tp
