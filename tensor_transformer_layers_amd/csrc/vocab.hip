// Vocab-parallel cross-entropy after the output head (the logits of each
// shard's vocab partition come from the GEMM kernel):
//   ce_stats_kernel    per (shard, token): max, sum of exp(l - max) over the
//                      shard's real vocab entries, and the label's logit when
//                      the shard owns the label
//   ce_combine_kernel  per token: the fold over shards in shard order,
//                      loss = log S + M - target
//   ce_mean_kernel     the mean over tokens, in a fixed order
// The blog post at 2kiu.com, section 6.2: each shard computes only its own
// vocab partition's logits and its part of the loss, an all-reduce combines
// them, and the vocab padding is left out of the loss.
//
// All three are deterministic (fixed orders, no atomics).  ce_stats_kernel is
// HBM-bound (each fp32 logit read once, one exponential per logit).
#include <math.h>

#include "tp_device.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

// Running (max, sum of exp(x - max)) pairs.  A pair with max = -inf holds
// nothing (sum 0); the scale of a side is 1 when it holds the new max, so
// -inf never meets -inf in an exponential.
struct MaxSum {
  float m, s;
};

__device__ __forceinline__ MaxSum ms_merge(MaxSum a, MaxSum b) {
  const float mx = fmaxf(a.m, b.m);
  const float sa = a.m == mx ? a.s : a.s * __expf(a.m - mx);
  const float sb = b.m == mx ? b.s : b.s * __expf(b.m - mx);
  return {mx, sa + sb};
}

__device__ __forceinline__ MaxSum ms_add(MaxSum a, float x) {
  if (x > a.m) return {x, a.s * __expf(a.m - x) + 1.0f};  // a.m = -inf: a.s = 0
  return {a.m, a.s + __expf(x - a.m)};
}

// One wave per (shard, token) row of logits.  Lane l takes the 16-byte
// pieces l, l + 64, ... of the row's real entries in order, then an xor
// butterfly merges the lanes.
__global__ __launch_bounds__(kThreads) void ce_stats_kernel(CeStatsParams p) {
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= (int64_t)p.shards * p.T) return;  // whole waves leave together
  const int lane = lane_id();
  const int s = (int)(row / p.T);
  const int64_t t = row - (int64_t)s * p.T;
  const int64_t base = (int64_t)(p.shard0 + s) * p.Vs;  // first vocab id of the shard
  const int64_t valid = min((int64_t)p.Vs, max((int64_t)0, p.V - base));
  const float* const L = p.logits + (int64_t)s * p.sL + t * p.ldl;
  MaxSum acc = {-INFINITY, 0.0f};
  const int64_t full4 = valid / 4;
  for (int64_t q = lane; q < full4; q += kWave) {
    const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(L + 4 * q));
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = ms_add(acc, v[e]);
  }
  for (int64_t c = 4 * full4 + lane; c < valid; c += kWave) acc = ms_add(acc, L[c]);
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    const MaxSum other = {__shfl_xor(acc.m, o), __shfl_xor(acc.s, o)};
    acc = ms_merge(acc, other);
  }
  if (lane == 0) {
    const int64_t y = (int64_t)p.labels[t] - base;
    const float z = (y >= 0 && y < valid) ? L[y] : 0.0f;
    const int64_t slot = (int64_t)(p.shard0 + s) * p.T + t;
    p.m[slot] = acc.m;
    p.s[slot] = acc.s;
    p.z[slot] = z;
  }
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

hipError_t launch_ce_stats(const CeStatsParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.shards * p.T;
  const int64_t grid = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  launch_kernel(ce_stats_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
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
