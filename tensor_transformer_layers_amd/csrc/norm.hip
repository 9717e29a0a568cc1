// Norms of the tensor-parallel sublayer boundary (2kiu.com blog post, section
// 3.3: the norm needs the statistics of the whole hidden vector).
//
// Entry side of the sequence-parallel region: RMSNorm or LayerNorm of each
// rank's sequence slice, written straight into that slice's rows of the
// gathered [T x H] buffer -- the buffer every rank holds after the
// all-gather that feeds the next column linear.  The norm runs on sequence
// slices because it is row-wise (blog post, section 4.3; "张量并行",
// Megatron-SP section):
//
//   RMSNorm    Y[r*T/N + t, :] = X_r[t, :] / sqrt(mean(X_r[t, :]^2) + eps) * g
//   LayerNorm  Y[r*T/N + t, :] = (X_r[t, :] - m) / sqrt(v + eps) * g + b
//              (m, v the mean and the mean squared deviation of the row)
//
// HBM-bound streaming kernel, one to eight waves per token row (wide rows are
// split so that each wave holds at most 4 KB of its row and enough waves stay
// resident to keep HBM busy):
//  * the row is read once into registers (U 16-byte pieces per lane, lane i
//    taking bytes 16i.. of every KB of its wave's part), so X leaves HBM
//    exactly once;
//  * each statistic is an fp32 sum, per lane in piece order, then across the
//    wave by an xor butterfly -- every pair adds the same two values, so all
//    lanes end with the same bits -- then, for split rows, over the row's
//    waves in wave order through LDS; the result repeats run to run.
//    RMSNorm sums squares; LayerNorm first sums the values (the mean), then
//    the squared deviations from that mean (a second pass over the registers,
//    so no cancellation between a sum of squares and a squared mean);
//  * the scale is the hardware reciprocal square root of mean + eps (about
//    one ulp in fp32, far below the bf16 output step);
//  * one round-to-nearest-even cast, 16-byte stores into the gathered buffer.
//
// Norm of an input split along hidden across ranks (blog post, section 3.3:
// keep the input split, reduce a small statistic, correct by a formula), in
// two kernels standing for the two sides of the statistic's all-reduce:
//  * norm_split_stats_kernel: each shard's statistic of each of its row
//    slices into slot (shard, row) of a slab -- RMSNorm the slice's sum of
//    squares; LayerNorm the slice's mean and sum of squared deviations about
//    it (same register-resident structure as above);
//  * norm_split_apply_kernel: each (shard, row) folds the N slots of its row
//    in shard order -- sums of squares added; (count, mean, M2) triples
//    merged by the pairwise update  d = m_i - m, n' = n + c,
//    m += d c/n', M2 += M2_i + d^2 n c/n'  -- so every shard computes the
//    same bits (the broadcast), then scales its own slice.
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

// Sum of x over the lanes of each wave (xor butterfly: every lane ends with
// the same bits), then over the WPR waves of a row part in wave order
// through LDS.  Called by every wave of the workgroup; the trailing barrier
// lets the next call reuse the buffer.
template <int WPR, int NT>
__device__ __forceinline__ float row_sum(float x, float* buf, int wv, int part, int lane) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  if constexpr (WPR > 1) {
    if (lane == 0) buf[wv] = x;
    __syncthreads();
    const int w0 = wv - part;
    x = buf[w0];
#pragma unroll
    for (int k = 1; k < WPR; ++k) x += buf[w0 + k];
    __syncthreads();
  }
  return x;
}

// Statistics of a row part of n elements held in v (pieces past n are zero
// and are left out): RMS -> (sum of squares, 0); LayerNorm -> (mean, sum of
// squared deviations about it).
template <typename T, int U, int WPR, int NT, bool LAYER>
__device__ __forceinline__ float2 part_stats(const typename Vec<T>::V (&v)[U], int n, float inv_n, float* buf,
                                             int wv, int part, int lane) {
  constexpr int E = Vec<T>::E;
  if constexpr (!LAYER) {
    float ss = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float f = static_cast<float>(v[u][e]);
        ss = fmaf(f, f, ss);
      }
    return {row_sum<WPR, NT>(ss, buf, wv, part, lane), 0.0f};
  } else {
    float sx = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) sx += static_cast<float>(v[u][e]);
    const float mean = row_sum<WPR, NT>(sx, buf, wv, part, lane) * inv_n;
    float q = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = ((part * U + u) * 64 + lane) * E;
      if (c < n)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float d = static_cast<float>(v[u][e]) - mean;
          q = fmaf(d, d, q);
        }
    }
    return {mean, row_sum<WPR, NT>(q, buf, wv, part, lane)};
  }
}

template <typename T, int U, int WPR, int NT, bool LAYER>
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
  __shared__ float red[NT / 64];
  const float2 st = part_stats<T, U, WPR, NT, LAYER>(v, p.H, p.inv_h, red, wv, part, lane);
  const float mean = LAYER ? st.x : 0.0f;
  const float scale = __builtin_amdgcn_rsqf((LAYER ? st.y : st.x) * p.inv_h + p.eps);
  const T* const b = static_cast<const T*>(p.beta);

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = ((part * U + u) * 64 + lane) * E;
    if (live && c < p.H) {
      const V gv = *reinterpret_cast<const V*>(g + c);
      V bv;
      if (LAYER && b) {
        bv = *reinterpret_cast<const V*>(b + c);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) bv[e] = static_cast<T>(0.0f);
      }
      V o;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float f;
        if constexpr (LAYER)
          f = (static_cast<float>(v[u][e]) - mean) * scale * static_cast<float>(gv[e]) + static_cast<float>(bv[e]);
        else
          f = static_cast<float>(v[u][e]) * scale * static_cast<float>(gv[e]);
        if constexpr (std::is_same<T, bf16>::value)
          o[e] = to_bf16(f);
        else
          o[e] = f;
      }
      *reinterpret_cast<V*>(y + c) = o;
    }
  }
}

// Hidden-split norm, first half: the statistic of each (shard, row) slice of
// Hs elements (shard s of the launch = shard shard0 + s, its columns
// [(shard0 + s) Hs, +Hs)), into slot ((shard0 + s) T + t) of the slab
// (two floats per slot).
template <typename T, int U, int WPR, int NT, bool LAYER>
__global__ __launch_bounds__(NT) void norm_split_stats_kernel(NormSplitParams p) {
  using V = typename Vec<T>::V;
  constexpr int E = Vec<T>::E;
  constexpr int kRows = NT / 64 / WPR;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int part = wv % WPR;
  // workgroup -> (block of kRows tokens, shard), every shard of a block
  // before the next block, so that neighbouring workgroups read neighbouring
  // memory
  const int64_t blk = blockIdx.x / p.shards;
  const int64_t s = blockIdx.x - blk * p.shards;
  const int64_t t0 = blk * kRows + wv / WPR;
  if (WPR == 1 && t0 >= p.T) return;  // split rows keep every wave for the barriers
  const bool live = t0 < p.T;
  const int64_t t = live ? t0 : 0;
  const int64_t shard = p.shard0 + s;
  const T* const x = static_cast<const T*>(p.X) + t * p.ldx + shard * p.Hs;
  V v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = ((part * U + u) * 64 + lane) * E;
    if (live && c < p.Hs) {
      v[u] = *reinterpret_cast<const V*>(x + c);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) v[u][e] = static_cast<T>(0.0f);
    }
  }
  __shared__ float red[NT / 64];
  const float2 st = part_stats<T, U, WPR, NT, LAYER>(v, p.Hs, p.inv_hs, red, wv, part, lane);
  if (live && part == 0 && lane == 0) *reinterpret_cast<float2*>(p.stats + 2 * (shard * p.T + t)) = st;
}

// Hidden-split norm, second half: one wave per (shard, row) slice folds the
// row's N statistics in shard order (every shard the same bits), then scales
// its slice: 16-byte pieces, lanes striding by 1 KB.  With U > 0 the slice
// has at most U pieces per lane and every load (all pieces of x, gamma and
// beta, and the statistics when N <= 8) is issued before the arithmetic.
template <typename T, int U, bool LAYER>
__global__ __launch_bounds__(256) void norm_split_apply_kernel(NormSplitParams p) {
  using V = typename Vec<T>::V;
  constexpr int E = Vec<T>::E;
  constexpr int kMaxN = 8;
  const int lane = threadIdx.x & 63;
  // workgroup -> (block of 4 tokens, shard), as in the statistics kernel
  const int64_t blk = blockIdx.x / p.shards;
  const int64_t s = blockIdx.x - blk * p.shards;
  const int64_t t = blk * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int64_t shard = p.shard0 + s;
  const float2* const st = reinterpret_cast<const float2*>(p.stats) + t;
  const T* const x = static_cast<const T*>(p.X) + t * p.ldx + shard * p.Hs;
  T* const y = static_cast<T*>(p.Y) + t * p.ldy + shard * p.Hs;
  const T* const g = static_cast<const T*>(p.gamma) + shard * p.Hs;
  const T* const b = p.beta ? static_cast<const T*>(p.beta) + shard * p.Hs : nullptr;
  V xs[U > 0 ? U : 1], gs[U > 0 ? U : 1], bs[U > 0 ? U : 1];
  if constexpr (U > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (u * 64 + lane) * E;
#pragma unroll
      for (int e = 0; e < E; ++e) xs[u][e] = gs[u][e] = bs[u][e] = static_cast<T>(0.0f);
      if (c < p.Hs) {
        xs[u] = *reinterpret_cast<const V*>(x + c);
        gs[u] = *reinterpret_cast<const V*>(g + c);
        if (LAYER && b) bs[u] = *reinterpret_cast<const V*>(b + c);
      }
    }
  }
  // the N statistics of the token, folded in shard order
  float mean = 0.0f, q;
  const float cs = (float)p.Hs;
  float n = cs;
  auto merge = [&](float2 a) {
    if constexpr (!LAYER) {
      q += a.x;
    } else {
      const float n1 = n + cs;
      const float d = a.x - mean;
      mean = fmaf(d, cs / n1, mean);
      q = q + a.y + d * d * (n * cs / n1);
      n = n1;
    }
  };
  {
    const float2 a0 = st[0];
    mean = LAYER ? a0.x : 0.0f;
    q = LAYER ? a0.y : a0.x;
  }
  if (p.N <= kMaxN) {
    float2 sv[kMaxN];
#pragma unroll
    for (int i = 1; i < kMaxN; ++i)
      if (i < p.N) sv[i] = st[(int64_t)i * p.T];
#pragma unroll
    for (int i = 1; i < kMaxN; ++i)
      if (i < p.N) merge(sv[i]);
  } else {
    for (int i = 1; i < p.N; ++i) merge(st[(int64_t)i * p.T]);
  }
  const float scale = __builtin_amdgcn_rsqf(q * p.inv_h + p.eps);
  auto out = [&](const V& xv, const V& gv, const V& bv, int c) {
    V o;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float f;
      if constexpr (LAYER)
        f = (static_cast<float>(xv[e]) - mean) * scale * static_cast<float>(gv[e]) + static_cast<float>(bv[e]);
      else
        f = static_cast<float>(xv[e]) * scale * static_cast<float>(gv[e]);
      if constexpr (std::is_same<T, bf16>::value)
        o[e] = to_bf16(f);
      else
        o[e] = f;
    }
    *reinterpret_cast<V*>(y + c) = o;
  };
  if constexpr (U > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (u * 64 + lane) * E;
      if (c < p.Hs) out(xs[u], gs[u], bs[u], c);
    }
  } else {
    for (int c = lane * E; c < p.Hs; c += 64 * E) {
      const V xv = *reinterpret_cast<const V*>(x + c);
      const V gv = *reinterpret_cast<const V*>(g + c);
      V bv;
      if (LAYER && b) {
        bv = *reinterpret_cast<const V*>(b + c);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) bv[e] = static_cast<T>(0.0f);
      }
      out(xv, gv, bv, c);
    }
  }
}

template <typename T, int U, int WPR, bool LAYER, int NT = 256>
hipError_t launch_shape(const NormParams& p, hipStream_t s) {
  constexpr int kRows = NT / 64 / WPR;
  const dim3 g((unsigned)((p.rows + kRows - 1) / kRows)), b(NT);
  launch_kernel((rmsnorm_gather_kernel<T, U, WPR, NT, LAYER>), g, b, 0u, s, p);
  return hipGetLastError();
}

template <typename T, int U, int WPR, bool LAYER, int NT = 256>
hipError_t launch_split_shape(const NormSplitParams& p, hipStream_t s) {
  constexpr int kRows = NT / 64 / WPR;
  const dim3 g((unsigned)((p.T + kRows - 1) / kRows * p.shards)), b(NT);
  launch_kernel((norm_split_stats_kernel<T, U, WPR, NT, LAYER>), g, b, 0u, s, p);
  return hipGetLastError();
}

// pieces = 1 KB pieces of a row (part); rows of more than 2 pieces are split
// over 2 to 8 waves (at most 4 pieces, 16 registers of row data, per wave)
template <typename T, bool LAYER, class P, class F>
hipError_t by_pieces(const P& p, int64_t n, hipStream_t s, F) {
  constexpr int per_piece = 64 * Vec<T>::E;
  const int64_t pieces = (n + per_piece - 1) / per_piece;
  if (pieces <= 1) return F::template go<T, 1, 1, LAYER>(p, s);
  if (pieces <= 2) return F::template go<T, 2, 1, LAYER>(p, s);
  if (pieces <= 4) return F::template go<T, 2, 2, LAYER>(p, s);
  if (pieces <= 8) return F::template go<T, 2, 4, LAYER>(p, s);
  if (pieces <= 16) return F::template go<T, 4, 4, LAYER>(p, s);
  if (pieces <= 24) return F::template go512<T, 3, 8, LAYER>(p, s);
  if (pieces <= 32) return F::template go512<T, 4, 8, LAYER>(p, s);
  return hipErrorInvalidValue;
}

struct GatherLaunch {
  template <typename T, int U, int WPR, bool LAYER>
  static hipError_t go(const NormParams& p, hipStream_t s) { return launch_shape<T, U, WPR, LAYER>(p, s); }
  template <typename T, int U, int WPR, bool LAYER>
  static hipError_t go512(const NormParams& p, hipStream_t s) { return launch_shape<T, U, WPR, LAYER, 512>(p, s); }
};

struct SplitStatsLaunch {
  template <typename T, int U, int WPR, bool LAYER>
  static hipError_t go(const NormSplitParams& p, hipStream_t s) { return launch_split_shape<T, U, WPR, LAYER>(p, s); }
  template <typename T, int U, int WPR, bool LAYER>
  static hipError_t go512(const NormSplitParams& p, hipStream_t s) {
    return launch_split_shape<T, U, WPR, LAYER, 512>(p, s);
  }
};

template <typename T, bool LAYER>
hipError_t launch_split_apply(const NormSplitParams& p, hipStream_t s) {
  const dim3 g((unsigned)((p.T + 3) / 4 * p.shards)), b(256);
  const int64_t pieces = (p.Hs + 64 * Vec<T>::E - 1) / (64 * Vec<T>::E);
  if (pieces <= 1)
    launch_kernel((norm_split_apply_kernel<T, 1, LAYER>), g, b, 0u, s, p);
  else if (pieces <= 2)
    launch_kernel((norm_split_apply_kernel<T, 2, LAYER>), g, b, 0u, s, p);
  else if (pieces <= 3)
    launch_kernel((norm_split_apply_kernel<T, 3, LAYER>), g, b, 0u, s, p);
  else if (pieces <= 4)
    launch_kernel((norm_split_apply_kernel<T, 4, LAYER>), g, b, 0u, s, p);
  else
    launch_kernel((norm_split_apply_kernel<T, 0, LAYER>), g, b, 0u, s, p);
  return hipGetLastError();
}

}  // namespace

int64_t rmsnorm_max_hidden(bool bf16_io) { return 32 * 64 * (bf16_io ? 8 : 4); }

hipError_t launch_rmsnorm_gather(const NormParams& p, bool bf16_io, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  if (p.layer)
    return bf16_io ? by_pieces<bf16, true>(p, p.H, s, GatherLaunch{}) : by_pieces<float, true>(p, p.H, s, GatherLaunch{});
  return bf16_io ? by_pieces<bf16, false>(p, p.H, s, GatherLaunch{}) : by_pieces<float, false>(p, p.H, s, GatherLaunch{});
}

hipError_t launch_norm_split_stats(const NormSplitParams& p, bool bf16_io, hipStream_t s) {
  if (p.T <= 0 || p.shards <= 0) return hipSuccess;
  if (p.layer)
    return bf16_io ? by_pieces<bf16, true>(p, p.Hs, s, SplitStatsLaunch{})
                   : by_pieces<float, true>(p, p.Hs, s, SplitStatsLaunch{});
  return bf16_io ? by_pieces<bf16, false>(p, p.Hs, s, SplitStatsLaunch{})
                 : by_pieces<float, false>(p, p.Hs, s, SplitStatsLaunch{});
}

hipError_t launch_norm_split_apply(const NormSplitParams& p, bool bf16_io, hipStream_t s) {
  if (p.T <= 0 || p.shards <= 0) return hipSuccess;
  if (p.layer) return bf16_io ? launch_split_apply<bf16, true>(p, s) : launch_split_apply<float, true>(p, s);
  return bf16_io ? launch_split_apply<bf16, false>(p, s) : launch_split_apply<float, false>(p, s);
}

}  // namespace tp
