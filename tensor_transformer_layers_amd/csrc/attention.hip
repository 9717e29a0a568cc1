// Causal softmax attention over a shard's local heads (head_dim 128).
//
// Head split of the 2kiu.com blog post, section 3.1: each shard owns whole
// heads, the sequence stays whole, and attention needs no communication.  Per
// (batch, head): O = softmax(Q K^T / sqrt(d), keys <= query) V.
//
// Flash-style single pass with an online softmax, on v_mfma_f32_32x32x16_bf16.
// The score tile is computed transposed, S^T = K Q^T, so that every lane owns
// ONE query (its MFMA output column) and 32 of the 64 keys of a block; the
// running max and sum are then per lane, combined with the partner lane
// (lane ^ 32) by one cross-lane max per key block.  The output is accumulated
// transposed as well, O^T = V^T P^T: P^T feeds the B operand straight from the
// lane's own score registers (no data exchange), and V^T (stored d-major, key
// contiguous, by the QKV projection) feeds the A operand with two 8-byte LDS
// reads per lane.  The MFMA sums over k in an order that only has to agree
// between A and B, so the keys of a 16-wide step are taken in the order the
// score layout hands them over.
//
// Workgroup = 4 waves x 32 queries; key blocks of 64 are double-buffered in
// LDS.  Only the two key blocks that straddle the diagonal are masked.
// Workgroups are ordered heaviest (last query block) first.
#include <math.h>

#include "tp_device.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int kThreads = 256;
constexpr int D = 128;        // head dim
constexpr int BQ = 128;       // queries per workgroup (32 per wave)
constexpr int BKEY = 64;      // keys per block
constexpr int KLD = D + 8;    // LDS row (key) of K, padded
constexpr int VLD = BKEY + 8; // LDS row (d) of V^T, padded

__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BKEY * KLD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][D * VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;

  const int nqb = p.seq / BQ;
  const int units = p.heads * p.batch * p.nshards;
  const int u = blockIdx.x % units;
  const int qb = nqb - 1 - blockIdx.x / units;  // heaviest query blocks first
  const int h = u % p.heads;
  const int b = (u / p.heads) % p.batch;
  const int z = u / (p.heads * p.batch);

  const bf16* QK = static_cast<const bf16*>(p.QK) + z * p.sQK;
  const bf16* Vt = static_cast<const bf16*>(p.Vt) + z * p.sVt;
  bf16* O = static_cast<bf16*>(p.O) + z * p.sO;
  const int64_t tok0 = (int64_t)b * p.seq;  // first token row of this sequence

  const int q0 = qb * BQ;
  const int q = q0 + wave * 32 + lr;  // this lane's query (sequence position)

  // query fragments (B operand of S^T = K Q^T): 8 steps of 16 dims
  bf16x8 qf[D / 16];
  {
    const bf16* qrow = QK + (tok0 + q) * p.ldqk + h * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
  }

  // global -> register staging of one key block: K [64 x 128], V^T [128 x 64]
  u32x4 rk[4], rv[4];
  const bf16* kbase = QK + tok0 * p.ldqk + p.kcol0 + h * D;
  const bf16* vbase = Vt + (int64_t)h * D * p.ldvt + tok0;
  auto load_block = [&](int kb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + r * kThreads;
      const int key = c >> 4, col = (c & 15) * 8;
      rk[r] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(kb * BKEY + key) * p.ldqk + col);
      const int d = c >> 3, kc = (c & 7) * 8;
      rv[r] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)d * p.ldvt + kb * BKEY + kc);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + r * kThreads;
      *reinterpret_cast<u32x4*>(&Ks[buf][(c >> 4) * KLD + (c & 15) * 8]) = rk[r];
      *reinterpret_cast<u32x4*>(&Vs[buf][(c >> 3) * VLD + (c & 7) * 8]) = rv[r];
    }
  };

  floatx16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  const int nkb = (q0 + BQ) / BKEY;  // key blocks up to the end of this query block
  load_block(0);
  store_block(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) load_block(kb + 1);

    // S^T tile: rows = 64 keys (two 32-key MFMA tiles), columns = 32 queries
    floatx16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[t][v] = 0.0f;
    const bf16* krow = &Ks[cur][lr * KLD + 8 * lg];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + t * 32 * KLD + ks * 16);
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[t], 0, 0, 0);
      }

    // scale into the log2 domain, mask keys after the query, block max
    const bool diag = kb * BKEY + BKEY - 1 > q0;  // block reaches past the first query
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = s[t][v] * p.scale_log2e;
        if (diag) {
          const int key = kb * BKEY + t * 32 + ((v >> 2) << 3) + (lg << 2) + (v & 3);
          if (key > q) x = -INFINITY;
        }
        s[t][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);      // finite: key 0 is in block 0 for every query
    const float alpha = exp2f(m_run - m_new);  // 0 on the first block
    m_run = m_new;

    bf16x8 pb[2][2];
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = exp2f(s[t][v] - m_new);
        psum += e;
        pb[t][v >> 3][v & 7] = to_bf16(e);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[i][v] *= alpha;

    // O^T += V^T P^T.  MFMA step c covers score tile t = c/2, accumulator
    // rows v = 8*(c%2) .. +7, i.e. keys t*32 + 16*(c%2) + 4*lg + {0..3} and
    // the same + 8: the A operand reads exactly those keys of V^T.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = c >> 1, half = c & 1;
      const int k1 = t * 32 + half * 16 + lg * 4;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        const bf16* vrow = &Vs[cur][(i * 32 + lr) * VLD];
        const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vrow + k1);
        const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vrow + k1 + 8);
        const bf16x8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[t][half], o[i], 0, 0, 0);
      }
    }

    if (kb + 1 < nkb) store_block(cur ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  bf16* orow = O + (tok0 + q) * p.ldo + h * D;
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = i * 32 + r * 8 + lg * 4;
      bf16x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = to_bf16(o[i][r * 4 + j] * inv);
      *reinterpret_cast<bf16x4*>(orow + d) = w;
    }
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  const int64_t grid = (int64_t)(p.seq / BQ) * p.heads * p.batch * p.nshards;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace tp
