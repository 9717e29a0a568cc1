// Causal softmax attention over a shard's local heads (head_dim 128).
//
// Head split of the 2kiu.com blog post, section 3.1: each shard owns whole
// heads, the sequence stays whole, and attention needs no communication.  Per
// (batch, head): O = softmax(Q K^T / sqrt(d), keys <= query) V.
//
// Flash-style single pass with an online softmax, on v_mfma_f32_32x32x16_bf16.
// The score tile is computed transposed, S^T = K Q^T, so that every lane owns
// ONE query (its MFMA output column) and half of the keys of a block; the
// running max and sum are then per lane, combined with the partner lane
// (lane ^ 32) by one cross-lane max per key block.  The output is accumulated
// transposed as well, O^T = V^T P^T: P^T feeds the B operand from the lane's
// own score registers after two v_permlane32_swap per 16 keys (which put 8
// consecutive keys in each lane half), and V^T (stored d-major, key
// contiguous, by the QKV projection) feeds the A operand with one 16-byte
// LDS read per lane.
//
// Workgroup = 8 waves x 32 queries (two waves per SIMD, so one wave's softmax
// arithmetic overlaps the other's MFMAs), or 4 waves when the grid would not
// fill the chip.  Key blocks of 128 (K [128 x 128] and V^T [128 x 128],
// 64 KB) stream through a 2-stage LDS ring with the buffer-load-to-LDS path,
// one block ahead of use (128-key blocks halve the barriers per key against
// 64-key blocks in a 4-stage ring of the same size); both are XOR-swizzled at
// 16-byte granularity so the fragment reads of consecutive rows spread over
// the banks.  A wave skips the MFMAs of key blocks that lie wholly after its
// last query; only the blocks that straddle its diagonal are masked.
// Workgroups are ordered heaviest (last query block) first.  Exponentials use
// the hardware exp2 directly (results below 2^-126 flush to zero, which no
// softmax weight can tell apart from zero at bf16).
#include <math.h>

#include "tp_device.hpp"
#include "tp_dma.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int D = 128;             // head dim
constexpr int BKEY = 128;          // keys per block
constexpr int TT = BKEY / 32;      // 32-key score tiles per block
constexpr int NST = 2;             // LDS ring stages
constexpr int VROW = BKEY * 2;     // bytes of a V^T block row
constexpr int K_BYTES = BKEY * D * 2;    // K block: 128 rows of 256 bytes
constexpr int V_BYTES = D * BKEY * 2;    // V^T block: 128 rows of 256 bytes
constexpr int ST_BYTES = K_BYTES + V_BYTES;

// 16-byte chunk position of logical chunk c in row r of a K or V^T block
// (16 chunks per row in both).
__device__ __forceinline__ int kswz(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int vswz(int r, int c) { return c ^ (r & 15); }

template <int kWaves>
__global__ __launch_bounds__(kWaves * 64) void attn_fwd_kernel(AttnParams p) {
  constexpr int BQ = 32 * kWaves;              // queries per workgroup (32 per wave)
  constexpr int KI = K_BYTES / 1024 / kWaves;  // 1 KB load instructions per wave per block, K
  constexpr int VI = V_BYTES / 1024 / kWaves;  //                                          V^T
  constexpr int GROUP = KI + VI;
  static_assert(KI * kWaves * 1024 == K_BYTES && VI * kWaves * 1024 == V_BYTES, "load split");
  static_assert((NST - 1) * GROUP < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[NST * ST_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;

  const int nqb = (p.seq + BQ - 1) / BQ;
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
  const int qw = q0 + w * 32;                 // this wave's first query
  const bool wave_live = qw < p.seq;          // seq is a multiple of 32
  const int q = qw + lr;                      // this lane's query (sequence position)
  const int nkb = min(q0 + BQ, p.seq) / BKEY;  // key blocks up to the end of this query block
  const int wave_kb = wave_live ? (qw + 31) / BKEY + 1 : 0;  // blocks this wave needs

  // query fragments (B operand of S^T = K Q^T): 8 steps of 16 dims
  bf16x8 qf[D / 16];
  if (wave_live) {
    const bf16* qrow = QK + (tok0 + q) * p.ldqk + h * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
  }

  // buffer resources over this sequence's K rows and V^T columns
  const bf16* kbase = QK + tok0 * p.ldqk + p.kcol0 + h * D;
  const bf16* vbase = Vt + (int64_t)h * D * p.ldvt + tok0;
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(kbase, (uint32_t)(((int64_t)(p.seq - 1) * p.ldqk + D) * 2));
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(vbase, (uint32_t)(((int64_t)(D - 1) * p.ldvt + p.seq) * 2));
  const __amdgpu_buffer_rsrc_t rZ = make_rsrc(kbase, 0u);

  // per-lane offsets of this wave's load instructions: instruction j covers
  // rows 4j..4j+3 of the K or V^T block (16 chunks each)
  uint32_t voK[KI], voV[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int j = w * KI + i, r = 4 * j + (lane >> 4), pc = lane & 15;
    voK[i] = (uint32_t)r * (uint32_t)p.ldqk * 2u + (uint32_t)kswz(r, pc) * 16u;
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int j = w * VI + i, r = 4 * j + (lane >> 4), pc = lane & 15;
    voV[i] = (uint32_t)r * (uint32_t)p.ldvt * 2u + (uint32_t)vswz(r, pc) * 16u;
  }
  // key block kb into stage st; blocks past the end read zeros and move no data
  auto issue = [&](int kb, int st) {
    const bool live = kb < nkb;
    const __amdgpu_buffer_rsrc_t rk = live ? rK : rZ;
    const __amdgpu_buffer_rsrc_t rv = live ? rV : rZ;
    char* s = smem + st * ST_BYTES;
#pragma unroll
    for (int i = 0; i < KI; ++i)
      dma16(rk, s + (w * KI + i) * 1024, voK[i], live ? (uint32_t)kb * BKEY * (uint32_t)p.ldqk * 2u : 0u);
#pragma unroll
    for (int i = 0; i < VI; ++i)
      dma16(rv, s + K_BYTES + (w * VI + i) * 1024, voV[i], live ? (uint32_t)kb * BKEY * 2u : 0u);
  };

  floatx16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // fragment read offsets (the swizzles depend on the lane only)
  const int ko = lr * 256;  // + (kswz chunk) * 16, key row lr of each 32-row tile
  const int vo = lr * VROW;

#pragma unroll
  for (int s = 0; s < NST - 1; ++s) issue(s, s);

  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb % NST;
    wait_vmcnt<(NST - 2) * GROUP>();  // block kb has landed (this wave's part)
    lds_barrier();                     // ... every wave's part; stage (kb-1)%NST is free
    issue(kb + NST - 1, (kb + NST - 1) % NST);
    if (kb >= wave_kb) continue;  // every key of this block is after this wave's queries

    const char* ks_ = smem + st * ST_BYTES;
    const char* vs_ = ks_ + K_BYTES;

    // S^T tile: rows = BKEY keys (TT 32-key MFMA tiles), columns = 32 queries
    floatx16 s[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[t][v] = 0.0f;
#pragma unroll
    for (int kstep = 0; kstep < D / 16; ++kstep)
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(ks_ + t * 32 * 256 + ko + (kswz(lr, 2 * kstep + lg) << 4));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kstep], s[t], 0, 0, 0);
      }

    // mask keys after the query (blocks that straddle this wave's diagonal),
    // block max of the raw scores; the scale into the log2 domain is positive,
    // so it is applied after the max, fused into the exponent's argument
    const bool diag = kb * BKEY + BKEY - 1 > qw;  // block reaches past the wave's first query
    if (diag) {
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb * BKEY + t * 32 + ((v >> 2) << 3) + (lg << 2) + (v & 3);
          if (key > q) s[t][v] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[t][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * p.scale_log2e;
    // The reference point of the exponentials moves only when the block max
    // exceeds it by more than kLazy (log2 units): the softmax does not depend
    // on the point, and weights up to 2^kLazy are exact enough in fp32 and
    // bf16, so after the first blocks the accumulators are almost never
    // rescaled.  The first block always moves it (m_run = -inf; key 0 is in
    // block 0 for every query, so the new point is finite).
    constexpr float kLazy = 8.0f;
    const float m_new = mx > m_run + kLazy ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first block, else 1 or < 2^-8
    m_run = m_new;

    bf16x8 pb[TT][2];
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[t][v], p.scale_log2e, -m_new));
        psum += e;
        pb[t][v >> 3][v & 7] = to_bf16(e);
      }
    l_run = l_run * alpha + psum;
    if (__ballot(alpha != 1.0f)) {  // some running max moved: rescale the accumulators
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
    }

    // O^T += V^T P^T.  MFMA step c covers score tile t = c/2, accumulator
    // rows v = 8*(c%2) .. +7: lane half lg holds keys t*32 + 16*(c%2) +
    // 4*lg + {0..3} and the same + 8.  Two lane-half swaps give half lg the
    // keys t*32 + 16*(c%2) + 8*lg + {0..7} instead, so that the A operand is
    // one 16-byte read of V^T (logical chunk 4t + 2*(c%2) + lg).
#pragma unroll
    for (int c = 0; c < 2 * TT; ++c) {
      const int t = c >> 1, half = c & 1;
      const u32x4 d = __builtin_bit_cast(u32x4, pb[t][half]);
      const auto s0 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
      const bf16x8 pk = __builtin_bit_cast(bf16x8, u32x4{s0[0], s1[0], s0[1], s1[1]});
      const int ch = 4 * t + 2 * half + lg;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vs_ + i * 32 * VROW + vo + (vswz(lr, ch) << 4));
        o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk, o[i], 0, 0, 0);
      }
    }
  }
  wait_vmcnt<0>();  // no load may still target this workgroup's LDS when it exits

  if (!wave_live) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  bf16* orow = O + (tok0 + q) * p.ldo + h * D;
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = i * 32 + r * 8 + lg * 4;
      bf16x4 wv;
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = to_bf16(o[i][r * 4 + j] * inv);
      *reinterpret_cast<bf16x4*>(orow + d) = wv;
    }
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  // 8 waves (256 queries) per workgroup when that still gives every CU a
  // workgroup; otherwise 4 waves (128 queries)
  const int64_t units = (int64_t)p.heads * p.batch * p.nshards;
  const int64_t grid8 = (int64_t)((p.seq + 255) / 256) * units;
  if (units <= 0 || p.seq <= 0) return hipSuccess;
  if (grid8 >= 256) {
    launch_kernel(attn_fwd_kernel<8>, dim3((unsigned)grid8), dim3(512), 0, s, p);
  } else {
    const int64_t grid4 = (int64_t)((p.seq + 127) / 128) * units;
    launch_kernel(attn_fwd_kernel<4>, dim3((unsigned)grid4), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace tp
