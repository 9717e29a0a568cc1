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
// Workgroup = 8 waves x 32 queries (two waves per SIMD), or 4 waves when the
// grid would not fill the chip.  Inside a wave each key block is split in two
// halves of 64 keys and software-pipelined: the exponentials of one half run
// between the MFMAs of the next product (S^T of half 1, then O^T of half 0),
// so the matrix cores keep working through the softmax arithmetic.
// Key blocks of 128 (K [128 x 128] and V^T [128 x 128], 64 KB) stream
// through a 2-stage LDS ring with the buffer-load-to-LDS path,
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
    const bool diag = kb * BKEY + BKEY - 1 > qw;  // block reaches past the wave's first query

    floatx16 s[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[t][v] = 0.0f;
    // K fragment of score tile t, k-step ks; V^T fragment of output tile i,
    // logical key chunk ch
    auto kfrag = [&](int t, int ks) __attribute__((always_inline)) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(ks_ + t * 32 * 256 + ko + (kswz(lr, 2 * ks + lg) << 4));
    };
    auto vfrag = [&](int i, int ch) __attribute__((always_inline)) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(vs_ + i * 32 * VROW + vo + (vswz(lr, ch) << 4));
    };
    // keys after the query are masked (only in blocks that straddle the
    // wave's diagonal); key of tile t, register v: t*32 + 8*(v/4) + 4*lg + v%4
    auto mask = [&](int half) __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < TT / 2; ++tt) {
        const int t = half * (TT / 2) + tt;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb * BKEY + t * 32 + ((v >> 2) << 3) + (lg << 2) + (v & 3);
          if (key > q) s[t][v] = -INFINITY;
        }
      }
    };
    // max of the half's raw scores (the scale into the log2 domain is
    // positive, so it is applied after the max, fused into the exponent's
    // argument; the partner lane's half by a lane-half swap), then the lazy
    // move of the reference point: it moves only when the max exceeds it by
    // more than kLazy (log2 units) -- the softmax does not depend on the
    // point, and weights up to 2^kLazy are exact enough in fp32 and bf16, so
    // after the first keys the accumulators are almost never rescaled.  Key
    // 0 is in half 0 of block 0 for every query, so the first move gives a
    // finite point.
    constexpr float kLazy = 8.0f;
    auto new_point = [&](int half) __attribute__((always_inline)) -> float {
      float mx = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < TT / 2; ++tt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[half * (TT / 2) + tt][v]);
      const uint32_t mb = __builtin_bit_cast(uint32_t, mx);
      const auto sw = __builtin_amdgcn_permlane32_swap(mb, mb, false, false);
      mx = fmaxf(__builtin_bit_cast(float, sw[0]), __builtin_bit_cast(float, sw[1])) * p.scale_log2e;
      const float m_new = mx > m_run + kLazy ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 at the first move, else 1 or < 2^-8
      m_run = m_new;
      return alpha;
    };
    auto rescale = [&](float alpha) __attribute__((always_inline)) {
      if (__ballot(alpha != 1.0f)) {  // some running max moved
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
      }
    };
    // Exponentials of a half, packed to bf16 and permuted into the B operand
    // of its O^T MFMAs.  O^T step c covers score tile t = c/2, accumulator
    // rows v = 8*(c%2) .. +7, where lane half lg holds keys t*32 + 16*(c%2) +
    // 4*lg + {0..3} and the same + 8; two lane-half swaps give half lg the
    // keys t*32 + 16*(c%2) + 8*lg + {0..7} instead, so that the A operand is
    // one 16-byte read of V^T (logical chunk 4t + 2*(c%2) + lg).  Element e
    // (of 32) of the half is tile half*2 + e/16, register e%16; a finished
    // group of 8 is permuted at once.  The empty asm statement pins each
    // operand where it is made: without it the compiler sinks the chain
    // into the block of its MFMAs, after the branch that follows.
    bf16x8 pk[TT][2];
    bf16x8 pb;
    auto soft2 = [&](int half, int g, float& psum) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = 2 * g + j, t = half * (TT / 2) + e / 16, v = e % 16;
        const float x = __builtin_amdgcn_exp2f(fmaf(s[t][v], p.scale_log2e, -m_run));
        psum += x;
        pb[v & 7] = to_bf16(x);
      }
      if (g % 4 == 3) {
        const int e = 2 * g + 1, t = half * (TT / 2) + e / 16, hf = (e % 16) >> 3;
        const u32x4 d = __builtin_bit_cast(u32x4, pb);
        const auto s0 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
        u32x4 k = u32x4{s0[0], s1[0], s0[1], s1[1]};
        asm volatile("" : "+v"(k));
        pk[t][hf] = __builtin_bit_cast(bf16x8, k);
      }
    };

    // The block is processed in two halves of 64 keys (score tiles 0-1 and
    // 2-3), software-pipelined inside the wave so that the matrix cores keep
    // working through the softmax arithmetic:
    //   steps  0..15  S^T of half 0
    //   steps 16..31  S^T of half 1           one MFMA, then two exponentials of half 0
    //   steps 32..47  O^T += V^T P^T, half 0  one MFMA, then two exponentials of half 1
    //   steps 48..63  O^T += V^T P^T, half 1
    // Each half updates the running max (lazily) and sum on its own: the same
    // online softmax at a 64-key grain.  The LDS operand of step n (a K
    // fragment for steps < 32, a V^T fragment after) is read kAhead steps
    // ahead into a ring of registers, which covers the LDS latency (with the
    // read one step ahead, each MFMA waited for its fragment).
    constexpr int kAhead = 3;
    auto frag = [&](int n) __attribute__((always_inline)) -> bf16x8 {
      if (n < 32) {  // S^T step: tile 2*(n/16) + n%2, k-step (n%16)/2
        const int g = n % 16;
        return kfrag(2 * (n / 16) + g % 2, g / 2);
      }
      const int m = n - 32, c = 4 * (m / 16) + (m % 16) / 4;  // O^T step c, output tile m%4
      return vfrag(m % 4, 4 * (c >> 1) + 2 * (c & 1) + lg);
    };
    bf16x8 ring[kAhead + 1];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) ring[n] = frag(n);
    auto next = [&](int n) __attribute__((always_inline)) {
      if (n + kAhead < 64) ring[(n + kAhead) % (kAhead + 1)] = frag(n + kAhead);
    };
#pragma unroll
    for (int g = 0; g < 16; ++g) {  // S^T, half 0: tile g%2, k-step g/2
      next(g);
      s[g % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[g % (kAhead + 1)], qf[g / 2], s[g % 2], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // The serial parts of the online softmax (mask, max, reference point,
    // rescale) run at wave priority 0, the rest at 1: while one wave of a
    // SIMD is in them, the other wave's MFMAs take the issue slots first
    // (measured at workload 4: 293 -> 286 us).
    __builtin_amdgcn_s_setprio(0);
    if (diag) mask(0);
    const float alpha0 = new_point(0);
    __builtin_amdgcn_s_setprio(1);
    float psum0 = 0.0f;
#pragma unroll
    for (int g = 0; g < 16; ++g) {  // S^T, half 1: tile 2 + g%2, k-step g/2
      const int n = 16 + g;
      next(n);
      s[2 + g % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[n % (kAhead + 1)], qf[g / 2], s[2 + g % 2], 0, 0, 0);
      soft2(0, g, psum0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    l_run = l_run * alpha0 + psum0;
    rescale(alpha0);
    if (diag) mask(1);
    const float alpha1 = new_point(1);
    __builtin_amdgcn_s_setprio(1);
    float psum1 = 0.0f;
#pragma unroll
    for (int g = 0; g < 16; ++g) {  // O^T, half 0: step c = g/4 (tile c/2, rows 8 (c%2)), output tile g%4
      const int n = 32 + g, c = g / 4, i = g % 4;
      next(n);
      o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[n % (kAhead + 1)], pk[c >> 1][c & 1], o[i], 0, 0, 0);
      soft2(1, g, psum1);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    l_run = l_run * alpha1 + psum1;
    rescale(alpha1);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int g = 0; g < 16; ++g) {  // O^T, half 1: step c = 4 + g/4, output tile g%4
      const int n = 48 + g, c = 4 + g / 4, i = g % 4;
      next(n);
      o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[n % (kAhead + 1)], pk[c >> 1][c & 1], o[i], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
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
