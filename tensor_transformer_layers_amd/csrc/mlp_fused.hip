// One shard's whole MLP in one kernel, for narrow hidden sizes (H = 256, 512):
//
//   P_i = act(X A_i^T + a_i) B_i^T        (fp32 partial, no row bias)
//
// The column product, the activation on the shard-local slice and the row
// partial follow each other with no communication in between (2kiu.com blog
// post, section 2.3; "张量并行", MLP formula GELU(XA)B), so the shard-local
// intermediate H_i never has to leave the chip: it lives in registers, 32
// intermediate features at a time, between the two products.  The partials
// equal those of the separate column and row kernels up to fp32 rounding
// (summation order inside the products; the bias enters first here).
//
// Layout of the work (gfx950, 4 waves = one per SIMD, 1 workgroup per CU):
//  * A workgroup owns 128 tokens of one shard; wave w owns tokens 32w..32w+31.
//    Its X rows stay in VGPRs for the whole kernel (the MFMA's second operand
//    of the column product), its [32 x H] fp32 partial fills the 256 AGPRs.
//  * The intermediate features are consumed in chunks of 32.  Per chunk, the
//    column product H^T[32 f x 32 tok] = A_i[f rows] X^T is one chain of
//    H/16 v_mfma_f32_32x32x16_bf16 that starts from the chunk's bias (the
//    bias is the chain's initial accumulator, so no vector add is needed)
//    and accumulates in VGPRs: with every AGPR holding the partial, the
//    compiler would otherwise park a partial tile in VGPRs around each chain
//    (48 register moves per chunk).  The row product P += H B_i^T[f rows] is
//    2*H/32 MFMAs, the activated chunk being the MFMA's first operand.
//  * The accumulator layout of the column product gives each lane one token
//    and 16 features; two v_permlane32_swap per 16 features move them into
//    the operand layout of the row product (8 consecutive features per lane
//    half), so no LDS round trip is needed.
//  * A_i and B_i chunks (32 KB each at H = 512) stream through a two-slot LDS
//    ring by buffer loads to LDS, XOR-swizzled so that the 16-byte fragment
//    reads are bank-conflict free; one barrier per chunk.
//  * Software pipeline.  The activation costs about as many vector cycles as
//    the chunk's MFMAs take (a wave64 fp32 op issues every ~5 cycles, an exp
//    or reciprocal every ~16; GELU is 11 ops + 2 of those per value, 16
//    values per lane per chunk), and a wave's vector instructions run while
//    its own MFMAs execute, so the activation is spread evenly over all of a
//    step's MFMAs, one stage of one value per MFMA: each step issues the
//    column product of chunk c (with the loads of chunk c's B part and chunk
//    c+1's A part between its MFMAs) carrying the second half of chunk c-1's
//    activation, then the row product of chunk c-1 carrying the first half
//    of chunk c's.
//  * Workgroups are renumbered so that the shards of a token block run on
//    one XCD: X is read from HBM once per token block (it is the largest
//    input; each shard's weights are 1 MB and stream chunk by chunk through
//    every XCD's L2).
#include <type_traits>

#include "tp_device.hpp"
#include "tp_dma.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int kFThreads = 256;
constexpr int kTokWave = 32;
constexpr int kTokBlock = 4 * kTokWave;
constexpr int kFC = 32;            // intermediate features per chunk
constexpr int kBiasMax = 4096;     // features of a shard whose bias fits the LDS area

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int NT_>
struct FC {
  static constexpr int NT = NT_;                 // 32-wide output tiles of the row product
  static constexpr int H = NT * 32;              // hidden size
  static constexpr int KB1 = H / 16;             // k-blocks of the column product
  // A_i chunk [32 f x H]: one load instruction fills RPD rows (1 KB); each
  // such group of rows is followed by 16 bytes of padding, so that row r's
  // chunk c sits 16(r/RPD) bytes further along the banks than row 0's and
  // the fragment reads of 16 consecutive rows are conflict free.  With two
  // rows per group the second row's chunks are also XOR-ed with 8.
  static constexpr int RPD = 1024 / (H * 2);
  static constexpr int A_GROUP = 1024 + 16;
  static constexpr int A_SLOT = (kFC / RPD) * A_GROUP;
  static constexpr int A_DMA = kFC / 4 / RPD;    // load instructions per wave per chunk
  // B_i chunk [H out x 32 f], 64-byte rows, chunk c of row r at c ^ ((r>>2)&3)
  static constexpr int B_SLOT = H * kFC * 2;
  static constexpr int B_DMA = H / 16 / 4;
  static constexpr int B_OFF = 2 * A_SLOT;
  static constexpr int BIAS_OFF = B_OFF + 2 * B_SLOT;
  static constexpr int LDS = BIAS_OFF + kBiasMax * 4;  // fp32 bias
  static_assert((RPD == 1 || RPD == 2) && (kFC / 4) % RPD == 0, "A chunk rows per wave");
  static_assert(H % 64 == 0 && B_DMA >= 1, "B chunk rows per wave");
};

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {to_bf16(a), to_bf16(b)};
  return __builtin_bit_cast(uint32_t, v);
}

template <class C, bool GELU>
__global__ __launch_bounds__(kFThreads, 1) void mlp_fused_kernel(FusedMlpParams p, int tblocks) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lh = lane >> 5;

  // consecutive ids (one XCD) take the shards of one token block: its X rows
  // come from HBM once per XCD and then from the XCD's L2
  const int pid = xcd_remap(blockIdx.x, gridDim.x);
  const int shard = pid % p.shards;
  const int tb = pid / p.shards;
  const int tok0 = tb * kTokBlock;
  const int Fs = p.Fs;
  const int nchunk = Fs / kFC;

  const bf16* const Ai = static_cast<const bf16*>(p.A) + shard * p.sA;
  const bf16* const Bi = static_cast<const bf16*>(p.B) + shard * p.sB;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(Ai, (uint32_t)(((int64_t)(Fs - 1) * p.lda + C::H) * 2));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bi, (uint32_t)(((int64_t)(C::H - 1) * p.ldb + Fs) * 2));

  const __amdgpu_buffer_rsrc_t rZ = make_rsrc(Ai, 0u);  // reads nothing

  // Per-lane byte offset of every load instruction of this wave; the row
  // group and the chunk's feature offset go into soffset.
  //  A: lane i -> row (i / (64/RPD)) of the group, chunk i % (64/RPD)
  //  B: lane i -> row i/4 of a 16-row group, chunk (i&3) ^ ((i>>4)&3)
  const int a_b = lane / (64 / C::RPD), a_c = lane % (64 / C::RPD);
  const uint32_t vA = (uint32_t)a_b * (uint32_t)p.lda * 2u + (uint32_t)(a_c ^ (8 * a_b)) * 16u;
  const uint32_t vB = (uint32_t)(lane >> 2) * (uint32_t)p.ldb * 2u + (uint32_t)((lane & 3) ^ ((lane >> 4) & 3)) * 16u;
  auto dma_a = [&](int slot, int j, int c, bool live) {
    const int grp = w * C::A_DMA + j;
    dma16(live ? rA : rZ, smem + slot * C::A_SLOT + grp * C::A_GROUP, vA,
          (uint32_t)(grp * C::RPD + c * kFC) * (uint32_t)p.lda * 2u);
  };
  auto dma_b = [&](int slot, int j, int c) {
    const int grp = w * C::B_DMA + j;
    dma16(rB, smem + C::B_OFF + slot * C::B_SLOT + grp * 1024, vB,
          (uint32_t)(16 * grp) * (uint32_t)p.ldb * 2u + (uint32_t)(c * kFC) * 2u);
  };
  auto issue_a = [&](int slot, int c) {
#pragma unroll
    for (int j = 0; j < C::A_DMA; ++j) dma_a(slot, j, c, true);
  };
  auto issue_b = [&](int slot, int c) {
#pragma unroll
    for (int j = 0; j < C::B_DMA; ++j) dma_b(slot, j, c);
  };

  issue_a(0, 0);

  // the shard's column bias into LDS (zeros without one)
  {
    float* bl = reinterpret_cast<float*>(smem + C::BIAS_OFF);
    const bf16* bg = p.bias ? static_cast<const bf16*>(p.bias) + shard * p.sBias : nullptr;
    for (int i = tid; i < Fs / 8; i += kFThreads) {
      floatx4 lo = {0.0f, 0.0f, 0.0f, 0.0f}, hi = lo;
      if (bg) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(bg + 8 * i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = static_cast<float>(v[e]);
          hi[e] = static_cast<float>(v[4 + e]);
        }
      }
      *reinterpret_cast<floatx4*>(bl + 8 * i) = lo;
      *reinterpret_cast<floatx4*>(bl + 8 * i + 4) = hi;
    }
  }

  // this wave's X rows as MFMA operands: lane (l32, lh) holds token l32,
  // hidden features 16kb + 8lh .. +7 for every k-block kb.  Rows past T
  // repeat row T-1; their partials are never stored.
  bf16x8 xf[C::KB1];
  {
    const int row = min(tok0 + w * kTokWave + l32, p.T - 1);
    const bf16* xr = static_cast<const bf16*>(p.X) + (int64_t)row * p.ldx + 8 * lh;
#pragma unroll
    for (int kb = 0; kb < C::KB1; ++kb) xf[kb] = *reinterpret_cast<const bf16x8*>(xr + 16 * kb);
  }

  floatx16 P[C::NT];
#pragma unroll
  for (int n = 0; n < C::NT; ++n)
#pragma unroll
    for (int v = 0; v < 16; ++v) P[n][v] = 0.0f;
  // fragment addressing: lane (l32, lh) reads row l32, chunk 2kb + lh of A
  // (k-blocks with bit 2 set move the other way under the XOR with 8) and
  // row 32n + l32, chunk 2k + lh of B
  const int a_grp = l32 / C::RPD, a_odd = l32 % C::RPD;
  const int a_base = a_grp * C::A_GROUP + a_odd * (C::H * 2) + lh * 16;
  const int a_lo = a_base + 128 * a_odd, a_hi = a_base - 128 * a_odd;
  const int b_row = l32 * (kFC * 2);
  const int b_off0 = b_row + (((0 + lh) ^ ((l32 >> 2) & 3)) << 4);
  const int b_off1 = b_row + (((2 + lh) ^ ((l32 >> 2) & 3)) << 4);
  const float* const bias_lane = reinterpret_cast<const float*>(smem + C::BIAS_OFF) + 4 * lh;

  // The column product of a chunk accumulates in VGPRs (every AGPR holds
  // the partial P): its MFMAs are written out with VGPR operands, and the
  // hazards the compiler would otherwise handle are covered here.  The
  // first MFMA of the chain takes C = 0 and an early-clobber destination (no
  // overlap with its sources); each later one accumulates into exactly the
  // registers it reads as C, which needs no wait states; before any vector
  // instruction reads the result, col_done issues 21 wait states (an 8-pass
  // MFMA result needs 11).
  floatx16 acc, bvec;
  auto col_mfma = [&](int m, const bf16x8& f) {
    if (m == 0)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(acc) : "v"(f), "v"(xf[0]), "v"(bvec));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(f), "v"(xf[m]));
  };
  auto col_done = [&]() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(acc)); };
  auto frag = [&](int m, int aslot, int bslot) -> bf16x8 {
    if (m < C::KB1)
      return *reinterpret_cast<const bf16x8*>(smem + aslot + ((m & 4) ? a_hi : a_lo) + 32 * m);
    const int n = (m - C::KB1) % C::NT, k = (m - C::KB1) / C::NT;
    return *reinterpret_cast<const bf16x8*>(smem + bslot + (k ? b_off1 : b_off0) + n * 32 * (kFC * 2));
  };
  // row-product operands: hp0 / hp1 = features 0-15 / 16-31 of chunk c-1;
  // hc0 = features 0-15 of chunk c (ready for the next step)
  u32x4 hp0, hp1, hc0;
  auto row_mfma = [&](int m, const bf16x8& f) {
    const int n = (m - C::KB1) % C::NT, k = (m - C::KB1) / C::NT;
    P[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, k ? hp1 : hp0), f, P[n], 0, 0, 0);
  };
  // Activation in four stages per pair of accumulator registers, so that it
  // spreads over the MFMAs: the first half of chunk c (registers 0-7) during
  // the row product of chunk c-1, the second half (registers 8-15, kept in
  // accs) during the column product of chunk c+1.  Register v of lane
  // (l32, lh) holds feature 8(v/4) + 4lh + v%4; once a 16-feature half is
  // packed, two swaps give lane half h features 8h..8h+7, the operand order.
  float accs[8];
  // the chunk's bias as the column product's initial accumulator: register
  // v of lane (l32, lh) is feature 8(v/4) + 4lh + v%4
  auto load_bias = [&](int c) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx4 b = *reinterpret_cast<const floatx4*>(bias_lane + c * kFC + 8 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) bvec[4 * q + e] = b[e];
    }
  };
  // GELU of one register in four stages, the arithmetic of gelu_bf16out
  float g_t, g_w, g_f, g_e, g_r0;
  uint32_t d[4];
  auto finish = [&](int i, float r) {
    if (i & 1)
      d[i >> 1] = pack_bf16(g_r0, r);
    else
      g_r0 = r;
  };
  auto act_stage = [&](int st, int i, float z) {
    if constexpr (GELU) {
      // gelu_bf16out in four stages: the tail polynomial's Horner steps
      // spread over the first three, its exp2 in the third
      if (st == 0) {
        g_t = fminf(fabsf(z), kQxMax);
        g_w = z * kGeluNegHalfLog2e;
        g_f = fmaf(fmaf(kQc6, g_t, kQc5), g_t, kQc4);
      } else if (st == 1) {
        g_f = fmaf(fmaf(fmaf(g_f, g_t, kQc3), g_t, kQc2), g_t, kQc1);
      } else if (st == 2) {
        g_e = __builtin_amdgcn_exp2f(fmaf(g_w, z, fmaf(g_f, g_t, kQc0)));
      } else {
        finish(i, fmaf(-fabsf(z), g_e, fmaxf(z, 0.0f)));
      }
    } else {
      if (st == 3) finish(i, z);
    }
  };
  auto swap_pack = [&]() -> u32x4 {
    const auto s0 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
    return u32x4{s0[0], s1[0], s0[1], s1[1]};
  };
  // stage j (0..31) of the first half (registers 0-7 of acc) or the second
  // (accs); element j/4, stage j%4
  auto act_slot = [&](int half, int j) {
    const int i = j >> 2, st = j & 3;
    act_stage(st, i, half ? accs[i] : acc[i]);
  };
  constexpr int kLoads = C::A_DMA + C::B_DMA;
  static_assert(2 * kLoads <= C::KB1, "load placement");
  // 32 activation stages per half: SA per column / SB per row MFMA
  constexpr int SA = 32 / C::KB1, SB = 32 / (2 * C::NT);
  static_assert(SA >= 1 && SB >= 1 && SA * C::KB1 == 32 && SB * 2 * C::NT == 32, "activation placement");
  constexpr int NM = C::KB1 + 2 * C::NT;
  constexpr int PD = 2;  // fragment reads run PD MFMAs ahead

  // chunk 0: column product and the first half of its activation
  wait_vmcnt<0>();
  lds_barrier();
  if (nchunk > 1) issue_a(1, 1);
  issue_b(0, 0);
  load_bias(0);
  static_for<0, C::KB1>([&](auto mc) { col_mfma(decltype(mc)::value, frag(decltype(mc)::value, 0, 0)); });
  col_done();
  static_for<0, 32>([&](auto jc) { act_slot(0, decltype(jc)::value); });
  hc0 = swap_pack();
#pragma unroll
  for (int v = 0; v < 8; ++v) accs[v] = acc[8 + v];

  // chunk c (1 <= c < nchunk): A_c is in A slot c&1, B_{c-1} in B slot
  // (c-1)&1; A_{c+1} and B_c are loaded during the step
  for (int c = 1; c < nchunk; ++c) {
    const int par = c & 1;
    const int aslot = par * C::A_SLOT, bslot = C::B_OFF + (par ^ 1) * C::B_SLOT;
    hp0 = hc0;
    wait_vmcnt<0>();
    lds_barrier();
    const bool more = c + 1 < nchunk;
    load_bias(c);
    bf16x8 fr[PD + 1];
#pragma unroll
    for (int m = 0; m < PD; ++m) fr[m] = frag(m, aslot, bslot);
    static_for<0, NM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if (m + PD < NM) fr[(m + PD) % (PD + 1)] = frag(m + PD, aslot, bslot);
      if (m < C::KB1)
        col_mfma(m, fr[m % (PD + 1)]);
      else
        row_mfma(m, fr[m % (PD + 1)]);
      if ((m & 1) && (m >> 1) < kLoads) {
        const int j = m >> 1;  // load j of chunk c+1's A part, then of chunk c's B part
        if (j < C::A_DMA)
          dma_a(par ^ 1, j, c + 1, more);
        else
          dma_b(par, j - C::A_DMA, c);
      }
      // column product of chunk c: the second half of chunk c-1's
      // activation; row product of chunk c-1: the first half of chunk c's
      if (m < C::KB1) {
        static_for<0, SA>([&](auto sc) { act_slot(1, m * SA + decltype(sc)::value); });
        if (m == C::KB1 - 1) hp1 = swap_pack();
      } else {
        const int r = m - C::KB1;
        if (r == 0) {
          col_done();
#pragma unroll
          for (int v = 0; v < 8; ++v) accs[v] = acc[8 + v];
        }
        static_for<0, SB>([&](auto sc) { act_slot(0, r * SB + decltype(sc)::value); });
        if (m == NM - 1) hc0 = swap_pack();
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // last chunk: the second half of its activation, then its row product
  {
    const int bslot = C::B_OFF + ((nchunk - 1) & 1) * C::B_SLOT;
    hp0 = hc0;
    static_for<0, 32>([&](auto jc) { act_slot(1, decltype(jc)::value); });
    hp1 = swap_pack();
    wait_vmcnt<0>();
    lds_barrier();
    static_for<C::KB1, NM>([&](auto mc) { row_mfma(decltype(mc)::value, frag(decltype(mc)::value, 0, bslot)); });
  }

  // P_i rows: register v of tile n holds token 8(v/4) + 4lh + v%4, output
  // column 32n + l32 -- each store instruction writes two 128-byte row runs
  float* const Pi = p.P + shard * p.sP;
  const int trow0 = tok0 + w * kTokWave + 4 * lh;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = trow0 + 8 * (v >> 2) + (v & 3);
    if (t < p.T) {
      float* dst = Pi + (int64_t)t * p.ldp + l32;
#pragma unroll
      for (int n = 0; n < C::NT; ++n) dst[32 * n] = P[n][v];
    }
  }
}

template <class C>
hipError_t launch_cfg(const FusedMlpParams& p, hipStream_t s) {
  const int tblocks = (p.T + kTokBlock - 1) / kTokBlock;
  const dim3 g((unsigned)(tblocks * p.shards)), b(kFThreads);
  if (p.act == FUSED_GELU)
    launch_kernel((mlp_fused_kernel<C, true>), g, b, 0, s, p, tblocks);
  else
    launch_kernel((mlp_fused_kernel<C, false>), g, b, 0, s, p, tblocks);
  return hipGetLastError();
}

}  // namespace

bool mlp_fused_supported(int64_t H, int64_t Fs) {
  return (H == 256 || H == 512) && Fs > 0 && Fs % kFC == 0 && Fs <= kBiasMax;
}

hipError_t launch_mlp_fused(const FusedMlpParams& p, hipStream_t s) {
  if (p.T <= 0 || p.shards <= 0) return hipSuccess;
  if (!mlp_fused_supported(p.H, p.Fs)) return hipErrorInvalidValue;
  return p.H == 512 ? launch_cfg<FC<16>>(p, s) : launch_cfg<FC<8>>(p, s);
}

}  // namespace tp
