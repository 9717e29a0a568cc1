// One shard's whole MLP in one kernel, for narrow hidden sizes (H = 256, 512):
//
//   P_i = act(X A_i^T + a_i) B_i^T        (fp32 partial, no row bias)
//
// The column product, the activation on the shard-local slice and the row
// partial follow each other with no communication in between (2kiu.com blog
// post, section 2.3; "张量并行", MLP formula GELU(XA)B), so the shard-local
// intermediate H_i never has to leave the chip: it lives in registers, 32
// intermediate features at a time, between the two products.  The partials
// are the same as those of the separate column and row kernels up to the
// fp32 summation order inside the products.
//
// Layout of the work (gfx950, 4 waves = one per SIMD, 1 workgroup per CU):
//  * A workgroup owns 128 tokens of one shard; wave w owns tokens 32w..32w+31.
//    Its X rows stay in VGPRs for the whole kernel (the MFMA's second operand
//    of the column product), its [32 x H] fp32 partial in AGPRs.
//  * The intermediate features are consumed in chunks of 32.  Per chunk, the
//    column product H^T[32 f x 32 tok] = A_i[f rows] X^T is one chain of
//    H/16 v_mfma_f32_32x32x16_bf16, the activation runs on its 16
//    accumulators per lane, and the row product P += H B_i^T[f rows] is
//    2*H/32 MFMAs, the activated chunk being the MFMA's first operand.
//  * The accumulator layout of the column product gives each lane one token
//    and 16 features; two v_permlane32_swap per 16 features move them into
//    the operand layout of the row product (8 consecutive features per lane
//    half), so no LDS round trip is needed.
//  * A_i and B_i chunks (32 KB each at H = 512) stream through a two-slot LDS
//    ring by buffer loads to LDS, XOR-swizzled so that the 16-byte fragment
//    reads are bank-conflict free; one barrier per chunk.
//  * Software pipeline: each chunk step issues the column product of chunk c
//    (with the loads of chunk c's B part and chunk c+1's A part between its
//    MFMAs), then the row product of chunk c-1, between whose MFMAs the
//    activation of chunk c runs: a wave hides a few vector instructions
//    behind each of its own MFMAs.
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
  static constexpr int LDS = BIAS_OFF + kBiasMax * 2;
  static_assert((RPD == 1 || RPD == 2) && (kFC / 4) % RPD == 0, "A chunk rows per wave");
  static_assert(H % 64 == 0 && B_DMA >= 1, "B chunk rows per wave");
};

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
    char* bl = smem + C::BIAS_OFF;
    const bf16* bg = p.bias ? static_cast<const bf16*>(p.bias) + shard * p.sBias : nullptr;
    for (int i = tid; i < Fs / 8; i += kFThreads) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (bg) v = *reinterpret_cast<const u32x4*>(bg + 8 * i);
      *reinterpret_cast<u32x4*>(bl + 16 * i) = v;
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
  const char* const bias_lane = smem + C::BIAS_OFF + 8 * lh;

  // One chunk step is a sequence of NM MFMAs: the column product of chunk c
  // (k-blocks 0..KB1-1) into acc, then the row product of chunk c-1 (k-block
  // 0 over the NT output tiles, then k-block 1) from hp, the activated chunk
  // c-1.  The activation of chunk c runs during the row product and fills hc.
  constexpr int NM = C::KB1 + 2 * C::NT;
  constexpr int PD = 2;  // fragment reads run PD MFMAs ahead
  // fragment of MFMA m; aslot / bslot are the byte offsets of the A and B
  // ring slots in use
  auto frag = [&](int m, int aslot, int bslot) -> bf16x8 {
    if (m < C::KB1)
      return *reinterpret_cast<const bf16x8*>(smem + aslot + ((m & 4) ? a_hi : a_lo) + 32 * m);
    const int n = (m - C::KB1) % C::NT, k = (m - C::KB1) / C::NT;
    return *reinterpret_cast<const bf16x8*>(smem + bslot + (k ? b_off1 : b_off0) + n * 32 * (kFC * 2));
  };
  floatx16 acc;
  u32x4 hp[2], hc[2];  // activated chunk (c-1, c) in the row product's operand layout
  auto mfma = [&](int m, const bf16x8& f) {
    if (m < C::KB1) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, xf[m], acc, 0, 0, 0);
    } else {
      const int n = (m - C::KB1) % C::NT, k = (m - C::KB1) / C::NT;
      P[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, hp[k]), f, P[n], 0, 0, 0);
    }
  };
  // Activation of accumulator registers 2e, 2e+1 of chunk c (register v of
  // lane (l32, lh) holds feature 8(v/4) + 4lh + v%4), packed to bf16.
  // Lane half 0 holds features {0-3, 8-11} (+16k), half 1 {4-7, 12-15}
  // (+16k); once a 16-feature block is packed, two swaps give half h
  // features 8h..8h+7 (+16k), the operand order.
  uint32_t d[8];
  // the chunk's bias pairs for this lane, read before the chunk's fragment
  // reads so that waiting for them never waits for a fragment
  uint32_t bias2[8];
  auto load_bias = [&](int c) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint2 b = *reinterpret_cast<const uint2*>(bias_lane + (c * kFC + 8 * q) * 2);
      bias2[2 * q] = b.x;
      bias2[2 * q + 1] = b.y;
    }
  };
  auto act_pair = [&](int e, int c) {
    const int v = 2 * e;
    const uint32_t b2 = bias2[e];
    const float z0 = acc[v] + __builtin_bit_cast(float, b2 << 16);
    const float z1 = acc[v + 1] + __builtin_bit_cast(float, b2 & 0xffff0000u);
    d[e] = GELU ? pack_bf16(gelu_bf16out(z0), gelu_bf16out(z1)) : pack_bf16(z0, z1);
    if ((e & 3) == 3) {
      const int k = e >> 2;
      const auto s0 = __builtin_amdgcn_permlane32_swap(d[4 * k + 0], d[4 * k + 2], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(d[4 * k + 1], d[4 * k + 3], false, false);
      hc[k] = u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
  };
  constexpr int kLoads = C::A_DMA + C::B_DMA;
  static_assert(2 * kLoads <= C::KB1, "load placement");
  static_assert(2 * C::NT >= 16, "activation placement: one bf16 pair per two row-product MFMAs");

  // chunk 0: column product and activation
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  wait_vmcnt<0>();
  lds_barrier();
  if (nchunk > 1) issue_a(1, 1);
  issue_b(0, 0);
  load_bias(0);
#pragma unroll
  for (int m = 0; m < C::KB1; ++m) mfma(m, frag(m, 0, 0));
#pragma unroll
  for (int e = 0; e < 8; ++e) act_pair(e, 0);

  // chunk c (1 <= c < nchunk): A_c is in A slot c&1, B_{c-1} in B slot
  // (c-1)&1; A_{c+1} and B_c are loaded during the step
  for (int c = 1; c < nchunk; ++c) {
    const int par = c & 1;
    const int aslot = par * C::A_SLOT, bslot = C::B_OFF + (par ^ 1) * C::B_SLOT;
    hp[0] = hc[0];
    hp[1] = hc[1];
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    wait_vmcnt<0>();
    lds_barrier();
    const bool more = c + 1 < nchunk;
    load_bias(c);
    bf16x8 fr[PD + 1];
#pragma unroll
    for (int m = 0; m < PD; ++m) fr[m] = frag(m, aslot, bslot);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + PD < NM) fr[(m + PD) % (PD + 1)] = frag(m + PD, aslot, bslot);
      mfma(m, fr[m % (PD + 1)]);
      if ((m & 1) && (m >> 1) < kLoads) {
        const int j = m >> 1;  // load j of chunk c+1's A part, then of chunk c's B part
        if (j < C::A_DMA)
          dma_a(par ^ 1, j, c + 1, more);
        else
          dma_b(par, j - C::A_DMA, c);
      }
      // the row product's MFMAs carry the activation of chunk c, one pair
      // per two MFMAs (the first waits for the column product's last MFMA)
      if (m >= C::KB1 && ((m - C::KB1) & 1) && ((m - C::KB1) >> 1) < 8) act_pair((m - C::KB1) >> 1, c);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // last chunk's row product
  {
    const int bslot = C::B_OFF + ((nchunk - 1) & 1) * C::B_SLOT;
    hp[0] = hc[0];
    hp[1] = hc[1];
    wait_vmcnt<0>();
    lds_barrier();
#pragma unroll
    for (int m = C::KB1; m < NM; ++m) mfma(m, frag(m, 0, bslot));
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
