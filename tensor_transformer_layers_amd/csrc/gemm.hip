// Column / row GEMMs of the tensor-parallel linear pair on CDNA4 matrix cores.
//
// C[M x N] = A[M x K] * B[N x K]^T with the activation fused into the
// epilogue.  Both operands are K-contiguous ([out x in] weights, row-major
// activations), so every lane feeds the MFMA with 16-byte reads of 8
// consecutive k values.  Column split: 2kiu.com blog post section 2.1 and
// "Tensor Parallelism基础：模型切分原理" (column-wise splitting); row split and
// its fp32 partial: the same post, section 2.2; activation on the shard-local
// slice between them: section 2.3 and "张量并行" (MLP formula GELU(XA)B).
//
// bf16 path (gfx950):
//  * 256 threads = 4 waves in a 2x2 grid; each wave owns a (BM/2) x (BN/2)
//    block of 32x32 tiles computed with v_mfma_f32_32x32x16_bf16 (fp32
//    accumulators live in AGPRs).  The weight fragment is the MFMA's first
//    operand and the activation fragment its second, so each lane ends up
//    holding one output row and runs of 4 consecutive output columns: the
//    epilogue stores 8-byte (bf16) or 16-byte (fp32) vectors, non-temporal:
//    outputs are read by a later kernel, not by this one, and keeping them out
//    of L2 measurably shortens the store burst at the end of each tile.
//  * Global -> LDS staging uses the buffer-load-to-LDS path (no registers, no
//    LDS write instructions): one wave instruction fills 1 KB of LDS, lane i
//    landing at byte 16*i.  The lane -> global chunk assignment applies an
//    XOR swizzle (chunk c of tile row r sits at chunk c ^ ((r >> 1) & 7))
//    so that the 16-byte fragment reads of consecutive rows hit distinct LDS
//    banks.  Rows past the matrix edge and chunks past K read as zero through
//    the buffer range check; the tail chunks are also cleared explicitly.
//  * Two LDS stages of 64-wide k-tiles, one barrier per tile.  The barrier
//    sits before the last k-step's MFMAs of tile t: after it, tile t's stage
//    is free, and the loads of tile t+2 into it are issued in three parts --
//    during that last k-step and during k-steps 0 and 1 of tile t+1 -- one
//    load instruction after each MFMA, in an order pinned against the
//    scheduler, so the loads stream out between the MFMAs and still have 2-4
//    k-steps to land.  Fragment reads of k-step kk+1 are issued before the
//    MFMAs of step kk (across the tile boundary too).  A partial k-tile is
//    consumed first, so only the prologue handles K tails.
//  * Workgroup ids are renumbered so that the 256 tiles in flight form a
//    16 x 16 block of the tile grid, each XCD an 8 x 4 sub-block (its L2
//    serves 8 + 4 tile rows of operand), the XCDs sharing rows through the
//    memory-side cache; grids that do not split into such rounds keep groups
//    of 8 M-tiles per XCD.
//
// fp32 path: 64x64 tiles, v_mfma_f32_16x16x4_f32, used for fp32 workloads.
#include <math.h>

#include <type_traits>

#include "tp_device.hpp"
#include "tp_dma.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int kThreads = 256;

// Swizzle shift of the LDS layout (16 consecutive rows hit 16 bank groups).
constexpr int kGemmSwizzleShift = 1;

// AKO_ / BKO_: the A (B) operand is stored K-outer, [K x M] ([K x N]) with
// the M (N) index contiguous, instead of K-contiguous rows.
template <int BM_, int BN_, int BK_, int S_, int SH_, int EPI_, bool AKO_ = false, bool BKO_ = false>
struct G {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_, SH = SH_, EPI = EPI_;
  static constexpr bool AKO = AKO_, BKO = BKO_;
  static constexpr int CPR = BK / 8;         // 16-byte chunks per tile row
  static constexpr int RPI = 64 / CPR;       // tile rows one wave load instruction fills
  static constexpr int IA = BM / (4 * RPI);  // load instructions per wave per stage, A tile
  static constexpr int IB = BN / (4 * RPI);  //                                        B tile
  static constexpr int GROUP = IA + IB;
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int STAGE_BYTES = (BM + BN) * BK * 2;
  static constexpr int LDS_BYTES = S * STAGE_BYTES;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int KK = BK / 16;
  static constexpr int OUT_N = is_swiglu_fwd(EPI) ? BN / 2 : BN;
  static_assert(IA >= 1 && IB >= 1 && BM % (4 * RPI) == 0 && BN % (4 * RPI) == 0, "load split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(S >= 2 && (S - 2) * GROUP < 64, "vmcnt range");
  static_assert((32 >> SH) % CPR == 0, "swizzle must repeat every 32 rows");
  static_assert(!is_swiglu_fwd(EPI) || (TN % 2 == 0 && (BN / 4) % 32 == 0), "SwiGLU halves");
  static_assert(!(AKO || BKO) || (BK == 64 && (BM == 128 || BM == 256) && (BN == 128 || BN == 256) &&
                                  !is_swiglu_fwd(EPI) && EPI != EPI_GELU_FUSED), "K-outer operands");
};

// K-outer operand tiles in LDS: k row r of a tile (BMN columns, 2*BMN bytes)
// at r * 2*BMN; its 64-byte blocks are XOR-ed with (r & 3) ^ 2*bit3(r) and
// its 32-byte halves with bit3(r), so that the transposing fragment reads
// (ds_read_b64_tr_b16: 16 lanes read 4 k rows x 16 columns) spread over the
// banks.  As a mask on the 16-byte chunk index of the row (an involution):
__device__ __forceinline__ int ko_chunk_mask(int r) {
  const int b3 = (r >> 3) & 1;
  return ((((r & 3) ^ (b3 << 1)) << 2) | (b3 << 1));
}

template <class C>
__device__ __forceinline__ int swz(int r) {
  return (r >> C::SH) & (C::CPR - 1);
}

// Waves per SIMD the register allocation must allow: the two-pass GELU
// kernel runs on 128x128 tiles and needs two workgroups per CU to hide its
// epilogues; every other variant leaves the choice to the compiler.
template <class C>
constexpr int kWavesPerEu = C::EPI == EPI_GELU_FUSED ? 2 : 1;

template <class C>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEu<C>)))
void gemm_bf16_kernel(GemmParams p, int tilesM, int tilesN) {
  // The operand stages.  With a K-outer operand, one LDS array per stage: the
  // compiler inserts a wait on every outstanding LDS-bound load before a
  // transposing LDS read unless it can tell the two apart, and separate arrays
  // let it see that the fragment reads of one stage never touch the stage the
  // in-flight loads fill.  Otherwise one array (every stage offset then folds
  // into the per-lane fragment offsets).
  static_assert(C::S == 2 && C::LDS_BYTES == 2 * C::STAGE_BYTES, "two stages");
  constexpr bool kStageArrays = C::AKO || C::BKO;
  __shared__ __attribute__((aligned(1024))) char smem0[kStageArrays ? C::STAGE_BYTES : C::LDS_BYTES];
  __shared__ __attribute__((aligned(1024))) char smem1[kStageArrays ? C::STAGE_BYTES : 1];  // unused otherwise
  auto stage = [&](int st) __attribute__((always_inline)) -> char* {
    if constexpr (kStageArrays)
      return st ? smem1 : smem0;
    else
      return smem0 + st * C::STAGE_BYTES;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  // Tile coordinates: XCD-aware renumbering, then groups of 8 M-tiles so that
  // tiles resident on one XCD share A rows and B columns in its L2.  When
  // every problem of the batch reads the same A (or B) operand -- the shards'
  // column GEMMs all read X -- the batch index joins the N (or M) tile index,
  // so the shards' tiles over the same rows run together and one pass over
  // the shared operand serves all of them.
  const bool shareA = p.sA == 0 && p.batch > 1, shareB = !shareA && p.sB == 0 && p.batch > 1;
  const int vM = shareB ? tilesM * p.batch : tilesM;  // virtual tile grid
  const int vN = shareA ? tilesN * p.batch : tilesN;
  // Problems that share nothing run one after another over the whole chip
  // (workgroups are dispatched in id order), each spread over all XCDs, so
  // that every XCD works on the same problem's operands at a time.
  // With p.xcd_per_problem (many small problems, a multiple of 8 of them:
  // the splits of a split-K product), each problem runs whole on one XCD
  // instead, problem z on XCD z % 8, so its operand blocks are fetched into
  // one L2 only.
  const int tps = vM * vN;
  // Chip-wide rounds (when the tile grid allows them): 256 tiles at a time,
  // one per CU, form a 16 x 16 block of the (virtual) tile grid.  XCD x takes
  // the 8 x 4 sub-block at M offset 8 (x % 2), N offset 4 (x / 2), so each
  // block of 8 M-tiles is shared by 4 XCDs and each block of 4 N-tiles by 2:
  // the rows all XCDs read in one round are 16 + 16 tile rows of operand,
  // fetched from HBM once and from the memory-side cache by the other XCDs,
  // instead of every XCD re-reading its own M-tile rows each round.  Rounds
  // advance along M first, so a block of N-tile rows is read by 16-tile-row
  // M blocks in consecutive rounds.  Measured on the 16384 x 49152 x 12288
  // column product: 9% fewer cycles per tile (shorter waits for the operand
  // loads at the k-tile barriers) than per-XCD M-tile groups.
  const bool chip_rounds = !p.xcd_per_problem && vM % 16 == 0 && vN % 16 == 0 && tps % 256 == 0;
  int bz0, t;
  if (p.xcd_per_problem) {
    const int xcd = (int)blockIdx.x % 8, local = (int)blockIdx.x / 8;
    bz0 = (local / tps) * 8 + xcd;
    t = local % tps;
  } else {
    bz0 = (shareA || shareB) ? 0 : (int)blockIdx.x / tps;
    t = (shareA || shareB) ? xcd_remap(blockIdx.x, gridDim.x) : xcd_remap((int)blockIdx.x - bz0 * tps, tps);
  }
  constexpr int GRP = 8;
  int vm, vn;
  if (chip_rounds) {
    // tps is a multiple of 256, so a problem starts on XCD 0 and the
    // hardware's XCD of workgroup b (b % 8) is also lp % 8
    const int lp = (shareA || shareB) ? (int)blockIdx.x : (int)blockIdx.x - bz0 * tps;
    const int xcd = lp % 8, local = lp / 8;  // local: dispatch order on the XCD
    const int r = local / 32, sl = local % 32;
    const int nMg = vM / 16;
    const int g = r % nMg, h = r / nMg;
    vm = g * 16 + (xcd % 2) * 8 + (sl % 8);
    vn = h * 16 + (xcd / 2) * 4 + sl / 8;
  } else {
    const int group = t / (GRP * vN);
    const int first_m = group * GRP;
    const int gm = min(vM - first_m, GRP);
    const int tin = t - group * GRP * vN;
    vm = first_m + tin % gm;
    vn = tin / gm;
  }
  const int bz = shareA ? vn / tilesN : shareB ? vm / tilesM : bz0;
  const int tm = shareB ? vm - bz * tilesM : vm;
  const int tn = shareA ? vn - bz * tilesN : vn;
  const int m0 = tm * C::BM;
  const int n0 = tn * C::OUT_N;

  // buffer resources: each covers the tile's valid rows, so rows past M / N
  // read as zero.  A K-outer operand's resource ends after the tile's last
  // valid column of k row K-1: columns past M (N) of earlier k rows read
  // whatever lies there inside the matrix, which reaches only accumulator
  // rows (columns) the epilogue never stores.
  const bf16* const Ab = static_cast<const bf16*>(p.A) + bz * p.sA + (C::AKO ? (int64_t)m0 : (int64_t)m0 * p.lda);
  const uint32_t a_rows = (uint32_t)min(C::BM, p.M - m0);
  __amdgpu_buffer_rsrc_t rA =
      make_rsrc(Ab, C::AKO ? (uint32_t)((int64_t)(p.K - 1) * p.lda * 2 + a_rows * 2) : a_rows * (uint32_t)p.lda * 2u);
  const bf16* const Bb = static_cast<const bf16*>(p.B) + bz * p.sB + (int64_t)n0 * p.ldb;
  __amdgpu_buffer_rsrc_t rB;
  int b_row0;  // first B-tile row this wave loads, relative to its buffer
  if constexpr (is_swiglu_fwd(C::EPI)) {
    const uint32_t rows = (uint32_t)min(C::BN / 2, p.N - n0);
    const bool up = w >= 2;  // waves 0,1 load the gate half, waves 2,3 the up half
    rB = make_rsrc(up ? Bb + p.upOff : Bb, rows * (uint32_t)p.ldb * 2u);
    b_row0 = w * C::IB * C::RPI - (up ? C::BN / 2 : 0);
  } else if constexpr (C::BKO) {
    const int64_t cols = min(C::BN, p.N - n0);
    rB = make_rsrc(static_cast<const bf16*>(p.B) + bz * p.sB + n0, (uint32_t)((int64_t)(p.K - 1) * p.ldb * 2 + cols * 2));
    b_row0 = 0;
  } else {
    const uint32_t rows = (uint32_t)min(C::BN, p.N - n0);
    rB = make_rsrc(Bb, rows * (uint32_t)p.ldb * 2u);
    b_row0 = w * C::IB * C::RPI;
  }

  // per-lane byte offsets of the load instructions (k advances through soffset)
  const int lrow = lane / C::CPR, lchunk = lane % C::CPR;
  uint32_t voA[C::IA], voB[C::IB];
  int chA[C::IA], chB[C::IB];
#pragma unroll
  for (int j = 0; j < C::IA; ++j) {
    if constexpr (C::AKO) {  // instruction fills 1024 / (2*BM) k rows of 2*BM bytes
      constexpr int cpr = C::BM * 2 / 16;
      const int r = (w * C::IA + j) * (64 / cpr) + lane / cpr;
      chA[j] = 0;
      voA[j] = (uint32_t)r * (uint32_t)p.lda * 2u + (uint32_t)((lane % cpr) ^ ko_chunk_mask(r)) * 16u;
    } else {
      const int r = (w * C::IA + j) * C::RPI + lrow;  // tile row
      chA[j] = lchunk ^ swz<C>(r);                     // logical chunk this lane fetches
      voA[j] = (uint32_t)r * (uint32_t)p.lda * 2u + (uint32_t)chA[j] * 16u;
    }
  }
#pragma unroll
  for (int j = 0; j < C::IB; ++j) {
    if constexpr (C::BKO) {
      constexpr int cpr = C::BN * 2 / 16;
      const int r = (w * C::IB + j) * (64 / cpr) + lane / cpr;
      chB[j] = 0;
      voB[j] = (uint32_t)r * (uint32_t)p.ldb * 2u + (uint32_t)((lane % cpr) ^ ko_chunk_mask(r)) * 16u;
    } else {
      const int r = (w * C::IB + j) * C::RPI + lrow;
      chB[j] = lchunk ^ swz<C>(r);
      voB[j] = (uint32_t)(b_row0 + j * C::RPI + lrow) * (uint32_t)p.ldb * 2u + (uint32_t)chB[j] * 16u;
    }
  }
  // byte offset of k-tile start k0 for each operand (K-outer: k0 rows)
  const uint32_t kstepA = C::AKO ? (uint32_t)p.lda * 2u : 2u, kstepB = C::BKO ? (uint32_t)p.ldb * 2u : 2u;

  const int K = p.K;
  const int nk = (K + C::BK - 1) / C::BK;  // k-tiles
  const int nfull = K / C::BK;             // k-tiles with no chunk past K
  const bool has_tail = !(C::AKO || C::BKO) && nk > nfull;  // K-outer operands: K % BK == 0 (host-checked)
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // K order: a partial k-tile (K not a multiple of BK) is consumed first, as
  // tile 0, so that every later tile is full.  Tile t covers k from
  // k_begin(t); the accumulation order is fixed, so results are
  // deterministic.
  auto k_begin = [&](int t) -> int { return has_tail ? (t == 0 ? nfull * C::BK : (t - 1) * C::BK) : t * C::BK; };

  // Loads of full k-tile t into stage STG.  Tiles past the end are still
  // issued, through buffer resources of size zero (they read zeros and move
  // no data), so every wave always has the same number of load groups in
  // flight and one vmcnt value serves every tile boundary.
  const __amdgpu_buffer_rsrc_t rZ = make_rsrc(Ab, 0u);
  auto issue = [&](auto stg, int t) {
    constexpr int STG = decltype(stg)::value;
    char* sa = stage(STG) + w * C::IA * 1024;
    char* sb = stage(STG) + C::A_BYTES + w * C::IB * 1024;
    const bool live = t < nk;
    const __amdgpu_buffer_rsrc_t ra = live ? rA : rZ;
    const __amdgpu_buffer_rsrc_t rb = live ? rB : rZ;
    const uint32_t soA = live ? (uint32_t)k_begin(t) * kstepA : 0u, soB = live ? (uint32_t)k_begin(t) * kstepB : 0u;
#pragma unroll
    for (int j = 0; j < C::IA; ++j) dma16(ra, sa + j * 1024, voA[j], soA);
#pragma unroll
    for (int j = 0; j < C::IB; ++j) dma16(rb, sb + j * 1024, voB[j], soB);
  };
  // The partial tile (tile 0 of stage 0): chunks past K read as zero through
  // the range check, and are also cleared once the loads have landed.
  auto issue_partial = [&]() {
    const int k0 = nfull * C::BK;
#pragma unroll
    for (int j = 0; j < C::IA; ++j)
      dma16(rA, smem0 + (w * C::IA + j) * 1024, k0 + 8 * chA[j] < K ? voA[j] : kOob, (uint32_t)k0 * 2u);
#pragma unroll
    for (int j = 0; j < C::IB; ++j)
      dma16(rB, smem0 + C::A_BYTES + (w * C::IB + j) * 1024, k0 + 8 * chB[j] < K ? voB[j] : kOob, (uint32_t)k0 * 2u);
  };
  auto clear_partial = [&]() {
    const int k0 = nfull * C::BK;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < C::IA; ++j)
      if (k0 + 8 * chA[j] >= K) *reinterpret_cast<u32x4*>(smem0 + (w * C::IA + j) * 1024 + lane * 16) = z;
#pragma unroll
    for (int j = 0; j < C::IB; ++j)
      if (k0 + 8 * chB[j] >= K) *reinterpret_cast<u32x4*>(smem0 + C::A_BYTES + (w * C::IB + j) * 1024 + lane * 16) = z;
  };

  // Fragment addressing.  The swizzle of a fragment row depends on the lane
  // only, so one per-lane offset per (stage, k-step) covers every subtile; the
  // subtile itself is a compile-time immediate.
  const int fsw = swz<C>(l32);
  const int b_wave_row = is_swiglu_fwd(C::EPI) ? wn * (C::BN / 4) : wn * C::WN;
  // relative to the stage's array (one array: to smem0, stage 1 at + STAGE_BYTES)
  int foA[2][C::KK], foB[2][C::KK];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const int f = l32 * (C::BK * 2) + (((2 * kk + lh) ^ fsw) << 4) + (kStageArrays ? 0 : st * C::STAGE_BYTES);
      foA[st][kk] = f + wm * C::WM * (C::BK * 2);
      foB[st][kk] = f + C::A_BYTES + b_wave_row * (C::BK * 2);
    }
  auto brow = [](int jn) -> int {  // B-tile row of subtile jn, relative to the wave's first row
    if constexpr (is_swiglu_fwd(C::EPI))
      return jn < C::TN / 2 ? jn * 32 : C::BN / 2 + (jn - C::TN / 2) * 32;
    else
      return jn * 32;
  };
  // K-outer fragments: two ds_read_b64_tr_b16, each giving a lane 4
  // consecutive k of its row.  In each 16-lane group (G = lane / 16) lane
  // 4j + q addresses k row 16kk + 8*lh + 4r + j (r = 0, 1: the read) at
  // columns 16*(G & 1) + 4q .. +3 of the 32-column subtile; lane i of the
  // group then holds column 16*(G & 1) + i, k = 16kk + 8*lh + 4r .. +3.  For
  // those rows (r & 3) = j and bit3(r) = lh, so the swizzle is a lane
  // constant: the per-subtile offsets below hold everything but the
  // (stage, k-step, read) part.
  const int ko_j = (lane & 15) >> 2, ko_q = lane & 3, ko_g1 = (lane >> 4) & 1;
  const int ko_s1 = ko_j ^ (lh << 1);
  int koA[C::AKO ? C::TM : 1], koB[C::BKO ? C::TN : 1];
  if constexpr (C::AKO) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      koA[i] = (8 * lh + ko_j) * (C::BM * 2) + ((((wm * C::WM) / 32 + i) ^ ko_s1) << 6) + ((ko_g1 ^ lh) << 5) + 8 * ko_q;
  }
  if constexpr (C::BKO) {
#pragma unroll
    for (int jn = 0; jn < C::TN; ++jn)
      koB[jn] = C::A_BYTES + (8 * lh + ko_j) * (C::BN * 2) + ((((wn * C::WN) / 32 + jn) ^ ko_s1) << 6) +
                ((ko_g1 ^ lh) << 5) + 8 * ko_q;
  }
  auto tr_pair = [&](char* base, int off, int rowbytes) __attribute__((always_inline)) -> bf16x8 {
    typedef short short4v __attribute__((ext_vector_type(4)));
    const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TP_LDS short4v*)(base + off));
    const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TP_LDS short4v*)(base + off + 4 * rowbytes));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // fragment of A subtile i / B subtile jn, stage STG, k-step kk
  auto frag_a = [&](int stg, int kk, int i) __attribute__((always_inline)) -> bf16x8 {
    if constexpr (C::AKO)
      return tr_pair(stage(stg), 16 * kk * (C::BM * 2) + koA[i], C::BM * 2);
    else
      return *reinterpret_cast<const bf16x8*>(stage(kStageArrays ? stg : 0) + foA[stg][kk] + i * 32 * (C::BK * 2));
  };
  auto frag_b = [&](int stg, int kk, int jn) __attribute__((always_inline)) -> bf16x8 {
    if constexpr (C::BKO)
      return tr_pair(stage(stg), 16 * kk * (C::BN * 2) + koB[jn], C::BN * 2);
    else
      return *reinterpret_cast<const bf16x8*>(stage(kStageArrays ? stg : 0) + foB[stg][kk] + brow(jn) * (C::BK * 2));
  };

  floatx16 acc[C::TN][C::TM];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;
  };
  zero_acc();

  bf16x8 af[2][C::TM], bfg[2][C::TN];
  auto load_frags = [&](auto stg, int kk, int buf) {
    constexpr int STG = decltype(stg)::value;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) af[buf][i] = frag_a(STG, kk, i);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) bfg[buf][j] = frag_b(STG, kk, j);
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfg[buf][j], af[buf][i], acc[j][i], 0, 0, 0);
  };
  static_assert(C::S == 2, "two LDS stages: tile t+2 is issued at the boundary that frees tile t's stage");
  static_assert(C::KK % 2 == 0, "fragment buffers alternate per k-step");
  constexpr int kFrag = C::TM + C::TN;  // fragment reads per k-step
  constexpr int kMfmaPerRead = (C::TM * C::TN) / kFrag;
  static_assert(C::GROUP % kFrag == 0 && (C::TM * C::TN) % kFrag == 0, "interleave pattern");

  // Tile t from stage STG: k-steps 0..KK-2 each prefetch the next step's
  // fragments.  Before the last step's MFMAs comes the tile boundary: wait for
  // tile t+1, barrier (after it stage STG is free), fetch tile t+1's first
  // fragments and issue the loads of tile t+2 into stage STG; the last step's
  // MFMAs cover the latency of both.
  // Load instruction g of this wave's group for a tile into stage STG
  // (g < IA: A-tile row block g, else B-tile row block g - IA).
  auto dma_one = [&](auto stg, int g, const __amdgpu_buffer_rsrc_t& ra, const __amdgpu_buffer_rsrc_t& rb,
                     uint32_t soA, uint32_t soB) {
    constexpr int STG = decltype(stg)::value;
    if (g < C::IA)
      dma16(ra, stage(STG) + (w * C::IA + g) * 1024, voA[g], soA);
    else
      dma16(rb, stage(STG) + C::A_BYTES + (w * C::IB + g - C::IA) * 1024, voB[g - C::IA], soB);
  };
  // A tile's load instructions are spread over the boundary step that frees
  // its stage and the first kParts-1 k-steps of the next tile.
  constexpr int kParts = 3;
  static_assert(kParts >= 1 && kParts <= C::KK - 1, "load parts");
  constexpr int kBoundaryLoads = (C::GROUP + kParts - 1) / kParts;
  constexpr int kStepLoads = kParts > 1 ? (C::GROUP - kBoundaryLoads + kParts - 2) / (kParts - 1) : 0;
  auto body = [&](auto stg, int t) {
    constexpr int STG = decltype(stg)::value;
    using NXT = std::integral_constant<int, STG ^ 1>;
#pragma unroll
    for (int kk = 0; kk < C::KK - 1; ++kk) {
      if (kk < kParts - 1) {
        // k-steps 0..kParts-2: the rest of tile t+1's loads into the other
        // stage, one after each MFMA, with the next k-step's fragment reads
        const bool live = t + 1 < nk;
        const __amdgpu_buffer_rsrc_t ra = live ? rA : rZ;
        const __amdgpu_buffer_rsrc_t rb = live ? rB : rZ;
        const uint32_t soA = live ? (uint32_t)k_begin(t + 1) * kstepA : 0u;
        const uint32_t soB = live ? (uint32_t)k_begin(t + 1) * kstepB : 0u;
        constexpr int NMF = C::TM * C::TN;
        const int lo = kBoundaryLoads + kk * kStepLoads;
        const int nl = min(kStepLoads, C::GROUP - lo);
        constexpr int NQ = NMF > kStepLoads ? NMF : kStepLoads;
        const int cb = kk & 1, nb = cb ^ 1;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          if (q < C::TM)
            af[nb][q] = frag_a(STG, kk + 1, q);
          else if (q < C::TM + C::TN)
            bfg[nb][q - C::TM] = frag_b(STG, kk + 1, q - C::TM);
          if (q < NMF) {
            const int j = q / C::TM, i = q % C::TM;
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfg[cb][j], af[cb][i], acc[j][i], 0, 0, 0);
          }
          if (q < nl) dma_one(NXT{}, lo + q, ra, rb, soA, soB);
          __builtin_amdgcn_sched_barrier(0);
        }
        continue;
      }
      load_frags(stg, kk + 1, (kk + 1) & 1);
      mfmas(kk & 1);
#pragma unroll
      for (int q = 0; q < kFrag; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);             // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerRead, 0);  // MFMA
      }
    }
    wait_vmcnt<0>();
    lds_barrier();
    // The boundary step, in an explicit order the scheduler may not change:
    // each of the last k-step's MFMAs is followed by one fragment read of
    // tile t+1 (while any remain) and one load of tile t+2 into the freed
    // stage, so the load instructions issue between MFMAs instead of in a
    // block (past the last tile the reads see a stale stage, unused).
    {
      constexpr int NB = NXT::value;
      const bool live = t + 2 < nk;
      const __amdgpu_buffer_rsrc_t ra = live ? rA : rZ;
      const __amdgpu_buffer_rsrc_t rb = live ? rB : rZ;
      const uint32_t soA = live ? (uint32_t)k_begin(t + 2) * kstepA : 0u;
      const uint32_t soB = live ? (uint32_t)k_begin(t + 2) * kstepB : 0u;
      constexpr int LB = (C::KK - 1) & 1;
      constexpr int NMF = C::TM * C::TN;
      constexpr int NQ = NMF > kBoundaryLoads ? NMF : kBoundaryLoads;
      static_assert(C::TM + C::TN <= NQ, "every fragment read has a slot");
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q < C::TM)
          af[0][q] = frag_a(NB, 0, q);
        else if (q < C::TM + C::TN)
          bfg[0][q - C::TM] = frag_b(NB, 0, q - C::TM);
        if (q < NMF) {
          const int j = q / C::TM, i = q % C::TM;
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfg[LB][j], af[LB][i], acc[j][i], 0, 0, 0);
        }
        if (q < kBoundaryLoads) dma_one(stg, q, ra, rb, soA, soB);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // GELU' epilogue with one phase (128-column tiles): the pre-activations of
  // the wave's whole output block -- the rows and columns its read-back loop
  // visits, 4 features of one row per lane and row block -- are loaded before
  // the k loop, so their latency hides behind it (WM/4 registers of 8 bytes).
  constexpr bool kZAll = C::EPI == EPI_GELU_BWD && C::TN == 2;
  bf16x4 zall[kZAll ? C::WM / 4 : 1];

  // ---------------------------------------------------------------- epilogue
  // The accumulators go through LDS so that the output leaves in full row
  // segments (16 lanes per 256-byte fp32 row piece, 8-byte bf16 pieces) from
  // a compact loop instead of per-element code.  acc[j][i][4g + e] holds
  // C[m][n] with m = m0 + wm*WM + i*32 + l32 and n = (B-tile row of subtile
  // j) + 8g + 4*lh + e.  Each wave stages its rows x 64 floats per phase in
  // its own 256-byte-row region, 16-byte chunk c of row r stored at chunk
  // c ^ (r & 15) (conflict-free for both the column writes and the row reads).
  // Phase h takes subtiles (2h, 2h+1), or for SwiGLU the gate subtile h and
  // its up subtile h + TN/2.
  auto epilogue = [&](auto mode_tag, void* outC, int64_t out_ldc, int64_t out_sC,
                      const void* out_bias) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_tag)::value;
    // EPI_CE_STATS: the label of each of this lane's epilogue rows, as a
    // shard-local column (out-of-range values simply match no column), loaded
    // once per tile before the staging
    int ce_label[MODE == EPI_CE_STATS ? C::WM / 4 : 1];
    if constexpr (MODE == EPI_CE_STATS) {
      const int64_t vbase = (int64_t)(p.ce.shard0 + bz) * p.N;
  #pragma unroll
      for (int it = 0; it < C::WM / 4; ++it) {
        const int m = m0 + wm * C::WM + it * 4 + (lane >> 4);
        const int64_t y = m < p.M ? (int64_t)p.ce.labels[m] - vbase : -1;
        ce_label[it] = (y >= 0 && y < p.N) ? (int)y : -1000000;
      }
    }
    lds_barrier();  // every wave is done with the operand stages
    // waves 0, 1 stage through the first operand stage, waves 2, 3 the second
    char* const ep = stage(w >> 1) + (w & 1) * (C::WM * 256);
    static_assert(2 * C::WM * 256 <= C::STAGE_BYTES, "epilogue staging fits the operand stages");
    constexpr bool SWI = is_swiglu_fwd(MODE);
  #pragma unroll
    for (int h = 0; h < C::TN / 2; ++h) {
      // GELU' epilogue: the pre-activations of this phase's rows are read in
      // blocks of ZB rows per lane, each block issued one block ahead of its
      // use (the first before the accumulators go to LDS), so the load latency
      // overlaps the staging and the previous block's arithmetic
      constexpr int ZB = C::WM / 4 < 16 ? C::WM / 4 : 16;
      const int zc_n = n0 + wn * C::WN + 64 * h + 4 * (lane & 15);
      auto load_z = [&](int blk, bf16x4* z) {
        const bf16* const zb = static_cast<const bf16*>(p.aux) + bz * p.sAux;
  #pragma unroll
        for (int j = 0; j < ZB; ++j) {
          const int m = m0 + wm * C::WM + (blk + j) * 4 + (lane >> 4);
          z[j] = bf16x4{};
          if (m < p.M && zc_n < p.N) {
            const bf16* zp = zb + (int64_t)m * p.ldaux + zc_n;
            if (zc_n + 3 < p.N)
              z[j] = *reinterpret_cast<const bf16x4*>(zp);
            else
              for (int e = 0; e < 4 && zc_n + e < p.N; ++e) z[j][e] = zp[e];
          }
        }
      };
      bf16x4 zc[ZB];
      if constexpr (MODE == EPI_GELU_BWD && !kZAll) load_z(0, zc);
      // SwiGLU backward: the stored gate and up of the phase's rows, in blocks
      // of GB rows per lane, each block issued one block ahead of its use
      constexpr int GB = ZB < 8 ? ZB : 8;
      auto load_gu = [&](int blk, bf16x4* g, bf16x4* u) {
        const bf16* const gb = static_cast<const bf16*>(p.aux) + bz * p.sAux;
  #pragma unroll
        for (int j = 0; j < GB; ++j) {
          const int m = m0 + wm * C::WM + (blk + j) * 4 + (lane >> 4);
          g[j] = bf16x4{};
          u[j] = bf16x4{};
          if (m < p.M && zc_n < p.N) {
            const bf16* zp = gb + (int64_t)m * p.ldaux + zc_n;
            if (zc_n + 3 < p.N) {
              g[j] = *reinterpret_cast<const bf16x4*>(zp);
              u[j] = *reinterpret_cast<const bf16x4*>(zp + p.upOff);
            } else {
              for (int e = 0; e < 4 && zc_n + e < p.N; ++e) {
                g[j][e] = zp[e];
                u[j][e] = zp[e + p.upOff];
              }
            }
          }
        }
      };
      bf16x4 gc[MODE == EPI_SWIGLU_BWD ? GB : 1], uc[MODE == EPI_SWIGLU_BWD ? GB : 1];
      if constexpr (MODE == EPI_SWIGLU_BWD) load_gu(0, gc, uc);
  #pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int j = SWI ? h + half * (C::TN / 2) : 2 * h + half;
  #pragma unroll
        for (int i = 0; i < C::TM; ++i)
  #pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int r = i * 32 + l32;
            const int c = half * 8 + 2 * g + lh;  // 16-byte chunk: columns 4c .. 4c+3
            const floatx4 v = {acc[j][i][4 * g], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]};
            *reinterpret_cast<floatx4*>(ep + r * 256 + ((c ^ (r & 15)) << 4)) = v;
          }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

      if constexpr (SWI) {
        // 8 lanes per row: gate chunk c, up chunk c + 8 -> 4 outputs
        const int c = lane & 7;
        const int n = n0 + wn * (C::BN / 4) + 32 * h + 4 * c;
        bf16* Cp = static_cast<bf16*>(outC) + bz * out_sC;
  #pragma unroll 2
        for (int it = 0; it < C::WM / 8; ++it) {
          const int r = it * 8 + (lane >> 3);
          const int m = m0 + wm * C::WM + r;
          const floatx4 gv = *reinterpret_cast<const floatx4*>(ep + r * 256 + ((c ^ (r & 15)) << 4));
          const floatx4 uv = *reinterpret_cast<const floatx4*>(ep + r * 256 + (((c + 8) ^ (r & 15)) << 4));
          if (m < p.M && n < p.N) {
            bf16x4 o;
  #pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = to_bf16(silu_bf16out(gv[e]) * uv[e]);
            bf16* dst = Cp + (int64_t)m * out_ldc + n;
            if (n + 3 < p.N)
              __builtin_nontemporal_store(o, reinterpret_cast<bf16x4*>(dst));
            else
              for (int e = 0; e < 4 && n + e < p.N; ++e) dst[e] = o[e];
            if constexpr (MODE == EPI_SWIGLU_Z) {  // the pre-activations, for the backward: [gate | up]
              bf16x4 zg, zu;
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                zg[e] = to_bf16(gv[e]);
                zu[e] = to_bf16(uv[e]);
              }
              bf16* zdst = static_cast<bf16*>(p.C2) + bz * p.sC2 + (int64_t)m * p.ldc2 + n;
              if (n + 3 < p.N) {
                __builtin_nontemporal_store(zg, reinterpret_cast<bf16x4*>(zdst));
                __builtin_nontemporal_store(zu, reinterpret_cast<bf16x4*>(zdst + p.N));
              } else {
                for (int e = 0; e < 4 && n + e < p.N; ++e) {
                  zdst[e] = zg[e];
                  zdst[p.N + e] = zu[e];
                }
              }
            }
          }
        }
      } else if constexpr (MODE == EPI_GELU_BWD) {
        // dZ = dH * GELU'(Z): 16 lanes per row, chunk c -> 4 outputs
        static_assert((C::WM / 4) % ZB == 0, "row blocks");
        const int c = lane & 15;
        const int n = zc_n;
        static_assert(!kZAll || ZB == C::WM / 4, "one row block holds the whole phase");
  #pragma unroll 1
        for (int blk = 0; blk < C::WM / 4; blk += ZB) {
          bf16x4 zn[ZB];
          if constexpr (kZAll) {
  #pragma unroll
            for (int j = 0; j < ZB; ++j) {
              zc[j] = zall[j];
              zn[j] = bf16x4{};
            }
          } else if (blk + ZB < C::WM / 4) {
            load_z(blk + ZB, zn);
          } else {
            for (int j = 0; j < ZB; ++j) zn[j] = bf16x4{};
          }
  #pragma unroll
          for (int j = 0; j < ZB; ++j) {
            const int r = (blk + j) * 4 + (lane >> 4);
            const int m = m0 + wm * C::WM + r;
            const floatx4 v = *reinterpret_cast<const floatx4*>(ep + r * 256 + ((c ^ (r & 15)) << 4));
            if (m < p.M && n < p.N) {
              bf16x4 o;
  #pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = to_bf16(v[e] * gelu_grad_bf16out(static_cast<float>(zc[j][e])));
              bf16* dst = static_cast<bf16*>(outC) + bz * out_sC + (int64_t)m * out_ldc + n;
              if (n + 3 < p.N)
                __builtin_nontemporal_store(o, reinterpret_cast<bf16x4*>(dst));
              else
                for (int e = 0; e < 4 && n + e < p.N; ++e) dst[e] = o[e];
              if (p.C2) {  // GELU(Z) as well, the weight gradient's operand
  #pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = to_bf16(gelu_bf16out(static_cast<float>(zc[j][e])));
                bf16* dst2 = static_cast<bf16*>(p.C2) + bz * p.sC2 + (int64_t)m * p.ldc2 + n;
                if (n + 3 < p.N)
                  __builtin_nontemporal_store(o, reinterpret_cast<bf16x4*>(dst2));
                else
                  for (int e = 0; e < 4 && n + e < p.N; ++e) dst2[e] = o[e];
              }
            }
          }
  #pragma unroll
          for (int j = 0; j < ZB; ++j) zc[j] = zn[j];
        }
      } else if constexpr (MODE == EPI_SWIGLU_BWD) {
        // SwiGLU backward from dH (the accumulators) and the stored gate G and
        // up U of the same token and feature:
        //   dG = dH U SiLU'(G),  dU = dH SiLU(G),  H = SiLU(G) U
        // with SiLU'(g) = s (1 + g (1 - s)), s = sigmoid(g) (hardware exp and
        // reciprocal).  16 lanes per row, 4 features each.
        static_assert((C::WM / 4) % GB == 0, "row blocks");
        const int c = lane & 15;
        const int n = zc_n;
        bf16* const cb = static_cast<bf16*>(outC) + bz * out_sC;
        bf16* const hb = static_cast<bf16*>(p.C2) + bz * p.sC2;
  #pragma unroll 1
        for (int blk = 0; blk < C::WM / 4; blk += GB) {
          bf16x4 gn[GB], un[GB];
          if (blk + GB < C::WM / 4) {
            load_gu(blk + GB, gn, un);
          } else {
            for (int j = 0; j < GB; ++j) gn[j] = un[j] = bf16x4{};
          }
  #pragma unroll
          for (int j = 0; j < GB; ++j) {
            const int r = (blk + j) * 4 + (lane >> 4);
            const int m = m0 + wm * C::WM + r;
            const floatx4 v = *reinterpret_cast<const floatx4*>(ep + r * 256 + ((c ^ (r & 15)) << 4));
            if (m < p.M && n < p.N) {
              bf16x4 og, ou, oh;
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float g = static_cast<float>(gc[j][e]), u = static_cast<float>(uc[j][e]);
                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
                const float si = g * sg;
                og[e] = to_bf16(v[e] * u * (sg * fmaf(g, 1.0f - sg, 1.0f)));
                ou[e] = to_bf16(v[e] * si);
                oh[e] = to_bf16(si * u);
              }
              bf16* const dg = cb + (int64_t)m * out_ldc + n;
              bf16* const hh = hb + (int64_t)m * p.ldc2 + n;
              if (n + 3 < p.N) {
                __builtin_nontemporal_store(og, reinterpret_cast<bf16x4*>(dg));
                __builtin_nontemporal_store(ou, reinterpret_cast<bf16x4*>(dg + p.upOff));
                __builtin_nontemporal_store(oh, reinterpret_cast<bf16x4*>(hh));
              } else {
                for (int e = 0; e < 4 && n + e < p.N; ++e) {
                  dg[e] = og[e];
                  dg[e + p.upOff] = ou[e];
                  hh[e] = oh[e];
                }
              }
            }
          }
  #pragma unroll
          for (int j = 0; j < GB; ++j) {
            gc[j] = gn[j];
            uc[j] = un[j];
          }
        }
      } else if constexpr (MODE == EPI_CE_STATS) {
        // Cross-entropy statistics of this phase's 64 logit columns per token
        // row (16 lanes per row, 4 logits each): the max over the row's real
        // vocab ids, then the sum of exp(l - max) against it, and the label's
        // logit.  Lane 0 of each row group writes the three values; the logits
        // themselves are never stored.
        const int c = lane & 15;
        const int ncol0 = n0 + wn * C::WN + 64 * h;  // first column of the 64-column chunk
        const int n = ncol0 + 4 * c;
        const int64_t vbase = (int64_t)(p.ce.shard0 + bz) * p.N;  // vocab id of the shard's column 0
        const int lim = (int)min((int64_t)p.N, max((int64_t)0, p.ce.V - vbase));  // columns >= lim: padding
        const int k = ncol0 / 64;
        float* const st = p.ce.stats + ((int64_t)bz * p.ce.cps + k) * p.M;
        const auto fmax_ = [](float a, float b) { return fmaxf(a, b); };
        const auto add_ = [](float a, float b) { return a + b; };
  #pragma unroll 4
        for (int it = 0; it < C::WM / 4; ++it) {
          const int r = it * 4 + (lane >> 4);
          const int m = m0 + wm * C::WM + r;
          const floatx4 v = *reinterpret_cast<const floatx4*>(ep + r * 256 + ((c ^ (r & 15)) << 4));
          float mx = -INFINITY;
  #pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < lim) mx = fmaxf(mx, v[e]);
          mx = row16_reduce(mx, fmax_);
          float sum = 0.0f;
  #pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < lim) sum += __expf(v[e] - mx);
          const int y = ce_label[it] - n;  // label column relative to this lane's first logit
          const float z = (y >= 0 && y < 4 && n + y < lim) ? (y == 0 ? v[0] : y == 1 ? v[1] : y == 2 ? v[2] : v[3]) : 0.0f;
          sum = row16_reduce(sum, add_);
          const float zr = row16_reduce(z, add_);  // one lane of the row holds the label, if any
          if (c == 0 && m < p.M && k < p.ce.cps) {
            st[m] = mx;
            st[m + p.ce.astride] = sum;
            st[m + 2 * p.ce.astride] = zr;
          }
        }
      } else {
        // 16 lanes per row: chunk c -> 4 outputs
        const int c = lane & 15;
        const int n = n0 + wn * C::WN + 64 * h + 4 * c;
        float bias[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (MODE != EPI_PARTIAL && MODE != EPI_GELU_BWD && MODE != EPI_CE_STATS &&
                      MODE != EPI_SWIGLU_BWD) {
          if (out_bias) {
            const bf16* bp = static_cast<const bf16*>(out_bias) + bz * p.sBias;
            for (int e = 0; e < 4; ++e) bias[e] = n + e < p.N ? static_cast<float>(bp[n + e]) : 0.0f;
          }
        }
  #pragma unroll 2
        for (int it = 0; it < C::WM / 4; ++it) {
          const int r = it * 4 + (lane >> 4);
          const int m = m0 + wm * C::WM + r;
          const floatx4 v = *reinterpret_cast<const floatx4*>(ep + r * 256 + ((c ^ (r & 15)) << 4));
          if (m < p.M && n < p.N) {
            const int64_t off = bz * out_sC + (int64_t)m * out_ldc + n;
            if constexpr (MODE == EPI_PARTIAL) {
              float* dst = static_cast<float*>(outC) + off;
              if (n + 3 < p.N)
                __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(dst));  // read once, much later
              else
                for (int e = 0; e < 4 && n + e < p.N; ++e) dst[e] = v[e];
            } else {
              bf16x4 o, zo;
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float x = v[e] + bias[e];
                o[e] = to_bf16(MODE == EPI_GELU || MODE == EPI_GELU_Z ? gelu_bf16out(x) : x);
                zo[e] = to_bf16(x);
              }
              bf16* dst = static_cast<bf16*>(outC) + off;
              if (n + 3 < p.N)
                __builtin_nontemporal_store(o, reinterpret_cast<bf16x4*>(dst));
              else
                for (int e = 0; e < 4 && n + e < p.N; ++e) dst[e] = o[e];
              if constexpr (MODE == EPI_GELU_Z) {  // the pre-activation, for the backward
                bf16* zdst = static_cast<bf16*>(p.C2) + bz * p.sC2 + (int64_t)m * p.ldc2 + n;
                if (n + 3 < p.N)
                  __builtin_nontemporal_store(zo, reinterpret_cast<bf16x4*>(zdst));
                else
                  for (int e = 0; e < 4 && n + e < p.N; ++e) zdst[e] = zo[e];
              }
            }
          }
        }
      }
      if (h + 1 < C::TN / 2) {  // the next phase reuses the region
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      }
    }
  };

  if constexpr (kZAll) {
    const bf16* const zb = static_cast<const bf16*>(p.aux) + bz * p.sAux;
    const int zn0 = n0 + wn * C::WN + 4 * (lane & 15);
#pragma unroll
    for (int j = 0; j < C::WM / 4; ++j) {
      const int m = m0 + wm * C::WM + j * 4 + (lane >> 4);
      zall[j] = bf16x4{};
      if (m < p.M && zn0 < p.N) {
        const bf16* zp = zb + (int64_t)m * p.ldaux + zn0;
        if (zn0 + 3 < p.N)
          zall[j] = *reinterpret_cast<const bf16x4*>(zp);
        else
          for (int e = 0; e < 4 && zn0 + e < p.N; ++e) zall[j][e] = zp[e];
      }
    }
  }

  // EPI_GELU_FUSED runs the k loop twice (see below); every other epilogue once.
  constexpr int kPasses = C::EPI == EPI_GELU_FUSED ? 2 : 1;
  floatx16 gp[C::EPI == EPI_GELU_FUSED ? C::TN : 1][C::EPI == EPI_GELU_FUSED ? C::TM : 1];
  for (int pass = 0; pass < kPasses; ++pass) {
    if constexpr (C::EPI == EPI_GELU_FUSED) {
      if (pass == 1) {
        lds_barrier();  // every wave is done with the staging region before pass 2 fills the stages
        zero_acc();
        rA = make_rsrc(static_cast<const bf16*>(p.A2) + bz * p.sA + (int64_t)m0 * p.lda, a_rows * (uint32_t)p.lda * 2u);
        rB = make_rsrc(static_cast<const bf16*>(p.B2) + bz * p.sB + (int64_t)n0 * p.ldb,
                       (uint32_t)min(C::BN, p.N - n0) * (uint32_t)p.ldb * 2u);
      }
    }
    // prologue: tile 0, the boundary part of tile 1, then tile 0's first fragments
    if (has_tail)
      issue_partial();
    else
      issue(I0{}, 0);
    {
      const bool live = 1 < nk;
      const __amdgpu_buffer_rsrc_t ra = live ? rA : rZ;
      const __amdgpu_buffer_rsrc_t rb = live ? rB : rZ;
      const uint32_t soA = live ? (uint32_t)k_begin(1) * kstepA : 0u;
      const uint32_t soB = live ? (uint32_t)k_begin(1) * kstepB : 0u;
  #pragma unroll
      for (int g = 0; g < kBoundaryLoads; ++g) dma_one(I1{}, g, ra, rb, soA, soB);
    }
    wait_vmcnt<kBoundaryLoads>();
    if (has_tail) clear_partial();
    lds_barrier();
    load_frags(I0{}, 0, 0);


    // two tiles per trip so that the stages are compile-time constants
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      body(I0{}, kt);
      body(I1{}, kt + 1);
    }
    if (kt < nk) body(I0{}, kt);
    wait_vmcnt<0>();  // no load may still target this workgroup's LDS when it exits
    if constexpr (C::EPI == EPI_GELU_FUSED) {
      if (pass == 0) {
        // dZ = (dY B) * GELU'(X A^T + a) and H = GELU(X A^T + a) from two
        // passes over the same k range: pass 1 (A = X, B = A rows) leaves the
        // pre-activation in the accumulators; its slope is kept in registers
        // and H goes out through the GELU epilogue; pass 2 (A2 = dY, B2 = B^T
        // rows) computes dH, which is scaled by the slope and stored.  The
        // pre-activation never leaves the chip.
        const bf16* const bias = static_cast<const bf16*>(p.bias) + bz * p.sBias;
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int n = n0 + wn * C::WN + j * 32 + 8 * g + 4 * lh + e;
              const float b = (p.bias && n < p.N) ? static_cast<float>(bias[n]) : 0.0f;
#pragma unroll
              for (int i = 0; i < C::TM; ++i) gp[j][i][4 * g + e] = gelu_grad_bf16out(acc[j][i][4 * g + e] + b);
            }
        epilogue(std::integral_constant<int, EPI_GELU>{}, p.C2, p.ldc2, p.sC2, p.bias);
      }
    }
  }

  if constexpr (C::EPI == EPI_GELU_FUSED) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int i = 0; i < C::TM; ++i) acc[j][i] *= gp[j][i];
    epilogue(std::integral_constant<int, EPI_STORE>{}, p.C, p.ldc, p.sC, nullptr);
  } else {
    epilogue(std::integral_constant<int, C::EPI>{}, p.C, p.ldc, p.sC, p.bias);
  }
}

// ---------------------------------------------------------------- fp32 path
template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmParams p, int tilesM, int tilesN) {
  constexpr int BM = 64, BN = 64, BK = 16, LDK = BK + 4;
  __shared__ __attribute__((aligned(16))) float As[2][BM][LDK];
  __shared__ __attribute__((aligned(16))) float Bs[2][BN][LDK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lq = lane >> 4;

  const int per_batch = tilesM * tilesN;
  const int pid = blockIdx.x;
  const int bz = pid / per_batch;
  const int t = pid - bz * per_batch;
  const int tm = t / tilesN, tn = t - (t / tilesN) * tilesN;
  const int m0 = tm * BM, n0 = tn * BN;

  const float* const A = static_cast<const float*>(p.A) + bz * p.sA;
  const float* const B = static_cast<const float*>(p.B) + bz * p.sB;
  const int lrow = tid >> 2, lcol = (tid & 3) * 4;

  floatx4 ra, rb;
  auto load_tile = [&](int k0) {
    const bool kok = (k0 + lcol) < p.K;  // K is a multiple of 4
    const int am = m0 + lrow, bn = n0 + lrow;
    ra = (kok && am < p.M) ? *reinterpret_cast<const floatx4*>(A + (int64_t)am * p.lda + k0 + lcol)
                           : floatx4{0.f, 0.f, 0.f, 0.f};
    rb = (kok && bn < p.N) ? *reinterpret_cast<const floatx4*>(B + (int64_t)bn * p.ldb + k0 + lcol)
                           : floatx4{0.f, 0.f, 0.f, 0.f};
  };
  auto store_tile = [&](int buf) {
    *reinterpret_cast<floatx4*>(&As[buf][lrow][lcol]) = ra;
    *reinterpret_cast<floatx4*>(&Bs[buf][lrow][lcol]) = rb;
  };

  floatx4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (p.K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 4; ++ks) {
      float af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = As[cur][wm * 32 + i * 16 + l16][ks * 4 + lq];
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = Bs[cur][wn * 32 + j * 16 + l16][ks * 4 + lq];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 32 + j * 16 + l16;
    if (n >= p.N) continue;
    float bias = 0.0f;
    if constexpr (EPI != EPI_PARTIAL && EPI != EPI_GELU_BWD) {
      if (p.bias) bias = static_cast<const float*>(p.bias)[bz * p.sBias + n];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * 32 + i * 16 + lq * 4 + v;
        if (m >= p.M) continue;
        const float x = acc[i][j][v];
        float* out = static_cast<float*>(p.C) + bz * p.sC + (int64_t)m * p.ldc + n;
        if constexpr (EPI == EPI_GELU)
          *out = gelu_erf(x + bias);
        else if constexpr (EPI == EPI_STORE)
          *out = x + bias;
        else if constexpr (EPI == EPI_GELU_BWD)  // dZ = dH * GELU'(Z), Z from aux
          *out = x * gelu_grad_erf(static_cast<const float*>(p.aux)[bz * p.sAux + (int64_t)m * p.ldaux + n]);
        else
          *out = x;
      }
  }
}

template <class C>
hipError_t launch_bf16_cfg(const GemmParams& p, hipStream_t s) {
  const int tilesM = (p.M + C::BM - 1) / C::BM;
  const int tilesN = (p.N + C::OUT_N - 1) / C::OUT_N;
  const int64_t grid = (int64_t)tilesM * tilesN * p.batch;
  if (grid <= 0) return hipSuccess;
  launch_kernel((gemm_bf16_kernel<C>), dim3((unsigned)grid), dim3(kThreads), 0, s, p, tilesM, tilesN);
  return hipGetLastError();
}

template <int EPI, bool AKO = false, bool BKO = false>
hipError_t launch_bf16_epi(const GemmParams& p, hipStream_t s) {
  // 256x256 tiles (128x128 per wave) when they fill every CU at least once;
  // smaller problems take 128x128 tiles, two workgroups per CU.
  constexpr int kCUs = 256;
  const int out256 = is_swiglu_fwd(EPI) ? 128 : 256;
  const int64_t big = (int64_t)((p.M + 255) / 256) * ((p.N + out256 - 1) / out256) * p.batch;
  // The GELU' and SwiGLU-backward epilogues read bf16 tiles of Z beside the
  // accumulators; with a short K (measured on the 16384 x 2048 x 512 GELU'
  // product: 120 us on 256x256 tiles, 95-99 us on 128x128) two 128x128
  // workgroups per CU hide one's epilogue behind the other's MFMAs better
  // than one 256x256 workgroup does.  The SwiGLU-backward product
  // (32768 x 8 x 1376 x 4096) gains the same way at any K when B is
  // K-contiguous (3.96 -> 3.80 ms), but with B read K-outer it is faster on
  // 256x256 tiles (3.22 vs 3.65 ms).
  const bool short_k_load_epilogue =
      (EPI == EPI_GELU_BWD && p.K <= 2048) || (EPI == EPI_SWIGLU_BWD && (p.K <= 2048 || !p.b_ko));
  if (big >= kCUs && !short_k_load_epilogue)
    return launch_bf16_cfg<G<256, 256, 64, 2, kGemmSwizzleShift, EPI, AKO, BKO>>(p, s);
  return launch_bf16_cfg<G<128, 128, 64, 2, kGemmSwizzleShift, EPI, AKO, BKO>>(p, s);
}

// Operands stored K-outer ([K x M] / [K x N], row pitch lda / ldb): the
// backward's products over the token and hidden axes read them as stored.
// K must be a multiple of 64 and (K-1)*ld*2 + 512 below 2^32 (the buffer
// range); the host checks.  M and N may be ragged.
template <int EPI>
hipError_t launch_bf16_ko(const GemmParams& p, hipStream_t s) {
  if constexpr (EPI == EPI_PARTIAL) {
    if (p.a_ko && p.b_ko) return launch_bf16_epi<EPI, true, true>(p, s);
    if (!p.a_ko && p.b_ko) return launch_bf16_epi<EPI, false, true>(p, s);
  } else if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_STORE || EPI == EPI_SWIGLU_BWD) {
    if (!p.a_ko && p.b_ko) return launch_bf16_epi<EPI, false, true>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, Epilogue epi, hipStream_t s) {
  if (p.a_ko || p.b_ko) {
    switch (epi) {
      case EPI_PARTIAL: return launch_bf16_ko<EPI_PARTIAL>(p, s);
      case EPI_GELU_BWD: return launch_bf16_ko<EPI_GELU_BWD>(p, s);
      case EPI_STORE: return launch_bf16_ko<EPI_STORE>(p, s);
      case EPI_SWIGLU_BWD: return launch_bf16_ko<EPI_SWIGLU_BWD>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epi) {
    case EPI_STORE: return launch_bf16_epi<EPI_STORE>(p, s);
    case EPI_GELU: return launch_bf16_epi<EPI_GELU>(p, s);
    case EPI_GELU_Z: return launch_bf16_epi<EPI_GELU_Z>(p, s);
    case EPI_PARTIAL: return launch_bf16_epi<EPI_PARTIAL>(p, s);
    case EPI_SWIGLU: return launch_bf16_epi<EPI_SWIGLU>(p, s);
    case EPI_SWIGLU_Z: return launch_bf16_epi<EPI_SWIGLU_Z>(p, s);
    case EPI_GELU_BWD: return launch_bf16_epi<EPI_GELU_BWD>(p, s);
    case EPI_CE_STATS: return launch_bf16_epi<EPI_CE_STATS>(p, s);
    case EPI_SWIGLU_BWD: return launch_bf16_epi<EPI_SWIGLU_BWD>(p, s);
    case EPI_GELU_FUSED: return launch_bf16_cfg<G<128, 128, 64, 2, kGemmSwizzleShift, EPI_GELU_FUSED>>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_f32(const GemmParams& p, Epilogue epi, hipStream_t s) {
  const int tilesM = (p.M + 63) / 64, tilesN = (p.N + 63) / 64;
  const int64_t grid = (int64_t)tilesM * tilesN * p.batch;
  if (grid <= 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE:
      launch_kernel(gemm_f32_kernel<EPI_STORE>, dim3((unsigned)grid), dim3(kThreads), 0, s, p, tilesM, tilesN);
      break;
    case EPI_GELU:
      launch_kernel(gemm_f32_kernel<EPI_GELU>, dim3((unsigned)grid), dim3(kThreads), 0, s, p, tilesM, tilesN);
      break;
    case EPI_PARTIAL:
      launch_kernel(gemm_f32_kernel<EPI_PARTIAL>, dim3((unsigned)grid), dim3(kThreads), 0, s, p, tilesM, tilesN);
      break;
    case EPI_GELU_BWD:
      launch_kernel(gemm_f32_kernel<EPI_GELU_BWD>, dim3((unsigned)grid), dim3(kThreads), 0, s, p, tilesM, tilesN);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tp
