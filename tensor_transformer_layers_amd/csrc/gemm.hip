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
// bf16 path: 256 threads = 4 waves in a 2x2 grid; each wave owns a
// (BM/2) x (BN/2) block of 32x32 output tiles computed with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulate).  A and B tiles are staged
// global -> registers -> LDS (double-buffered, rows padded by 16 bytes so the
// per-lane 16-byte reads of 32 consecutive rows hit distinct banks); the loads
// of tile k+1 are in flight while tile k feeds the matrix cores.  Workgroup
// ids are renumbered so that neighbouring output tiles run on the same XCD.
//
// fp32 path: 64x64 tiles, v_mfma_f32_16x16x4_f32, used for fp32 workloads.
#include "tp_device.hpp"
#include "tp_kernels.hpp"

namespace tp {
namespace {

constexpr int kThreads = 256;
constexpr int kPad = 8;  // bf16 elements of padding per LDS row (16 bytes)

template <int BM, int BN, int BK, int EPI>
struct TileCfg {
  static constexpr int WM = BM / 2, WN = BN / 2;    // wave tile, 2x2 waves
  static constexpr int TM = WM / 32, TN = WN / 32;  // 32x32 MFMA tiles per wave
  static constexpr int LDK = BK + kPad;
  static constexpr int CPR = BK / 8;                // 16-byte chunks per tile row
  static constexpr int RPP = kThreads / CPR;        // tile rows per load pass
  static constexpr int CA = BM / RPP;               // load passes (chunks) per thread, A
  static constexpr int CB = BN / RPP;
  static constexpr int OUT_N = (EPI == EPI_SWIGLU) ? BN / 2 : BN;  // output columns per tile
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must split evenly over passes");
  static_assert(EPI != EPI_SWIGLU || (BN / 2) % RPP == 0, "gate/up halves per pass");
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU needs gate and up subtiles");
};

// Output row of accumulator element v of a 32x32 tile for lane group lg.
__device__ __forceinline__ int acc_row(int v, int lg) { return ((v >> 2) << 3) + (lg << 2) + (v & 3); }

template <int BM, int BN, int BK, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmParams p, int tilesM, int tilesN) {
  using C = TileCfg<BM, BN, BK, EPI>;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (BM + BN) * C::LDK];
  bf16* const As = smem;                    // [2][BM][LDK]
  bf16* const Bs = smem + 2 * BM * C::LDK;  // [2][BN][LDK]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lg = lane >> 5;

  // tile coordinates: XCD-aware renumbering, then groups of 8 M-tiles so that
  // tiles resident on one XCD share A rows and B columns in its L2
  const int per_batch = tilesM * tilesN;
  const int pid = xcd_remap(blockIdx.x, gridDim.x);
  const int bz = pid / per_batch;
  const int t = pid - bz * per_batch;
  constexpr int G = 8;
  const int group = t / (G * tilesN);
  const int first_m = group * G;
  const int gm = min(tilesM - first_m, G);
  const int tin = t - group * G * tilesN;
  const int tm = first_m + tin % gm;
  const int tn = tin / gm;
  const int m0 = tm * BM;
  const int n0 = tn * C::OUT_N;

  const bf16* const A = static_cast<const bf16*>(p.A) + bz * p.sA;
  const bf16* const B = static_cast<const bf16*>(p.B) + bz * p.sB;

  const int lrow = tid / C::CPR;
  const int lcol = (tid % C::CPR) * 8;

  u32x4 ra[C::CA], rb[C::CB];

  auto load_tile = [&](int k0) {
    const bool kok = (k0 + lcol) < p.K;  // K is a multiple of 8: chunks are all-in or all-out
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int gr = m0 + lrow + i * C::RPP;
      if (kok && gr < p.M)
        ra[i] = *reinterpret_cast<const u32x4*>(A + (int64_t)gr * p.lda + k0 + lcol);
      else
        ra[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < C::CB; ++i) {
      const int r = lrow + i * C::RPP;
      int gr;
      const bf16* base;
      if constexpr (EPI == EPI_SWIGLU) {
        const bool up = i >= (BN / 2) / C::RPP;  // gate rows fill the first passes, up rows the rest
        gr = n0 + (up ? r - BN / 2 : r);
        base = up ? B + p.upOff : B;
      } else {
        gr = n0 + r;
        base = B;
      }
      if (kok && gr < p.N)
        rb[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)gr * p.ldb + k0 + lcol);
      else
        rb[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  auto store_tile = [&](int buf) {
    bf16* as = As + buf * BM * C::LDK;
    bf16* bs = Bs + buf * BN * C::LDK;
#pragma unroll
    for (int i = 0; i < C::CA; ++i)
      *reinterpret_cast<u32x4*>(as + (lrow + i * C::RPP) * C::LDK + lcol) = ra[i];
#pragma unroll
    for (int i = 0; i < C::CB; ++i)
      *reinterpret_cast<u32x4*>(bs + (lrow + i * C::RPP) * C::LDK + lcol) = rb[i];
  };

  // LDS row of B subtile nt for this wave (gate subtiles first for SwiGLU)
  auto brow = [&](int nt) -> int {
    if constexpr (EPI == EPI_SWIGLU)
      return nt < C::TN / 2 ? wn * (BN / 4) + nt * 32 : BN / 2 + wn * (BN / 4) + (nt - C::TN / 2) * 32;
    else
      return wn * C::WN + nt * 32;
  };

  floatx16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (p.K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * BK);  // in flight during the MFMAs below

    const bf16* as = As + cur * BM * C::LDK + (wm * C::WM + lr) * C::LDK + 8 * lg;
    const bf16* bs = Bs + cur * BN * C::LDK + lr * C::LDK + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[C::TM], bfr[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(as + i * 32 * C::LDK + kk * 16);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(bs + brow(j) * C::LDK + kk * 16);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }

    if (kt + 1 < nk) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  const int mw = m0 + wm * C::WM;
  if constexpr (EPI == EPI_SWIGLU) {
    bf16* Cp = static_cast<bf16*>(p.C) + bz * p.sC;
#pragma unroll
    for (int j = 0; j < C::TN / 2; ++j) {
      const int n = n0 + wn * (BN / 4) + j * 32 + lr;
      if (n >= p.N) continue;
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = mw + i * 32 + acc_row(v, lg);
          if (m < p.M) {
            const float g = acc[i][j][v], u = acc[i][j + C::TN / 2][v];
            Cp[(int64_t)m * p.ldc + n] = to_bf16(silu(g) * u);
          }
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int n = n0 + wn * C::WN + j * 32 + lr;
      if (n >= p.N) continue;
      float bias = 0.0f;
      if constexpr (EPI != EPI_PARTIAL) {
        if (p.bias) bias = static_cast<float>(static_cast<const bf16*>(p.bias)[bz * p.sBias + n]);
      }
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = mw + i * 32 + acc_row(v, lg);
          if (m >= p.M) continue;
          const int64_t off = bz * p.sC + (int64_t)m * p.ldc + n;
          const float x = acc[i][j][v];
          if constexpr (EPI == EPI_PARTIAL) {
            static_cast<float*>(p.C)[off] = x;
          } else if constexpr (EPI == EPI_GELU) {
            static_cast<bf16*>(p.C)[off] = to_bf16(gelu_erf(x + bias));
          } else {
            static_cast<bf16*>(p.C)[off] = to_bf16(x + bias);
          }
        }
    }
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
    if constexpr (EPI != EPI_PARTIAL) {
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
        else
          *out = x;
      }
  }
}

template <int BM, int BN, int BK, int EPI>
hipError_t launch_bf16_cfg(const GemmParams& p, hipStream_t s) {
  using C = TileCfg<BM, BN, BK, EPI>;
  const int tilesM = (p.M + BM - 1) / BM;
  const int tilesN = (p.N + C::OUT_N - 1) / C::OUT_N;
  const int64_t grid = (int64_t)tilesM * tilesN * p.batch;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, EPI>), dim3((unsigned)grid), dim3(kThreads), 0, s, p,
                     tilesM, tilesN);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_bf16_epi(const GemmParams& p, hipStream_t s) {
  // Large problems take 256x256 tiles (128x128 per wave, LDS traffic per flop
  // halved against 64x64 waves); problems that would not put two tiles on
  // every CU take 128x128 tiles.
  constexpr int kCUs = 256;
  const int out256 = (EPI == EPI_SWIGLU) ? 128 : 256;
  const int64_t big = (int64_t)((p.M + 255) / 256) * ((p.N + out256 - 1) / out256) * p.batch;
  if (big >= 2 * kCUs) return launch_bf16_cfg<256, 256, 64, EPI>(p, s);
  return launch_bf16_cfg<128, 128, 64, EPI>(p, s);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, Epilogue epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_bf16_epi<EPI_STORE>(p, s);
    case EPI_GELU: return launch_bf16_epi<EPI_GELU>(p, s);
    case EPI_PARTIAL: return launch_bf16_epi<EPI_PARTIAL>(p, s);
    case EPI_SWIGLU: return launch_bf16_epi<EPI_SWIGLU>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_f32(const GemmParams& p, Epilogue epi, hipStream_t s) {
  const int tilesM = (p.M + 63) / 64, tilesN = (p.N + 63) / 64;
  const int64_t grid = (int64_t)tilesM * tilesN * p.batch;
  if (grid <= 0) return hipSuccess;
  switch (epi) {
    case EPI_STORE:
      hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, dim3((unsigned)grid), dim3(kThreads), 0, s, p, tilesM, tilesN);
      break;
    case EPI_GELU:
      hipLaunchKernelGGL(gemm_f32_kernel<EPI_GELU>, dim3((unsigned)grid), dim3(kThreads), 0, s, p, tilesM, tilesN);
      break;
    case EPI_PARTIAL:
      hipLaunchKernelGGL(gemm_f32_kernel<EPI_PARTIAL>, dim3((unsigned)grid), dim3(kThreads), 0, s, p, tilesM, tilesN);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tp
