// Host-visible launch interface of the libtp kernels (internal; the public
// interface is include/tp.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

// Per-kernel timing.  While the library times its kernels, the host code
// arms a start/stop event pair before a launch and the launch attaches it to
// its own dispatch, so the pair spans exactly that kernel's execution (no
// marker packets between kernels).  take_launch_events() returns the armed
// pair (null events when timing is off) and disarms it; tp_api.cpp owns it.
struct LaunchEvents {
  hipEvent_t start, stop;
};
LaunchEvents take_launch_events();

template <typename K, typename... Args>
inline void launch_kernel(K kernel, const dim3& grid, const dim3& block, uint32_t shm, hipStream_t s,
                          Args... args) {
  const LaunchEvents ev = take_launch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, shm, s, ev.start, ev.stop, 0u, args...);
}

// Epilogue applied to the fp32 accumulator tile of a GEMM.
enum Epilogue : int {
  EPI_STORE = 0,   // C = acc (+ bias)              out dtype = input dtype
  EPI_GELU = 1,    // C = GELU(acc + bias)          out dtype = input dtype
  EPI_PARTIAL = 2, // C = acc                       out fp32 (row partial)
  EPI_SWIGLU = 3,  // C = SiLU(acc_gate) * acc_up   out bf16
  EPI_GELU_BWD = 4,  // C = acc * GELU'(Z), Z = aux   out bf16 (bf16 path only)
  EPI_CE_STATS = 5,  // no C: per (row, 64-column chunk) cross-entropy statistics of the logits acc
  EPI_SWIGLU_BWD = 6,  // acc = dH; G, U = aux at n, n + upOff: C[n] = dG, C[n + upOff] = dU, C2 = SiLU(G)*U
  EPI_GELU_FUSED = 7,  // two passes: Z = A B^T + bias, then dH = A2 B2^T; C = dH * GELU'(Z), C2 = GELU(Z)
  EPI_GELU_Z = 8,      // C = GELU(acc + bias), C2 = acc + bias (the pre-activation, kept for the backward); bf16
  EPI_SWIGLU_Z = 9,    // EPI_SWIGLU, and the pre-activations to C2: gate at column n, up at n + N; bf16
};

// The forward SwiGLU epilogues (gate and up rows side by side in one tile).
constexpr bool is_swiglu_fwd(int epi) { return epi == EPI_SWIGLU || epi == EPI_SWIGLU_Z; }

// EPI_CE_STATS: problem z of the batch is vocab shard ce_shard0 + z, whose
// column n is vocab id (ce_shard0 + z)*N + n; ids >= ce_V are padding.  For
// every token row m and 64-column chunk k of the shard (k < ce_cps), the
// epilogue writes, at index (z*ce_cps + k)*M + m of three arrays ce_stats,
// ce_stats + ce_astride, ce_stats + 2*ce_astride: the chunk's max logit
// (-inf if it holds no real id), the sum of exp(logit - max), and the
// logit of ce_labels[m] if the chunk holds that id (else 0).
struct CeEpilogue {
  const int32_t* labels;
  float* stats;
  int64_t astride, V;
  int shard0, cps;
};

// C[M x N] = A[M x K] * B[N x K]^T, batched over `batch` problems whose
// pointers advance by sA/sB/sC/sBias elements.  Operands are K-contiguous
// unless a_ko / b_ko say otherwise.  For EPI_SWIGLU, B holds gate rows at B
// and up rows at B + upOff; N is the output width (gate rows used: N).  For
// EPI_GELU_BWD, aux is a bf16 matrix of the output's shape (ld ldaux,
// advancing by sAux per problem), and C2, when not null, receives GELU(aux).
struct GemmParams {
  const void* A;
  int64_t lda, sA;
  const void* B;
  int64_t ldb, sB;
  void* C;
  int64_t ldc, sC;
  const void* bias;  // [N] per batch or nullptr
  int64_t sBias;
  int64_t upOff;
  const void* aux;
  int64_t ldaux, sAux;
  int M, N, K;
  int batch;
  int xcd_per_problem;  // nonzero: batch % 8 == 0, each problem runs whole on one XCD
  CeEpilogue ce;        // EPI_CE_STATS only
  void* C2;             // EPI_SWIGLU_BWD, EPI_GELU_FUSED, EPI_GELU_Z, EPI_GELU_BWD: second bf16 output
                        // (ld ldc2, advancing by sC2)
  int64_t ldc2, sC2;
  const void* A2;       // EPI_GELU_FUSED: second pass operands (same ld and batch strides as A, B)
  const void* B2;
  int a_ko, b_ko;       // nonzero: A is stored K-outer ([K x M], row pitch lda), B likewise ([K x N], ldb);
                        // bf16, EPI_PARTIAL (A and B, or B only), EPI_GELU_BWD / EPI_STORE /
                        // EPI_SWIGLU_BWD (B only); K a multiple of 64, (K-1)*ld*2 + 512 < 2^32
};

hipError_t launch_gemm_bf16(const GemmParams& p, Epilogue epi, hipStream_t s);
hipError_t launch_gemm_f32(const GemmParams& p, Epilogue epi, hipStream_t s);

// One kernel for the whole MLP of each shard s in [0, shards), narrow hidden
// sizes only (mlp_fused_supported):
//   P + s*sP  [T x H] fp32  =  act(X A_s^T + bias_s) B_s^T
// with A_s = A + s*sA ([Fs x H], ld lda), bias_s = bias + s*sBias ([Fs] or
// nullptr), B_s = B + s*sB ([H x Fs], ld ldb).  bf16 inputs; the activated
// intermediate is rounded to bf16, as the separate column kernel stores it.
enum FusedAct : int { FUSED_NONE = 0, FUSED_GELU = 1 };
struct FusedMlpParams {
  const void* X;
  int64_t ldx;
  const void* A;
  int64_t lda, sA;
  const void* bias;
  int64_t sBias;
  const void* B;
  int64_t ldb, sB;
  float* P;
  int64_t ldp, sP;
  int T, H, Fs, shards;
  int act;
};
bool mlp_fused_supported(int64_t H, int64_t Fs);
hipError_t launch_mlp_fused(const FusedMlpParams& p, hipStream_t s);

// Y[rows x H] = fold_k P[k][row0 + r, :] (+ bias), see tp_reduce_partials.
// Output row r is written at Y + r*ldy (ldy == H: contiguous).
struct ReduceParams {
  const float* P;
  int64_t part_stride;
  int n_parts;
  int64_t rows, H, row0;
  const void* bias;
  void* Y;
  int64_t ldy;
};
hipError_t launch_reduce(const ReduceParams& p, bool out_bf16, hipStream_t s);

// RMSNorm or LayerNorm of sequence slices into the gathered buffer.  Row `row` of the
// launch is row t of slice r (r = slice if slice >= 0, else row / slice_rows),
// read at X + r*slice_stride + t*ldx and written at Y + (r*slice_rows + t)*ldy.
struct NormParams {
  const void* X;
  int64_t slice_stride, ldx;
  const void* gamma;
  void* Y;
  int64_t ldy;
  int64_t rows;        // rows this launch normalizes
  int64_t slice_rows;  // T / n_slices
  int64_t slice;       // -1: every slice
  int H;
  float inv_h, eps;
  const void* beta;    // LayerNorm shift [H] or nullptr
  int layer;           // 0: RMSNorm, 1: LayerNorm
};
int64_t rmsnorm_max_hidden(bool bf16_io);
hipError_t launch_rmsnorm_gather(const NormParams& p, bool bf16_io, hipStream_t s);

// Norm of an input split along hidden into N slices of Hs = H/N columns
// (slice i = columns [i Hs, (i+1) Hs) of X and Y).  Stats: for shards
// [shard0, shard0 + shards) and every row t, the slice's statistic into
// stats[2 (i T + t) .. +1] (RMSNorm: sum of squares, 0; LayerNorm: mean, sum
// of squared deviations).  Apply: for the same shards, the fold of all N
// statistics of the row in shard order, then the slice scaled into Y.
struct NormSplitParams {
  const void* X;
  int64_t ldx;
  const void* gamma;   // [H]
  const void* beta;    // [H] or nullptr (LayerNorm only)
  void* Y;
  int64_t ldy;
  float* stats;        // [N x T x 2]
  int64_t T;
  int Hs, N, shard0, shards;
  float inv_hs, inv_h, eps;
  int layer;
};
hipError_t launch_norm_split_stats(const NormSplitParams& p, bool bf16_io, hipStream_t s);
hipError_t launch_norm_split_apply(const NormSplitParams& p, bool bf16_io, hipStream_t s);

// Causal attention over local heads (head_dim 128), batched over `nshards`
// problems advancing by sQK / sVt / sO elements.
struct AttnParams {
  const void* QK;
  int64_t ldqk, sQK, kcol0;
  const void* Vt;
  int64_t ldvt, sVt;
  void* O;
  int64_t ldo, sO;
  int batch, seq, heads, nshards;
  float scale_log2e;  // log2(e) / sqrt(head_dim)
};
hipError_t launch_attention(const AttnParams& p, hipStream_t s);


// Layout kernels of the MLP pair's backward (bwd.hip), bf16 or fp32.
//   out[c][r] = op(in[r][c]) for in [R x C] (ld_in), out [C x R] (ld_out);
//   op = identity, or GELU (the activation recomputed from a stored
//   pre-activation).  R, C, ld_in, ld_out multiples of 8 (bf16) or 4 (fp32).
struct TransposeParams {
  const void* in;
  int64_t ld_in;
  void* out;
  int64_t ld_out;
  int64_t R, C;
};
hipError_t launch_transpose(const TransposeParams& p, bool gelu, bool f32, hipStream_t s);

//   out[r] = sum over c of in[r][c] (bf16 or fp32 in), fp32, in a fixed order.
//   C a multiple of 8 (bf16) or 4 (fp32).
struct RowSumParams {
  const void* in;
  int64_t ld;
  float* out;
  int64_t R, C;
};
hipError_t launch_rowsum(const RowSumParams& p, bool f32, hipStream_t s);

//   out[c] = sum over r of in[r][c], bf16 in [R x C] (ld), fp32 out, in a
//   fixed order: chunks of rows summed into part (colsum_part_floats(R, C)
//   floats of workspace), then the chunks folded in order.  C a multiple of 8.
//   n (at most 2) independent sums share the two launches: the chunk sums
//   (launch_colsum_chunks), then their fold (launch_colsum_fold, same ps);
//   each sum's bits are those it has alone.
struct ColSumParams {
  const void* in;
  int64_t ld;
  int64_t R, C;
  float* part;
  float* out;
};
size_t colsum_part_floats(int64_t R, int64_t C);
hipError_t launch_colsum_chunks(const ColSumParams* ps, int n, hipStream_t s);
hipError_t launch_colsum_fold(const ColSumParams* ps, int n, hipStream_t s);

// Vocab-parallel cross-entropy (vocab.hip).
// Folds the per-chunk statistics of the GEMM epilogue (layout of CeEpilogue,
// shards local to the launch) into the per-shard ones, chunk order, slot
// (shard0 + s)*T + t of m, s, z.
struct CeFoldParams {
  const float* stats;
  int64_t astride, T;
  float *m, *s, *z;
  int shard0, shards, cps;
};
hipError_t launch_ce_fold(const CeFoldParams& p, hipStream_t s);

// loss[t] = log S + M - target from the N shards' statistics (slots i*T + t).
struct CeCombineParams {
  const float *m, *s, *z;
  float* loss;
  int64_t T;
  int N;
};
hipError_t launch_ce_combine(const CeCombineParams& p, hipStream_t s);
hipError_t launch_ce_mean(const float* loss, int64_t T, float* mean, hipStream_t s);

// Vocab-parallel embedding, one partial per shard of the launch, in the
// table's type: partial s (at P + s*sP elements, [T x H]) holds row ids[t]
// of E for the tokens whose id lies in [(shard0+s)*Vs, min(+Vs, V)) and
// zeros elsewhere.  H a multiple of 8.
struct EmbedParams {
  const int32_t* ids;
  const void* E;
  void* P;
  int64_t sP, T, H, V, Vs;
  int shard0, shards;
};
hipError_t launch_embed_partial(const EmbedParams& p, bool f32, hipStream_t s);

// Y[j] = fold over k < N in order of P[k*sP + j] (fp32 adds), cast to the
// table's type; n = T*H elements, a multiple of 8.
struct EmbedFoldParams {
  const void* P;
  int64_t sP, n;
  int N;
  void* Y;
};
hipError_t launch_embed_fold(const EmbedFoldParams& p, bool f32, hipStream_t s);

}  // namespace tp
