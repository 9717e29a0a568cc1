/*
 * tp.h -- C ABI of libtp.so: the tensor-parallel column -> activation -> row
 * linear pair (MLP and head-split attention), N shards on one MI355X (gfx950),
 * partial sums combined by an on-device fixed-order reduction that stands in
 * for the all-reduce.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *   allocates, frees or keeps device memory; scratch comes from a
 *   caller-provided workspace.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *   call only enqueues work on `stream` and returns; execution errors surface
 *   on the caller's next synchronisation.
 * - Matrices are row-major.  Activations are [rows x features].  Weights use
 *   the [out x in] storage of the weight chunks in the PyTorch listing of
 *   "Tensor Parallelism基础：模型切分原理" (section on implementation details):
 *   a linear layer computes Y = X * W^T with W of shape [out x in].  `ld*` are
 *   leading dimensions (row strides) in elements, so a shard may be a view
 *   into a larger matrix.
 * - bf16 inputs accumulate in fp32; outputs are rounded once,
 *   round-to-nearest-even.
 * - Every argument is validated before the first HIP call.  On error the call
 *   returns a status, launches nothing, and tp_last_error() (thread-local)
 *   names the offending argument and, for divisibility errors, the shard
 *   shapes (the fail-fast divisibility check of the blog post at 2kiu.com,
 *   section 6.1).  No call aborts or throws across the ABI.
 * - Alignment: device pointers 16-byte aligned (int32 token ids and labels:
 *   4-byte); bf16 leading dimensions and contraction sizes multiples of 8
 *   elements, fp32 ones multiples of 4.
 * - All kernels are deterministic: no atomics, fixed summation order.
 */
#ifndef TP_H_
#define TP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TP_OK = 0,
  TP_ERR_NULL = 1,          /* a required pointer is NULL                  */
  TP_ERR_SHAPE = 2,         /* negative/zero size, ld too small, bad slice */
  TP_ERR_DIVISIBILITY = 3,  /* F, heads or T not divisible as required     */
  TP_ERR_DTYPE = 4,         /* dtype/activation combination not supported  */
  TP_ERR_ALIGN = 5,         /* pointer or ld alignment                     */
  TP_ERR_WORKSPACE = 6,     /* workspace NULL or too small                 */
  TP_ERR_HIP = 7            /* a HIP launch failed                         */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

typedef enum { TP_ACT_NONE = 0, TP_ACT_GELU = 1, TP_ACT_SWIGLU = 2 } tp_act;

/*
 * Column-parallel linear for one shard:  Y_i = act(X * W_i^T + bias_i).
 * Column split of "Tensor Parallelism基础：模型切分原理" (column-wise splitting)
 * and of the 2kiu.com blog post, section 2.1: X is replicated, shard i holds
 * output features i*F/N .. (i+1)*F/N - 1, the bias is sliced with them and is
 * added before the activation.  Concatenating the N outputs along features
 * (the all-gather) is a matter of layout: pass Y_i = Y + i*Ns with ldy = F.
 *
 *   X    [T x K]  (ldx)        dt
 *   W_i  NONE/GELU:  [Ns x K]  (ldw)            dt
 *        SWIGLU:     [2Ns x K] (ldw): rows 0..Ns-1 gate, Ns..2Ns-1 up
 *   bias_i [Ns] or NULL (must be NULL for SWIGLU)   dt
 *   Y_i  [T x Ns] (ldy)        dt
 * act: GELU = x*Phi(x) (erf form); SWIGLU = SiLU(gate) * up (bf16 only).
 * T == 0 is a no-op.
 */
tp_status tp_column_linear(void* stream, tp_dtype dt, tp_act act, int64_t T, int64_t K,
                           int64_t Ns, const void* X, int64_t ldx, const void* W_i,
                           int64_t ldw, const void* bias_i, void* Y_i, int64_t ldy);

/*
 * Row-parallel partial product for one shard:  P_i = X_i * W_i^T  (fp32 out,
 * never a bias: the row bias is added once, after the sum; the listing of
 * "Tensor Parallelism基础" adds it after the all-reduce).  Row split of the
 * 2kiu.com blog post, section 2.2: every partial has the full output shape.
 *
 *   X_i  [T x Ks] (ldx)          dt
 *   W_i  [Nout x Ks] (ldw)       dt   (shard i's column block of the [H x F]
 *                                      out-in matrix: W + i*Ks, ldw = F)
 *   P_i  [T x Nout] (ldp)        fp32
 */
tp_status tp_row_linear_partial(void* stream, tp_dtype dt, int64_t T, int64_t Ks,
                                int64_t Nout, const void* X_i, int64_t ldx, const void* W_i,
                                int64_t ldw, float* P_i, int64_t ldp);

/*
 * The all-reduce stand-in:  Y = (((P_0 + P_1) + ...) + P_{n-1}) + bias, each
 * + one fp32 IEEE addition in shard order, then one round-to-nearest-even cast
 * to out_dt.  Row-split sum of the 2kiu.com blog post (section 2.2) and of
 * "张量并行" (row-split equation); bias once, after the sum.
 *
 *   P      n_parts partials, partial k at P + k*part_stride, each [T x H], ld = H
 *   bias   [H] in out_dt, or NULL
 *   n_slices >= 1, slice in [-1, n_slices): slice == -1 writes all T rows to
 *          Y [T x H]; slice == r writes only rows r*T/n .. (r+1)*T/n - 1 to
 *          Y [T/n x H] -- the reduce-scatter along the sequence of Megatron-SP
 *          ("张量并行", sequence section; blog post section 4.3).
 * H must be a multiple of 8; T a multiple of n_slices.
 */
tp_status tp_reduce_partials(void* stream, tp_dtype out_dt, int n_parts, int64_t T, int64_t H,
                             const float* P, int64_t part_stride, const void* bias, void* Y,
                             int n_slices, int slice);

/*
 * Entry side of the sequence-parallel region, before a column linear: each
 * rank's sequence slice is RMS-normalized and written into its rows of the
 * gathered buffer -- what every rank holds after the all-gather along the
 * sequence.  The norm is row-wise, so it runs on sequence slices exactly
 * (2kiu.com blog post, section 4.3; "张量并行", Megatron-SP section), and
 * RMSNorm needs only the mean of squares over the whole hidden vector (blog
 * post, section 3.3).
 *
 *   Y[r*T/n + t, :] = X_r[t, :] / sqrt(mean(X_r[t, :]^2) + eps) * gamma
 *
 *   X       slice r at X + r*slice_stride (elements), T/n rows of H, row stride
 *           ldx; the slices must not overlap
 *   gamma   [H], same dtype as X and Y
 *   eps     finite, >= 0 (a zero row with eps == 0 divides by zero: NaN)
 *   Y       [T x H] (ldy); slice == -1 normalizes every slice, slice == r only
 *           rank r's (rows r*T/n .. (r+1)*T/n - 1 of Y, the other rows untouched)
 * The statistic is an fp32 sum of squares in a fixed order (bit-identical run
 * to run); output rounded once, round-to-nearest-even.  H a multiple of 8
 * (bf16) or 4 (fp32), at most 16384 (bf16) / 8192 (fp32); T a multiple of
 * n_slices.
 */
tp_status tp_rmsnorm_gather(void* stream, tp_dtype dt, int n_slices, int64_t T, int64_t H,
                            const void* X, int64_t slice_stride, int64_t ldx, const void* gamma,
                            float eps, void* Y, int64_t ldy, int slice);

/*
 * The same entry side with LayerNorm (the blog post, section 3.3, names
 * LayerNorm beside RMSNorm: it needs the mean and the variance of the whole
 * hidden vector, so it too runs exactly on sequence slices):
 *
 *   Y[r*T/n + t, :] = (X_r[t, :] - m) / sqrt(v + eps) * gamma + beta
 *
 * with m the row's mean and v its mean squared deviation from m (the biased
 * variance).  Arguments as tp_rmsnorm_gather; beta [H] (same dtype) or NULL
 * for no shift.  The statistics are fp32 sums in a fixed order: the values
 * first, then the squared deviations from their mean (two passes over the
 * row held on chip, so no cancellation between a sum of squares and a
 * squared mean); bit-identical run to run; one RNE cast.
 */
tp_status tp_layernorm_gather(void* stream, tp_dtype dt, int n_slices, int64_t T, int64_t H, const void* X,
                              int64_t slice_stride, int64_t ldx, const void* gamma, const void* beta, float eps,
                              void* Y, int64_t ldy, int slice);

/*
 * Norm of an input split along hidden across N shards (2kiu.com blog post,
 * section 3.3: keep the norm's input split along hidden, reduce the small
 * local statistics to the global ones, correct by a formula, scale locally).
 * Shard i holds columns [i*H/N, (i+1)*H/N) of X and writes the same columns
 * of Y.  Two steps, the two sides of the statistic's all-reduce:
 *   1. for each shard in [shard_begin, shard_begin + shard_count) and row t,
 *      the shard's local statistic into slot (i, t) of the workspace slab
 *      (N x T x 2 fp32):
 *        TP_NORM_RMS    its sum of squares
 *        TP_NORM_LAYER  its mean m_i and sum of squared deviations q_i
 *   2. each shard of the range folds the N slots of the row in shard order
 *      -- RMS: sums added; LAYER: (count, mean, q) merged by the pairwise
 *      update d = m_i - m, n' = n + H/N, m += d (H/N)/n',
 *      q += q_i + d^2 n (H/N)/n' -- and scales its own columns:
 *        RMS    Y = X / sqrt(sum/H + eps) * gamma
 *        LAYER  Y = (X - m) / sqrt(q/H + eps) * gamma + beta
 * Every shard folds the same slots in the same order, so every shard uses
 * the same bits (the broadcast of the reduced statistic).  With
 * shard_count < N, step 2 reads the other shards' slots as they are in the
 * slab (left there by earlier calls): one rank's share.
 *   X, Y   [T x H] (ldx, ldy), dt;  gamma [H] dt;  beta [H] dt or NULL (must
 *          be NULL for RMS);  eps finite, >= 0
 * H/N a multiple of 8 (bf16) or 4 (fp32), at most 16384 (bf16) / 8192 (fp32).
 */
typedef enum { TP_NORM_RMS = 0, TP_NORM_LAYER = 1 } tp_norm_kind;
typedef struct {
  tp_dtype dt;
  tp_norm_kind kind;
  int64_t T, H;
  int N, shard_begin, shard_count;
  const void* X;
  int64_t ldx;
  const void* gamma;
  const void* beta;
  float eps;
  void* Y;
  int64_t ldy;
} tp_norm_split_desc;
/* Workspace bytes (the N x T x 2 fp32 statistics slab), 0 when invalid. */
size_t tp_norm_split_workspace_size(const tp_norm_split_desc* d);
tp_status tp_norm_hidden_split(void* stream, const tp_norm_split_desc* d, void* ws, size_t ws_bytes);

/* Whole MLP sublayer over shards [shard_begin, shard_begin + shard_count). */
typedef struct {
  tp_dtype dt;      /* TP_F32 or TP_BF16 (inputs, intermediate and output)      */
  tp_act act;       /* TP_ACT_GELU (or NONE) with A [F x H]; TP_ACT_SWIGLU with */
                    /* A = N fused blocks [2F/N x H]: gate rows then up rows    */
  int64_t T, H, F;  /* tokens, hidden, intermediate (SWIGLU: intermediate size) */
  int N, shard_begin, shard_count;
  const void* X;    /* [T x H]                                                  */
  const void* A;    /* column weight, see act                                   */
  const void* a;    /* [F] column bias or NULL                                  */
  const void* B;    /* [H x F] row weight (out-in); shard i = columns i*F/N..   */
  const void* b;    /* [H] row bias or NULL (added once, after the sum)         */
  void* Y;          /* [T x H], or [T/n_slices x H] when slice >= 0             */
  int n_slices, slice;
  void* Z;          /* [T x F] (ld F), SwiGLU [T x 2F] (ld 2F), or NULL.  When
                       set (bf16), the forward also writes the range's
                       pre-activation Z_i = X A_i^T + a_i (shard i = columns
                       i*F/N.., SwiGLU: columns 2i*F/N.. holding [gate | up]
                       of shard i), rounded to bf16 once, so that
                       tp_mlp_backward can take it instead of recomputing it
                       (training keeps the activation's input).  The fused
                       narrow-hidden kernel keeps its intermediate on chip, so
                       asking for Z selects the two-GEMM path there. */
  void* Hact;       /* [T x F] (ld F) or NULL (bf16, GELU or SwiGLU).  When set,
                       the range's activated intermediate H_i = act(Z_i)
                       (shard i = columns i*F/N..), rounded to bf16 once, is
                       written there instead of into the workspace, and the
                       row product reads it from there: the row layer's input,
                       which a training forward keeps for the weight gradient
                       (tp_mlp_backward's Hact).  Like Z, it selects the
                       two-GEMM path at narrow hidden sizes. */
} tp_mlp_desc;

/* Whole attention sublayer over shards [shard_begin, shard_begin + shard_count).
 * Shard i owns whole heads i*heads/N .. (i+1)*heads/N - 1 (2kiu.com post,
 * section 3.1).  Token row = b*seq + s.  bf16 only, head_dim == 128,
 * seq a multiple of 128. */
typedef struct {
  tp_dtype dt;
  int64_t batch, seq, hidden;
  int heads, head_dim, N, shard_begin, shard_count;
  const void* X;    /* [batch*seq x hidden]                                      */
  const void* Wqkv; /* N blocks [3*(heads/N)*head_dim x hidden]: Q rows, K rows, */
                    /* V rows of the shard's heads, in head order                */
  const void* Wo;   /* [hidden x hidden] out-in; shard i = columns i*hidden/N..  */
  const void* bo;   /* [hidden] or NULL                                          */
  void* Y;          /* [batch*seq x hidden] (or one slice, as for the MLP)       */
  int n_slices, slice;
} tp_attn_desc;

/* Workspace bytes needed by tp_mlp_forward / tp_attn_forward for this desc.
 * Layout: the fp32 partial slab comes first (slot i = shard i, each
 * [T x H]); tp_*_partials_offset returns its byte offset.  Returns 0 when
 * the descriptor is invalid (see tp_last_error). */
size_t tp_mlp_workspace_size(const tp_mlp_desc* d);
size_t tp_attn_workspace_size(const tp_attn_desc* d);
size_t tp_mlp_partials_offset(const tp_mlp_desc* d);
size_t tp_attn_partials_offset(const tp_attn_desc* d);

/*
 * Column GEMM (+bias, activation) and row partial of every shard in range,
 * then -- when the range covers all N shards -- the fixed-order reduction
 * into Y.  With shard_count < N the partials stay in the workspace slab
 * (slot i = shard i) and Y is untouched: one rank's share is its shard plus a
 * tp_reduce_partials over the slab.  The pairing (column output slice is the
 * row input slice, one reduction per sublayer) is section 2.3 of the 2kiu.com
 * post and the MLP paragraph of "张量并行".
 */
tp_status tp_mlp_forward(void* stream, const tp_mlp_desc* d, void* ws, size_t ws_bytes);

/*
 * The same sublayer with the reduction overlapped ("大模型分布式训练篇——从零实现
 * Tensor Para...", section 3: compute/communication overlap).  The token axis
 * is cut into `chunks` equal row blocks.  Block k's shard products run on
 * `stream`; as soon as they are done, the fold of block k's rows runs on
 * `stream2` while block k+1 computes.  `stream` waits for `stream2` at the
 * end, so work the caller enqueues on `stream` afterwards sees Y complete.
 * The result is bit-identical to tp_mlp_forward (same kernels, same per-row
 * fold).  Needs the whole shard range (shard_count == N), slice == -1, T a
 * multiple of chunks (1..64), and two distinct streams.  Calls that overlap on
 * the same workspace race.
 */
tp_status tp_mlp_forward_overlap(void* stream, void* stream2, const tp_mlp_desc* d, int chunks, void* ws,
                                 size_t ws_bytes);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the same
 * sublayer as tp_mlp_forward (same kernels, same bits), with no workspace
 * argument.  Its partial slab and intermediate live in a library-owned,
 * file-scope static device array of TP_NOALLOC_SCRATCH_BYTES, one copy per
 * GPU the library runs on, held until the process ends; the call itself
 * allocates and frees nothing.
 *   - Needs the whole shard range (shard_count == N): a partial range would
 *     leave its partials in a buffer the caller cannot see.
 *   - Fails with TP_ERR_WORKSPACE, before any HIP call, when the workspace
 *     tp_mlp_workspace_size(d) reports exceeds TP_NOALLOC_SCRATCH_BYTES.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero: each call
 *     writes every byte it reads).  Calls that overlap on one GPU -- on two
 *     streams, or from two threads -- race on it.
 *   - The array is resolved on the GPU of `stream` (the current device for
 *     the null stream) on that GPU's first call; errors of that lookup are
 *     returned as TP_ERR_HIP.
 */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
tp_status tp_mlp_forward_noalloc(void* stream, const tp_mlp_desc* d);

/* QKV projection of the shard's heads, causal softmax attention per local
 * head (scale 1/sqrt(head_dim), diagonal kept), row-parallel output
 * projection into the partial slab, then the reduction as for the MLP. */
tp_status tp_attn_forward(void* stream, const tp_attn_desc* d, void* ws, size_t ws_bytes);

/*
 * Backward of the MLP pair over shards [shard_begin, shard_begin + shard_count)
 * (activation GELU or NONE in bf16 or fp32; SwiGLU in bf16, see the end of
 * this comment), given the forward's input X, its weights and
 * the gradient dY of its output.  Per shard i, with no exchange:
 *   Z_i  = X A_i^T + a_i            (recomputed -- activation recomputation,
 *                                    2kiu.com blog post, section 5.3 -- unless
 *                                    the descriptor's Z holds the forward's)
 *   dZ_i = (dY B_i) * act'(Z_i)     (dY reaches every shard whole)
 *   dA_i = dZ_i^T X,  da_i = column sums of dZ_i
 *   dB_i = dY^T act(Z_i),           the shard's columns of dB
 *   dX_i = dZ_i A_i                 (a partial: X was replicated)
 * then, when the range covers all N shards, dX = ((dX_0 + dX_1) + ...) in
 * shard order, one RNE cast: the all-reduce of the column layer's backward
 * ("大模型分布式训练篇——从零实现 Tensor Para...", section 4: identity forward,
 * all-reduce backward; blog post, section 4.1).  db = column sums of dY, once
 * (the row bias enters once: listing of "Tensor Parallelism基础").
 * Storage order as in the forward: A [F x H], B [H x F] (out-in); gradients
 * come back in the same layout.  Weight and bias gradients are fp32.
 * bf16: Z_i and dZ_i are rounded to bf16 once (as a bf16 forward would store
 * its linear outputs), act(Z_i) is evaluated from the rounded Z_i (when it is
 * recomputed at H <= 2048, one two-pass kernel keeps Z_i on chip in fp32
 * instead).  fp32: everything stays fp32.  A stored Z (bf16: GELU, NONE or
 * SwiGLU) gives the same bits as recomputing it with the GEMM path: the
 * forward's column product and the recomputation accumulate in the same order.
 * A stored Hact (GELU, with Z) replaces GELU(Z_i) in dB_i only: dB then uses
 * the forward's activation of the unrounded pre-activation, so its bits
 * differ from the Z-only run; every other gradient keeps its bits.
 * SwiGLU (blog post section 3.2): A holds the N fused blocks [2F/N x H] of the
 * forward (gate rows, then up rows); Z_i = [G_i | U_i], dH_i = dY B_i,
 * dZ_i = [dH_i U_i SiLU'(G_i) | dH_i SiLU(G_i)], dA comes back in the same
 * fused-block layout ([2F x H]), dB_i = dY^T (SiLU(G_i) U_i); a and da must
 * be NULL.
 */
typedef struct {
  tp_dtype dt;     /* TP_BF16, or TP_F32 (GELU / NONE; all buffers fp32)        */
  tp_act act;      /* TP_ACT_GELU, TP_ACT_NONE, or TP_ACT_SWIGLU (see below)    */
  int64_t T, H, F; /* T, H, F/N multiples of 8                                  */
  int N, shard_begin, shard_count;
  const void* X;   /* [T x H] dt                                                */
  const void* A;   /* [F x H] dt ([2F x H] fused blocks for SwiGLU)             */
  const void* a;   /* [F] dt or NULL                                            */
  const void* B;   /* [H x F] dt                                                */
  const void* dY;  /* [T x H] dt                                                */
  void* dX;        /* [T x H] dt, written when shard_count == N, else unused    */
  float* dA;       /* [F x H] ([2F x H] SwiGLU): rows of the shard range written */
  float* da;       /* [F] (entries of the range) or NULL to skip                */
  float* dB;       /* [H x F]: columns of the shard range written               */
  float* db;       /* [H] or NULL to skip                                       */
  int n_slices, slice; /* the dX fold's layout, as in tp_reduce_partials: 1, -1 for
                       the all-reduce; n_slices > 1 and slice = r for rank r's
                       reduce-scatter slice along the sequence (dX then holds
                       the T/n_slices rows r*T/n_slices ..), the backward of the
                       sequence-parallel all-gather ("张量并行", Megatron-SP
                       section); slice = -1 writes every slice          */
  const void* Z;   /* [T x F] dt (ld F), SwiGLU [T x 2F] (ld 2F), or NULL: the
                      forward's pre-activation (tp_mlp_desc.Z, same layout),
                      read for the range's columns instead of recomputing
                      X A_i^T + a_i                                            */
  const void* Hact; /* [T x F] bf16 (ld F) or NULL: the forward's activated
                      intermediate (tp_mlp_desc.Hact), the B operand of
                      dB_i = dY^T H_i, read for the range's columns instead
                      of evaluating GELU(Z_i) from the stored Z.  GELU only,
                      and only together with Z.                                */
} tp_mlp_bwd_desc;

/* Workspace bytes for tp_mlp_backward (0 when the descriptor is invalid).
 * The fp32 dX partial slab comes first (slot i = shard i, each [T x H]): with
 * shard_count < N the partials of the range stay there, as in the forward. */
size_t tp_mlp_backward_workspace_size(const tp_mlp_bwd_desc* d);
tp_status tp_mlp_backward(void* stream, const tp_mlp_bwd_desc* d, void* ws, size_t ws_bytes);

/*
 * Vocab-parallel output head and cross-entropy over shards [shard_begin,
 * shard_begin + shard_count).  The vocab is padded to Vp = N*Vs entries
 * (tp_vocab_padded: Vs = ceil(V/N) rounded up to a multiple of 8) so that it
 * splits into N equal shards; entries >= V are padding and take no part in
 * the loss (2kiu.com blog post, section 6.2: pad the vocab to a size TP
 * divides and filter the padding out of the loss).  Shard i computes the
 * logits of its partition, X E_i^T (fp32), and from them its part of the
 * loss only: its maximum, its sum of exp(logit - maximum), and the label's
 * logit if it owns the label (same section: no shard assembles the full
 * logits; an all-reduce combines the parts).  When the range covers all N
 * shards, the parts are folded in shard order (the all-reduce stand-in):
 *   M = max_i m_i,  S = sum_i s_i exp(m_i - M),  loss[t] = log S + M - z_label
 * and mean_loss = (sum over t of loss[t]) / T in a fixed order.
 *
 *   X        [T x H] bf16
 *   E        [Vp x H] bf16 (out-in storage of the head / tied embedding); the
 *            padding rows V .. Vp-1 must exist (any finite values)
 *   labels   [T] int32 in [0, V); a label outside has no owner and its token's
 *            loss is log S + M (no target term)
 *   loss     [T] fp32, written when shard_count == N
 *   mean_loss  [1] fp32 or NULL
 * With shard_count < N the range's statistics stay in the workspace.
 * H a multiple of 8.  Deterministic (fixed orders, no atomics).
 */
typedef struct {
  tp_dtype dt;     /* TP_BF16                                                   */
  int64_t T, H, V;
  int N, shard_begin, shard_count;
  const void* X;
  const void* E;
  const int32_t* labels;
  float* loss;
  float* mean_loss;
} tp_vocab_ce_desc;

/* Padded vocab size Vp for V entries over N shards (0 if V < 1 or N < 1). */
int64_t tp_vocab_padded(int64_t V, int N);
size_t tp_vocab_ce_workspace_size(const tp_vocab_ce_desc* d);
tp_status tp_vocab_ce_forward(void* stream, const tp_vocab_ce_desc* d, void* ws, size_t ws_bytes);

/*
 * Vocab-parallel embedding lookup (the input side of the vocab split; blog
 * post at 2kiu.com, section 6.2: the embedding matrix is split along the
 * vocab like the output head, padded so TP divides it; "张量并行", practice
 * section: vocab-parallel embedding).  Shard i owns padded vocab rows
 * [i*Vs, (i+1)*Vs) (Vs as in tp_vocab_padded) and looks up only the ids it
 * owns, writing rows of -0.0 (the IEEE additive identity) for the others --
 * one partial [T x H] per shard in the table's type dt, slot i of the
 * workspace slab.  When the range covers all N shards the partials are
 * folded in shard order in fp32 from -0.0 (the all-reduce stand-in) and cast
 * back to dt: at most one term per element is not -0.0, so Y[t] = E[ids[t]]
 * bit for bit, signed zeros included.  Rows >= V of E are never read; an id
 * outside [0, V) has no owner and gets a row of -0.0.
 *
 *   ids  [T] int32;  E [Vp x H] dt (Vp = tp_vocab_padded(V, N));  Y [T x H] dt
 * dt is TP_BF16 or TP_F32; H a multiple of 8.
 */
typedef struct {
  tp_dtype dt;
  int64_t T, H, V;
  int N, shard_begin, shard_count;
  const int32_t* ids;
  const void* E;
  void* Y;
} tp_vocab_embed_desc;
size_t tp_vocab_embed_workspace_size(const tp_vocab_embed_desc* d);
tp_status tp_vocab_embed_forward(void* stream, const tp_vocab_embed_desc* d, void* ws, size_t ws_bytes);

/*
 * Local causal attention alone (the middle step of tp_attn_forward), for
 * `heads` heads of width 128 over `batch` sequences of length `seq`:
 *   QK  [batch*seq x ldqk]: head h's query at columns h*128.., its key at
 *       columns k_col0 + h*128..
 *   Vt  [heads*128 x ldvt]: V transposed; row h*128+d, column b*seq+s
 *   O   [batch*seq x ldo]: head h at columns h*128..
 */
tp_status tp_attn_local(void* stream, int64_t batch, int64_t seq, int heads, int head_dim,
                        const void* QK, int64_t ldqk, int64_t k_col0, const void* Vt,
                        int64_t ldvt, void* O, int64_t ldo);

/*
 * Per-kernel timing, for measurement (the pages read the share of time each
 * kernel takes from a profiler: "大模型分布式训练篇——从零实现 Tensor Para...",
 * section on practical advice).  While enabled, every kernel launch made by
 * the entry points above is bracketed by a HIP event pair recorded on the
 * caller's stream (no other effect on the work).  tp_timing_read waits for the
 * recorded events, adds their durations into per-kernel totals and copies up
 * to `max` of them (names stay valid until the next read; any output pointer
 * may be NULL); it returns the number of kernels with totals.
 * tp_timing_reset discards pending events and totals.
 */
tp_status tp_timing_enable(int on);
int tp_timing_read(int max, const char** names, double* total_ms, int64_t* launches);
void tp_timing_reset(void);

const char* tp_status_string(tp_status s);
const char* tp_last_error(void);
/* Library version string (build id); never NULL. */
const char* tp_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TP_H_ */
