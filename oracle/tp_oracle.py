"""fp64 CPU oracle for the tensor-parallel column -> activation -> row linear pair.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import or call this module.  The product
path (the HIP library and its Python binding) never touches it, and this module
imports nothing from the product package.

What it computes is the plain, *unsharded* layer in float64 (numpy, with
scipy's erf as the one special function), plus the sharded forms written out
step by step so that the sharding identities can be checked against the
unsharded definition.  Inputs are taken exactly as given (the caller passes
the values the GPU received, already rounded to the run's dtype); nothing here
rounds to a narrower type except ``reduce_partials_fp32`` and ``to_bf16``,
which exist to pin the fixed-order fp32 reduction bit for bit.

Matrices are in math layout here: a weight ``W`` is [in x out] and a linear
layer is ``X @ W``.  (Callers holding weights in the [out x in] storage of the
pages' PyTorch listing pass ``W.T``.)

Pages cited (titles as extracted):
  [Blog]    page at 2kiu.com whose extracted HTML title is "企业官网建设流程全解析";
            its body is a tensor-parallelism blog post with sections 1-6.
  [Wiki]    "张量并行" (ai-infra-wiki).
  [Scratch] "大模型分布式训练篇——从零实现 Tensor Para..." (makesence.top).
  [Basics]  "Tensor Parallelism基础：模型切分原理" (bjdmk.com.cn).

Pinned by tests/test_oracle_*.py (identities on integer inputs, closed forms,
textbook values, pure-Python brute force).  Every function below is pinned;
none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf, expit

__all__ = [
    "gelu", "silu", "linear", "mlp_gelu", "mlp_swiglu", "causal_attention",
    "attention_block", "column_shards", "row_shards", "column_linear_sharded",
    "row_partials", "mlp_gelu_sharded", "swiglu_fused_blocks",
    "mlp_swiglu_sharded", "attention_block_sharded", "rs_slice",
    "reduce_partials_fp32", "to_bf16", "attention_block_rows",
    "rmsnorm", "seq_slices", "all_gather_rows", "sp_entry", "rmsnorm_hidden_split",
    "layernorm", "sp_entry_layernorm", "merge_moments", "layernorm_hidden_split",
    "gelu_grad", "mlp_backward", "mlp_backward_sharded",
    "padded_vocab", "cross_entropy", "lm_head_ce", "vocab_parallel_ce",
    "silu_grad", "mlp_swiglu_backward", "mlp_swiglu_backward_sharded",
    "vocab_parallel_embedding",
]

_SQRT2 = math.sqrt(2.0)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# activations
# --------------------------------------------------------------------------
def gelu(z):
    """GELU in its exact form z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)).

    [Wiki] section on the two split directions writes the MLP as GELU(XA)B
    and names no approximation, so the exact (erf) form is used; the tanh
    approximation is not what is computed here.
    """
    z = _f64(z)
    return 0.5 * z * (1.0 + erf(z / _SQRT2))


def silu(g):
    """SiLU / Swish with beta = 1: g * sigmoid(g).

    [Blog] section 3.2 names a SwiGLU-type MLP with gate and up branches; the
    gate branch goes through SiLU and multiplies the up branch elementwise.
    ``expit`` is scipy's logistic function (stable for large |g|).
    """
    g = _f64(g)
    return g * expit(g)


# --------------------------------------------------------------------------
# unsharded layers (the definitions the sharded path must reproduce)
# --------------------------------------------------------------------------
def linear(X, W, bias=None):
    """Y = X W (+ bias): the dense linear layer every split starts from
    ([Blog] section 2.1, Y = XW with W of shape (H_in, H_out))."""
    Y = _f64(X) @ _f64(W)
    if bias is not None:
        Y = Y + _f64(bias)[None, :]
    return Y


def mlp_gelu(X, A, a, B, b):
    """Y = GELU(X A + a) B + b, unsharded ([Wiki] two-split section, MLP
    formula; biases as in the [Basics] listing: one per linear layer)."""
    Z = linear(X, A, a)
    return linear(gelu(Z), B, b)


def mlp_swiglu(X, Wg, Wu, Wd):
    """Y = (SiLU(X Wg) * (X Wu)) Wd, unsharded, no biases ([Blog] section 3.2)."""
    G = linear(X, Wg)
    U = linear(X, Wu)
    return linear(silu(G) * U, Wd)


def causal_attention(Q, K, V, batch, seq, heads):
    """Per-head causal softmax attention.

    Q, K, V are [batch*seq x heads*d]; token row = b*seq + s; head h owns
    columns h*d .. h*d+d-1.  For each (b, h): S = Q K^T / sqrt(d), entries with
    key index > query index are masked out (the diagonal is kept), P is the
    row softmax of S and O = P V.  Heads are concatenated back in head order.
    The whole sequence is present for every head ([Blog] section 3.1: the
    sequence dimension stays whole, only heads are divided).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    T, HD = Q.shape
    assert T == batch * seq and HD % heads == 0
    d = HD // heads
    O = np.empty_like(Q)
    mask = np.triu(np.ones((seq, seq), dtype=bool), k=1)  # key > query
    scale = 1.0 / math.sqrt(d)
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for h in range(heads):
            cols = slice(h * d, (h + 1) * d)
            S = (Q[rows, cols] @ K[rows, cols].T) * scale
            S[mask] = -np.inf
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            O[rows, cols] = P @ V[rows, cols]
    return O


def attention_block(X, Wq, Wk, Wv, Wo, batch, seq, heads, bo=None):
    """Y = Attn(X Wq, X Wk, X Wv) Wo (+ bo): QKV projection, per-head causal
    attention, output projection ([Blog] section 3.1; [Wiki] attention
    paragraph of the two-split section)."""
    X = _f64(X)
    O = causal_attention(X @ _f64(Wq), X @ _f64(Wk), X @ _f64(Wv), batch, seq, heads)
    return linear(O, Wo, bo)


def attention_block_rows(X, Wq, Wk, Wv, Wo, batch, seq, heads, rows, bo=None):
    """``attention_block`` evaluated at the token rows ``rows`` only.

    Output row t = b*seq + s needs the query of row t and the keys/values of
    rows b*seq .. t; this evaluates exactly that (the same definition as
    ``attention_block``, restricted to the requested outputs).
    """
    X = _f64(X)
    Wq, Wk, Wv, Wo = map(_f64, (Wq, Wk, Wv, Wo))
    d = Wq.shape[1] // heads
    scale = 1.0 / math.sqrt(d)
    rows = np.asarray(rows)
    out = np.empty((rows.size, Wo.shape[1]))
    kv_cache = {}
    for n, t in enumerate(rows.tolist()):
        b, s = divmod(t, seq)
        if b not in kv_cache:
            Xb = X[b * seq:(b + 1) * seq]
            kv_cache = {b: (Xb @ Wk, Xb @ Wv)}
        Kb, Vb = kv_cache[b]
        q = X[t] @ Wq
        o = np.empty(Wq.shape[1])
        for h in range(heads):
            c = slice(h * d, (h + 1) * d)
            sc = (Kb[: s + 1, c] @ q[c]) * scale
            sc = sc - sc.max()
            p = np.exp(sc)
            p /= p.sum()
            o[c] = p @ Vb[: s + 1, c]
        out[n] = o @ Wo
        if bo is not None:
            out[n] += _f64(bo)
    return out


# --------------------------------------------------------------------------
# sharded forms (each shard's work written out, then combined)
# --------------------------------------------------------------------------
def column_shards(W, N):
    """Column split: shard i holds W[:, i*out/N : (i+1)*out/N] ([Blog] 2.1,
    its split diagram; [Basics] column-split paragraph)."""
    W = _f64(W)
    out = W.shape[1]
    if out % N:
        raise ValueError(f"output width {out} is not divisible by N={N}")
    s = out // N
    return [W[:, i * s:(i + 1) * s] for i in range(N)]


def row_shards(W, N):
    """Row split: shard i holds W[i*in/N : (i+1)*in/N, :] ([Blog] 2.2)."""
    W = _f64(W)
    inp = W.shape[0]
    if inp % N:
        raise ValueError(f"input width {inp} is not divisible by N={N}")
    s = inp // N
    return [W[i * s:(i + 1) * s, :] for i in range(N)]


def column_linear_sharded(X, W, bias, N):
    """Per-shard column outputs Y_i = X W_i + bias_i; X is replicated and
    the bias is sliced with the columns ([Basics] listing: each rank adds
    its own bias chunk before the gather)."""
    Ws = column_shards(W, N)
    bs = [None] * N
    if bias is not None:
        bias = _f64(bias)
        s = bias.shape[0] // N
        bs = [bias[i * s:(i + 1) * s] for i in range(N)]
    return [linear(X, Wi, bi) for Wi, bi in zip(Ws, bs)]


def row_partials(Hs, W, N):
    """Row partials P_i = H_i W_i for input slices H_i (list, or a full
    matrix to be split by columns) ([Blog] 2.2: every partial has the full
    output shape and the result is their elementwise sum; [Wiki] the
    row-split equation)."""
    Ws = row_shards(W, N)
    if not isinstance(Hs, (list, tuple)):
        Hs = column_shards(Hs, N)
    return [_f64(Hi) @ Wi for Hi, Wi in zip(Hs, Ws)]


def _fold(parts):
    """Left fold in shard order: ((P_0 + P_1) + P_2) + ...  (the order the
    stand-in for the all-reduce uses)."""
    acc = _f64(parts[0]).copy()
    for p in parts[1:]:
        acc = acc + _f64(p)
    return acc


def mlp_gelu_sharded(X, A, a, B, b, N):
    """The paired column -> GELU -> row layer over N shards: each shard
    applies GELU to its own intermediate slice, its row partial has the full
    output shape, partials are summed in shard order and the row bias is
    added once after the sum ([Blog] 2.3 and 3.2; [Wiki] one all-reduce per
    MLP; [Basics] listing: bias after the all-reduce, once)."""
    Hs = [gelu(Zi) for Zi in column_linear_sharded(X, A, a, N)]
    Y = _fold(row_partials(Hs, B, N))
    if b is not None:
        Y = Y + _f64(b)[None, :]
    return Y


def swiglu_fused_blocks(Wg, Wu, N):
    """Per-shard fused gate/up blocks [Wg_i | Wu_i] ([Blog] 3.2: gate and up
    concatenated into one larger column-parallel matrix; the intermediate
    must divide by N so each shard gets whole, equal gate and up slices).

    Block i is [H x 2*I/N] whose first I/N columns are gate columns
    i*I/N .. (i+1)*I/N - 1 and whose last I/N columns are the matching up
    columns.
    """
    G = column_shards(Wg, N)
    U = column_shards(Wu, N)
    return [np.concatenate([g, u], axis=1) for g, u in zip(G, U)]


def mlp_swiglu_sharded(X, fused_blocks, Wd, N):
    """SwiGLU MLP over N shards from the fused per-shard blocks: shard i
    computes SiLU(gate half) * (up half) of X @ block_i, multiplies by its
    row block of Wd, and the partials are summed in shard order."""
    Hs = []
    for Fi in fused_blocks:
        Z = linear(X, Fi)
        s = Z.shape[1] // 2
        Hs.append(silu(Z[:, :s]) * Z[:, s:])
    return _fold(row_partials(Hs, Wd, N))


def attention_block_sharded(X, Wq, Wk, Wv, Wo, batch, seq, heads, N, bo=None):
    """Head-split attention over N shards: shard i owns whole heads
    i*heads/N .. (i+1)*heads/N - 1, projects its own Q/K/V columns, runs
    attention on those heads alone, multiplies its head outputs by its row
    block of Wo, and the N partials are summed in shard order, then the
    output bias is added once ([Blog] 3.1; [Wiki] attention paragraph)."""
    if heads % N:
        raise ValueError(f"heads={heads} is not divisible by N={N}")
    hl = heads // N
    X = _f64(X)
    Qs, Ks, Vs = (column_shards(W, N) for W in (Wq, Wk, Wv))
    Os = [causal_attention(X @ q, X @ k, X @ v, batch, seq, hl)
          for q, k, v in zip(Qs, Ks, Vs)]
    Y = _fold(row_partials(Os, Wo, N))
    if bo is not None:
        Y = Y + _f64(bo)[None, :]
    return Y


def rs_slice(Y, n_slices, r):
    """Sequence-parallel reduce-scatter output for rank r: the r-th of
    n_slices contiguous row blocks of the reduced output ([Blog] 4.3;
    [Wiki] Megatron-SP section)."""
    T = Y.shape[0]
    if T % n_slices:
        raise ValueError(f"T={T} is not divisible by n_slices={n_slices}")
    s = T // n_slices
    return Y[r * s:(r + 1) * s]


# --------------------------------------------------------------------------
# sequence-parallel entry side: RMSNorm on sequence slices, then all-gather
# --------------------------------------------------------------------------
def rmsnorm(X, g, eps):
    """RMSNorm over the hidden (last) axis: each row times 1/sqrt(mean of its
    squares + eps), then times the per-feature gain g.

    [Blog] 3.3: the norm needs the statistic of the *whole* hidden vector, and
    RMSNorm needs only the second-order one (the mean of squares).  eps is not
    given by the pages; it is an argument here.
    """
    X = _f64(X)
    inv = 1.0 / np.sqrt(np.mean(X * X, axis=-1, keepdims=True) + eps)
    return X * inv * _f64(g)[None, :]


def seq_slices(X, n_slices):
    """The sequence-parallel split: n_slices contiguous row blocks, block r
    held by rank r ([Blog] 4.3; [Wiki] Megatron-SP section)."""
    X = _f64(X)
    return [rs_slice(X, n_slices, r) for r in range(n_slices)]


def all_gather_rows(slices):
    """All-gather along the sequence: the slices concatenated in rank order,
    the full [T x H] tensor every rank holds afterwards ([Blog] 4.3)."""
    return np.concatenate([_f64(s) for s in slices], axis=0)


def sp_entry(X, g, eps, n_slices):
    """Entry side of the sequence-parallel region before a column linear: each
    rank normalizes its own sequence slice (the norm is row-wise, so the
    sequence split is exact -- [Blog] 4.3), then the all-gather restores the
    full input the column GEMM needs ([Blog] 4.3, [Wiki] Megatron-SP)."""
    return all_gather_rows([rmsnorm(s, g, eps) for s in seq_slices(X, n_slices)])


def rmsnorm_hidden_split(X_parts, g_parts, eps):
    """RMSNorm of an input split along hidden across ranks ([Blog] 3.3): each
    part's local sum of squares, the small statistic summed over the parts in
    part order (the all-reduce of one number per row), and each part scaled
    locally by the shared coefficient.  Equals rmsnorm of the concatenation.
    """
    X_parts = [_f64(x) for x in X_parts]
    H = sum(x.shape[-1] for x in X_parts)
    ss = np.sum(X_parts[0] * X_parts[0], axis=-1, keepdims=True)
    for x in X_parts[1:]:
        ss = ss + np.sum(x * x, axis=-1, keepdims=True)
    inv = 1.0 / np.sqrt(ss / H + eps)
    return [x * inv * _f64(gp)[None, :] for x, gp in zip(X_parts, g_parts)]


def layernorm(X, g, b, eps):
    """LayerNorm over the hidden (last) axis: each row minus its mean, times
    1/sqrt(variance + eps), then times the gain g plus the shift b (b may be
    None).  The variance is the biased one (the mean of squared deviations,
    divided by H).

    [Blog] 3.3: LayerNorm needs the mean and the variance of the *whole*
    hidden vector.  eps is not given by the pages; it is an argument here.
    """
    X = _f64(X)
    mean = np.mean(X, axis=-1, keepdims=True)
    var = np.mean((X - mean) ** 2, axis=-1, keepdims=True)
    y = (X - mean) / np.sqrt(var + eps) * _f64(g)[None, :]
    return y if b is None else y + _f64(b)[None, :]


def sp_entry_layernorm(X, g, b, eps, n_slices):
    """The sequence-parallel entry side with LayerNorm: each rank's sequence
    slice normalized on its own (the norm is row-wise -- [Blog] 4.3), then the
    all-gather along the sequence ([Blog] 4.3, [Wiki] Megatron-SP)."""
    return all_gather_rows([layernorm(s, g, b, eps) for s in seq_slices(X, n_slices)])


def merge_moments(a, b):
    """Count, mean and sum of squared deviations of the union of two sets,
    from those of each set (the pairwise update of Chan, Golub and LeVeque):
    with d = mean_b - mean_a and n = n_a + n_b,
        mean = mean_a + d n_b / n,   M2 = M2_a + M2_b + d^2 n_a n_b / n.
    Exact in exact arithmetic: it follows from expanding the squared
    deviations of each set about the union's mean."""
    na, ma, qa = a
    nb, mb, qb = b
    n = na + nb
    d = mb - ma
    return n, ma + d * (nb / n), qa + qb + d * d * (na * nb / n)


def layernorm_hidden_split(X_parts, g_parts, b_parts, eps):
    """LayerNorm of an input split along hidden across ranks ([Blog] 3.3: keep
    the norm's input split, reduce the local statistics to the global mean
    and variance, then correct by a formula).  Each part's local statistics
    (its count, mean and sum of squared deviations about its own mean), merged
    over the parts in part order by ``merge_moments`` (the all-reduce of a
    few numbers per row), then each part normalized locally with the global
    mean and variance.  Equals ``layernorm`` of the concatenation."""
    X_parts = [_f64(x) for x in X_parts]
    stats = []
    for x in X_parts:
        m = np.mean(x, axis=-1, keepdims=True)
        stats.append((x.shape[-1], m, np.sum((x - m) ** 2, axis=-1, keepdims=True)))
    n, mean, m2 = stats[0]
    for st in stats[1:]:
        n, mean, m2 = merge_moments((n, mean, m2), st)
    inv = 1.0 / np.sqrt(m2 / n + eps)
    b_parts = b_parts if b_parts is not None else [None] * len(X_parts)
    out = []
    for x, gp, bp in zip(X_parts, g_parts, b_parts):
        y = (x - mean) * inv * _f64(gp)[None, :]
        out.append(y if bp is None else y + _f64(bp)[None, :])
    return out


# --------------------------------------------------------------------------
# backward of the MLP pair
# --------------------------------------------------------------------------
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def gelu_grad(z):
    """Derivative of the exact GELU: d/dz [z Phi(z)] = Phi(z) + z phi(z),
    phi the standard normal density (product rule on the erf form of
    ``gelu``)."""
    z = _f64(z)
    return 0.5 * (1.0 + erf(z / _SQRT2)) + z * np.exp(-0.5 * z * z) * _INV_SQRT_2PI


def _act_and_grad(act):
    if act == "gelu":
        return gelu, gelu_grad
    if act == "none":
        return (lambda z: _f64(z)), (lambda z: np.ones_like(_f64(z)))
    raise ValueError(act)


def mlp_backward(X, A, a, B, dY, act="gelu"):
    """Gradients of the unsharded MLP Y = act(X A + a) B + b for an upstream
    gradient dY (the gradient of the scalar sum(dY * Y)):

        Z = X A + a,  Hd = act(Z)
        dB = Hd^T dY,  db = column sums of dY
        dZ = (dY B^T) * act'(Z)
        dA = X^T dZ,   da = column sums of dZ,   dX = dZ A^T

    Math layout as everywhere here (A [H x F], B [F x H]).  ``a`` may be
    None (no column bias; da is then still returned).  Returns a dict with
    dX, dA, da, dB, db.
    """
    f, fp = _act_and_grad(act)
    X, A, B, dY = _f64(X), _f64(A), _f64(B), _f64(dY)
    Z = linear(X, A, a)
    Hd = f(Z)
    dZ = (dY @ B.T) * fp(Z)
    return {"dX": dZ @ A.T, "dA": X.T @ dZ, "da": dZ.sum(axis=0),
            "dB": Hd.T @ dY, "db": dY.sum(axis=0)}


def mlp_backward_sharded(X, A, a, B, dY, N, act="gelu"):
    """The backward of the paired layer over N shards, each shard's work
    written out.

    The gradient of the full output reaches every shard whole (the forward's
    sum was an all-reduce), so shard i forms dH_i = dY B_i^T for its own
    intermediate slice, dZ_i = dH_i * act'(Z_i) on that slice, and its local
    weight gradients dA_i = X^T dZ_i, da_i, dB_i = H_i^T dY with no exchange.
    Its input gradient dZ_i A_i^T is only a partial of the full dX (X was
    replicated in the forward), so the N partials are summed: the all-reduce
    of the column layer's backward ([Scratch] section 4: identity in the
    forward, all-reduce in the backward; [Blog] 4.1: the input-gradient
    reduction needs an all-reduce).  The row bias gradient is the column sum
    of dY, formed once and not per shard ([Basics] bias remark: the row bias
    enters once).  Partials are summed in shard order.

    Returns the unsharded-layout gradients (dA with the shards' columns
    side by side, dB with their rows stacked) plus the list of dX partials.
    """
    f, fp = _act_and_grad(act)
    X, dY = _f64(X), _f64(dY)
    As = column_shards(A, N)
    Bs = row_shards(B, N)
    s = As[0].shape[1]
    a_s = [None] * N if a is None else [_f64(a)[i * s:(i + 1) * s] for i in range(N)]
    dA, da, dB, parts = [], [], [], []
    for Ai, ai, Bi in zip(As, a_s, Bs):
        Zi = linear(X, Ai, ai)
        dZi = (dY @ Bi.T) * fp(Zi)
        dA.append(X.T @ dZi)
        da.append(dZi.sum(axis=0))
        dB.append(f(Zi).T @ dY)
        parts.append(dZi @ Ai.T)
    return {"dX": _fold(parts), "dA": np.concatenate(dA, axis=1),
            "da": np.concatenate(da), "dB": np.concatenate(dB, axis=0),
            "db": dY.sum(axis=0), "dX_parts": parts}


def silu_grad(g):
    """Derivative of SiLU: d/dg [g sigmoid(g)] = sigmoid(g) (1 + g (1 - sigmoid(g)))."""
    g = _f64(g)
    sg = expit(g)
    return sg * (1.0 + g * (1.0 - sg))


def mlp_swiglu_backward(X, Wg, Wu, Wd, dY):
    """Gradients of the unsharded SwiGLU MLP Y = (SiLU(X Wg) * (X Wu)) Wd for
    an upstream gradient dY (no biases):

        G = X Wg, U = X Wu, Hd = SiLU(G) * U
        dWd = Hd^T dY,  dH = dY Wd^T
        dG = dH * U * SiLU'(G),  dU = dH * SiLU(G)
        dWg = X^T dG,  dWu = X^T dU,  dX = dG Wg^T + dU Wu^T

    Math layout (Wg, Wu [H x I], Wd [I x H])."""
    X, Wg, Wu, Wd, dY = (_f64(a) for a in (X, Wg, Wu, Wd, dY))
    G, U = X @ Wg, X @ Wu
    dH = dY @ Wd.T
    dG = dH * U * silu_grad(G)
    dU = dH * silu(G)
    return {"dX": dG @ Wg.T + dU @ Wu.T, "dWg": X.T @ dG, "dWu": X.T @ dU, "dWd": (silu(G) * U).T @ dY,
            "db": dY.sum(axis=0)}


def mlp_swiglu_backward_sharded(X, fused_blocks, Wd, dY, N):
    """The SwiGLU backward over N shards from the per-shard fused [gate | up]
    blocks: shard i forms dH_i = dY Wd_i^T, the gradient of its block
    dZ_i = [dG_i | dU_i], the block's weight gradient X^T dZ_i, its rows of
    dWd, and the input-gradient partial dZ_i F_i^T; the partials are summed
    in shard order (the column layer's backward all-reduce, [Scratch] 4)."""
    X, dY = _f64(X), _f64(dY)
    Wds = row_shards(Wd, N)
    dF, dWd, parts = [], [], []
    for Fi, Wdi in zip(fused_blocks, Wds):
        Fi = _f64(Fi)
        Z = X @ Fi
        s = Z.shape[1] // 2
        G, U = Z[:, :s], Z[:, s:]
        dH = dY @ Wdi.T
        dZ = np.concatenate([dH * U * silu_grad(G), dH * silu(G)], axis=1)
        dF.append(X.T @ dZ)
        dWd.append((silu(G) * U).T @ dY)
        parts.append(dZ @ Fi.T)
    return {"dX": _fold(parts), "dF": dF, "dWd": np.concatenate(dWd, axis=0), "db": dY.sum(axis=0),
            "dX_parts": parts}


# --------------------------------------------------------------------------
# vocab-parallel output head and cross-entropy
# --------------------------------------------------------------------------
def padded_vocab(V, N, multiple=8):
    """Vocab padded so that it splits into N equal shards whose width is a
    multiple of ``multiple`` ([Blog] 6.2: pad the vocab to a size TP divides,
    and drop the padding from the loss).  Returns (Vp, Vs)."""
    Vs = -(-V // N)
    Vs = -(-Vs // multiple) * multiple
    return N * Vs, Vs


def cross_entropy(logits, labels):
    """Per-row cross-entropy of softmax(logits) at the label:
    logsumexp(row) - row[label] (scipy's logsumexp)."""
    from scipy.special import logsumexp

    L = _f64(logits)
    labels = np.asarray(labels)
    return logsumexp(L, axis=1) - L[np.arange(L.shape[0]), labels]


def lm_head_ce(X, E, labels, V):
    """Unsharded output head and loss: logits = X E^T over the V real vocab
    rows of E ([V' x H], V' >= V rows; rows past V are padding and take no
    part), then the per-token cross-entropy."""
    E = _f64(E)[:V]
    return cross_entropy(_f64(X) @ E.T, labels)


def vocab_parallel_ce(X, E, labels, V, N):
    """The same loss with the vocab split over N shards ([Blog] 6.2: each
    shard computes only its own vocab partition's logits and its part of the
    loss, then an all-reduce combines them; padding is dropped from the loss).

    Shard i owns padded vocab rows [i Vs, (i+1) Vs); entries >= V are padding
    and are left out.  Per token, shard i forms its local maximum m_i, its
    local sum s_i = sum exp(l - m_i) and its target logit z_i (0 when the
    label is not in its partition).  The combine, in shard order, is
        M = max_i m_i,  S = sum_i s_i exp(m_i - M),  target = sum_i z_i,
        loss = log S + M - target.
    A shard with no real vocab entries contributes nothing.
    Returns (per-token losses, the per-shard (m, s, z) arrays).
    """
    X = _f64(X)
    labels = np.asarray(labels)
    Vp, Vs = padded_vocab(V, N)
    T = X.shape[0]
    ms, ss, zs = [], [], []
    for i in range(N):
        lo, hi = i * Vs, min((i + 1) * Vs, V)
        if hi <= lo:
            ms.append(np.full(T, -np.inf))
            ss.append(np.zeros(T))
            zs.append(np.zeros(T))
            continue
        L = X @ _f64(E)[lo:hi].T
        m = L.max(axis=1)
        ms.append(m)
        ss.append(np.exp(L - m[:, None]).sum(axis=1))
        own = (labels >= lo) & (labels < hi)
        z = np.zeros(T)
        z[own] = L[np.arange(T)[own], labels[own] - lo]
        zs.append(z)
    M = ms[0].copy()
    for m in ms[1:]:
        M = np.maximum(M, m)
    S = np.zeros(T)
    for m, s_ in zip(ms, ss):
        S = S + s_ * np.exp(m - M)
    target = _fold(zs)
    return np.log(S) + M - target, (ms, ss, zs)


def vocab_parallel_embedding(ids, E, V, N):
    """Input side of the vocab split ([Blog] 6.2: the embedding matrix
    (vocab, hidden) is split along the vocab like the output head;
    [Wiki] practice section: vocab-parallel embedding).  Shard i owns padded
    vocab rows [i Vs, (i+1) Vs) and looks up only the ids it owns, writing
    zero rows for the others; the N partials are summed in shard order (the
    all-reduce), so every token gets exactly its own row.  Rows >= V are
    padding and never read; an id outside [0, V) has no owner and gets a
    zero row.  The rows a shard does not own hold -0.0, the additive identity
    of IEEE arithmetic (x + (-0.0) == x bit for bit, a stored -0.0 included),
    so the sum reproduces the table's bits exactly, signed zeros too; an
    unowned id gets a -0.0 row.  Returns (rows [T x H], list of per-shard
    partials)."""
    ids = np.asarray(ids)
    E = _f64(E)
    Vp, Vs = padded_vocab(V, N)
    T, H = ids.shape[0], E.shape[1]
    parts = []
    for i in range(N):
        lo, hi = i * Vs, min((i + 1) * Vs, V)
        own = (ids >= lo) & (ids < hi)
        P = np.full((T, H), -0.0)
        P[own] = E[ids[own]]
        parts.append(P)
    return _fold(parts), parts


# --------------------------------------------------------------------------
# fixed-order fp32 reduction (for the bit-exact pin of the on-device fold)
# --------------------------------------------------------------------------
def to_bf16(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with round-to-nearest-even, returned as the uint16 bit
    patterns.  The rounding itself is torch's CPU cast (a library routine)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def reduce_partials_fp32(parts, bias=None, out="f32", n_slices=1, slice_=-1):
    """Sum of partials in fp32, left-folded in shard order, bias added once
    after the sum, then (for out='bf16') one round-to-nearest-even cast.

    This is the arithmetic of the stand-in for the row all-reduce written out
    in the precision the device uses: each ``+`` is one IEEE fp32 addition
    (numpy float32, round to nearest even).  ``slice_`` selects one of
    ``n_slices`` contiguous row blocks (the reduce-scatter output).
    Returns float32 values (out='f32') or uint16 bf16 bit patterns.
    """
    acc = np.array(parts[0], dtype=np.float32, copy=True)
    for p in parts[1:]:
        acc = acc + np.asarray(p, dtype=np.float32)
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float32)[None, :]
    if slice_ >= 0:
        acc = rs_slice(acc, n_slices, slice_)
    if out == "f32":
        return acc
    if out == "bf16":
        return to_bf16(acc)
    raise ValueError(out)
