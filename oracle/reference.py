"""Oracle evaluation of whole workloads on the generator's arrays.

TEST INFRASTRUCTURE ONLY (see tp_oracle).  Weights arrive in the [out x in]
storage the generator draws them in; the math-layout matrices the oracle
uses are their transposes.  ``rows`` restricts the evaluation to some token
rows (the layers are token-wise except attention, whose rows are evaluated
with their full causal prefix).
"""
from __future__ import annotations

import numpy as np

from . import tp_oracle as O


def mlp_gelu(X, A, a, B, b, rows=None):
    Xr = X if rows is None else X[rows]
    return O.mlp_gelu(Xr, A.T, a, B.T, b)


def mlp_swiglu(X, Wg, Wu, Wd, rows=None):
    Xr = X if rows is None else X[rows]
    return O.mlp_swiglu(Xr, Wg.T, Wu.T, Wd.T)


def attention(X, Wq, Wk, Wv, Wo, batch, seq, heads, rows=None, bo=None):
    if rows is None:
        return O.attention_block(X, Wq.T, Wk.T, Wv.T, Wo.T, batch, seq, heads, bo=bo)
    return O.attention_block_rows(X, Wq.T, Wk.T, Wv.T, Wo.T, batch, seq, heads, np.asarray(rows), bo=bo)


def vocab_ce(X, E, labels, V, rows=None):
    """Per-token cross-entropy of the output head over the V real vocab rows
    of E ([>= V x H] storage), on some token rows."""
    if rows is None:
        return O.lm_head_ce(X, E, labels, V)
    rows = np.asarray(rows)
    return O.lm_head_ce(X[rows], E, np.asarray(labels)[rows], V)


def vocab_embed(E, ids, V, N, rows=None):
    """Embedding rows of the vocab-parallel lookup for the token rows
    ``rows`` (all if None); E is the table over the real vocab, [V x H]."""
    ids = np.asarray(ids)
    if rows is not None:
        ids = ids[rows]
    return O.vocab_parallel_embedding(ids, E, V, N)[0]


def norm_split(kind, X, g, b, eps, N, rows=None):
    """The hidden-split norm ("norm_split_layer" | "norm_split_rms") of the
    rows ``rows`` of X (all if None) over N equal parts of the hidden axis.
    Row-wise, so a row's value needs no other row."""
    Xr = np.asarray(X)
    if rows is not None:
        Xr = Xr[np.asarray(rows)]
    parts = np.split(Xr.astype(np.float64), N, axis=1)
    gp = np.split(np.asarray(g, dtype=np.float64), N)
    if kind == "norm_split_layer":
        bp = None if b is None else np.split(np.asarray(b, dtype=np.float64), N)
        return np.concatenate(O.layernorm_hidden_split(parts, gp, bp, eps), axis=1)
    return np.concatenate(O.rmsnorm_hidden_split(parts, gp, eps), axis=1)


def workload(kind, host, batch=None, seq=None, heads=None, rows=None, N=None, eps=1e-6):
    """Expected output rows of one workload ("mlp_gelu" | "mlp_swiglu" |
    "attn" | "vocab_ce": the per-token loss | "vocab_embed": N shards |
    "norm_split_layer" / "norm_split_rms": N shards, eps)."""
    if kind == "vocab_embed":
        return vocab_embed(host["E"], host["ids"], host["E"].shape[0], N, rows)
    if kind.startswith("norm_split"):
        return norm_split(kind, host["X"], host["g"], host["b"] if kind == "norm_split_layer" else None, eps, N, rows)
    if kind == "vocab_ce":
        return vocab_ce(host["X"], host["E"], host["labels"], host["E"].shape[0], rows)
    if kind == "mlp_gelu":
        return mlp_gelu(host["X"], host["A"], host["a"], host["B"], host["b"], rows)
    if kind == "mlp_swiglu":
        return mlp_swiglu(host["X"], host["Wg"], host["Wu"], host["Wd"], rows)
    if kind == "attn":
        return attention(host["X"], host["Wq"], host["Wk"], host["Wv"], host["Wo"], batch, seq, heads, rows)
    raise ValueError(kind)


def mlp_gelu_backward(X, A, a, B, dY, act="gelu"):
    """Full backward of the GELU MLP on storage-layout weights (A [F x H],
    B [H x F]); gradients come back in that same storage layout
    (dA [F x H], dB [H x F])."""
    g = O.mlp_backward(X, A.T, a, B.T, dY, act=act)
    return {"dX": g["dX"], "dA": g["dA"].T, "da": g["da"], "dB": g["dB"].T, "db": g["db"]}


def mlp_gelu_backward_sample(X, A, a, B, dY, rows, feats):
    """Sampled entries of the same gradients (storage layout), each from the
    definition in ``tp_oracle.mlp_backward`` restricted to what it needs:
    dX[rows, :] needs dZ on those token rows only; dA[feats, :], da[feats]
    and dB[:, feats] need the pre-activation of those features over all
    tokens only; db is the full column sum of dY."""
    X64 = np.asarray(X, dtype=np.float64)
    dY64 = np.asarray(dY, dtype=np.float64)
    A64 = np.asarray(A, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    a64 = None if a is None else np.asarray(a, dtype=np.float64)
    rows = np.asarray(rows)
    feats = np.asarray(feats)
    Zr = O.linear(X64[rows], A64.T, a64)
    dZr = (dY64[rows] @ B64) * O.gelu_grad(Zr)
    Zf = O.linear(X64, A64[feats].T, None if a64 is None else a64[feats])
    dZf = (dY64 @ B64[:, feats]) * O.gelu_grad(Zf)
    return {"dX": dZr @ A64, "dA": dZf.T @ X64, "da": dZf.sum(axis=0),
            "dB": dY64.T @ O.gelu(Zf), "db": dY64.sum(axis=0)}


def mlp_swiglu_backward(X, Wg, Wu, Wd, dY):
    """SwiGLU backward on storage-layout weights (Wg, Wu [I x H], Wd [H x I]);
    gradients in the same layout."""
    g = O.mlp_swiglu_backward(X, Wg.T, Wu.T, Wd.T, dY)
    return {"dX": g["dX"], "dWg": g["dWg"].T, "dWu": g["dWu"].T, "dWd": g["dWd"].T, "db": g["db"]}


def mlp_swiglu_backward_sample(X, Wg, Wu, Wd, dY, rows, feats):
    """Sampled entries (storage layout): dX[rows, :]; dWg[feats, :],
    dWu[feats, :] and dWd[:, feats] for intermediate features ``feats``."""
    X64, dY64 = np.asarray(X, dtype=np.float64), np.asarray(dY, dtype=np.float64)
    Wg64, Wu64, Wd64 = (np.asarray(a, dtype=np.float64) for a in (Wg, Wu, Wd))
    rows, feats = np.asarray(rows), np.asarray(feats)
    Gr, Ur = X64[rows] @ Wg64.T, X64[rows] @ Wu64.T
    dHr = dY64[rows] @ Wd64
    dGr, dUr = dHr * Ur * O.silu_grad(Gr), dHr * O.silu(Gr)
    Gf, Uf = X64 @ Wg64[feats].T, X64 @ Wu64[feats].T
    dHf = dY64 @ Wd64[:, feats]
    dGf, dUf = dHf * Uf * O.silu_grad(Gf), dHf * O.silu(Gf)
    return {"dX": dGr @ Wg64 + dUr @ Wu64, "dWg": dGf.T @ X64, "dWu": dUf.T @ X64,
            "dWd": dY64.T @ (O.silu(Gf) * Uf), "db": dY64.sum(axis=0)}
