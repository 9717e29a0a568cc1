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


def workload(kind, host, batch=None, seq=None, heads=None, rows=None):
    """Expected output rows of one workload ("mlp_gelu" | "mlp_swiglu" | "attn")."""
    if kind == "mlp_gelu":
        return mlp_gelu(host["X"], host["A"], host["a"], host["B"], host["b"], rows)
    if kind == "mlp_swiglu":
        return mlp_swiglu(host["X"], host["Wg"], host["Wu"], host["Wd"], rows)
    if kind == "attn":
        return attention(host["X"], host["Wq"], host["Wk"], host["Wv"], host["Wo"], batch, seq, heads, rows)
    raise ValueError(kind)
