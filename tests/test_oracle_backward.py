"""Pins of the oracle's backward of the MLP pair.

The gradients are pinned against central finite differences of the
pure-Python brute-force forward (tests/_brute.py: nested loops and math.erf,
no numpy, no oracle code), which fixes every gradient term independently of
how the oracle writes it.  The sharding identities of the backward (local
weight gradients, one reduction of the input-gradient partials, the row bias
gradient formed once) are checked exactly on integer inputs with the identity
activation, and to 1e-12 with GELU.  Planted mistakes must fail the pins.
"""
import math

import numpy as np
import pytest

from oracle import reference as R
from oracle import tp_oracle as O
from tests import _brute as brute


def _loss(dY, X, A, a, B, b):
    Y = brute.mlp_gelu(X.tolist(), A.tolist(), None if a is None else a.tolist(), B.tolist(),
                       None if b is None else b.tolist())
    return sum(dy * y for dr, yr in zip(dY.tolist(), Y) for dy, y in zip(dr, yr))


def _fd_grads(X, A, a, B, b, dY, h=1e-5):
    """Central differences of sum(dY * Y) with respect to every input entry."""
    args = {"X": X, "A": A, "a": a, "B": B, "b": b}
    out = {}
    for name, arr in args.items():
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = _loss(dY, **args)
            arr[idx] = keep - h
            lm = _loss(dY, **args)
            arr[idx] = keep
            g[idx] = (lp - lm) / (2 * h)
        out["d" + name] = g
    return out


def _tiny(seed, T=3, H=4, F=8):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, H))
    A = rng.standard_normal((H, F)) * 0.7
    a = rng.standard_normal(F) * 0.3
    B = rng.standard_normal((F, H)) * 0.7
    b = rng.standard_normal(H) * 0.3
    dY = rng.standard_normal((T, H))
    return X, A, a, B, b, dY


def _close(g, ref, tol):
    return np.max(np.abs(np.asarray(g) - ref)) <= tol * max(1.0, np.max(np.abs(ref)))


def _matches_fd(grads, fd, tol=1e-7):
    return all(_close(grads[k], fd[k], tol) for k in ("dX", "dA", "da", "dB", "db"))


# ------------------------------------------------------------------ GELU'
def test_gelu_grad_matches_finite_differences_of_brute_gelu():
    """d/dz of the exact GELU, against central differences of math.erf's GELU."""
    h = 1e-5
    for z in np.linspace(-6.0, 6.0, 97):
        fd = (brute.gelu(z + h) - brute.gelu(z - h)) / (2 * h)
        assert abs(O.gelu_grad(z) - fd) <= 1e-9


def test_gelu_grad_closed_forms():
    # GELU'(0) = Phi(0) = 1/2
    assert O.gelu_grad(0.0) == 0.5
    # GELU(z) - GELU(-z) = z  =>  GELU'(z) + GELU'(-z) = 1
    z = np.linspace(-8, 8, 161)
    assert np.max(np.abs(O.gelu_grad(z) + O.gelu_grad(-z) - 1.0)) <= 1e-15
    # far tails: GELU -> z and -> 0, so the slope -> 1 and -> 0
    assert abs(O.gelu_grad(12.0) - 1.0) <= 1e-15 and abs(O.gelu_grad(-12.0)) <= 1e-15
    # the slope peaks where z phi'(z) + 2 phi(z) = 0, i.e. z = sqrt 2, at
    # Phi(sqrt 2) + sqrt 2 phi(sqrt 2)
    zs = np.linspace(1.0, 2.0, 100001)
    assert abs(zs[np.argmax(O.gelu_grad(zs))] - math.sqrt(2.0)) <= 2e-5


# ------------------------------------------------------------------ gradients
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mlp_backward_matches_finite_differences(seed):
    X, A, a, B, b, dY = _tiny(seed)
    fd = _fd_grads(X, A, a, B, b, dY)
    g = O.mlp_backward(X, A, a, B, dY)
    assert _matches_fd(g, fd)


def test_storage_layout_backward_matches_finite_differences():
    """The storage-layout wrapper (weights [out x in]) returns gradients in
    that layout: dA[f, h] = d sum(dY*Y) / d A_storage[f, h]."""
    X, A, a, B, b, dY = _tiny(7, T=4, H=4, F=6)
    fd = _fd_grads(X, A, a, B, b, dY)
    g = R.mlp_gelu_backward(X, A.T.copy(), a, B.T.copy(), dY)
    assert _close(g["dA"], fd["dA"].T, 1e-7) and _close(g["dB"], fd["dB"].T, 1e-7)
    assert _close(g["dX"], fd["dX"], 1e-7) and _close(g["da"], fd["da"], 1e-7)
    assert _close(g["db"], fd["db"], 1e-7)


def test_sampled_backward_equals_full():
    rng = np.random.default_rng(11)
    T, H, F = 40, 16, 24
    X = rng.standard_normal((T, H))
    A = rng.standard_normal((F, H)) * 0.3
    a = rng.standard_normal(F) * 0.1
    B = rng.standard_normal((H, F)) * 0.3
    dY = rng.standard_normal((T, H))
    full = R.mlp_gelu_backward(X, A, a, B, dY)
    rows, feats = [0, 5, 39], [1, 2, 23]
    s = R.mlp_gelu_backward_sample(X, A, a, B, dY, rows, feats)
    tol = 1e-12
    assert _close(s["dX"], full["dX"][rows], tol)
    assert _close(s["dA"], full["dA"][feats], tol)
    assert _close(s["da"], full["da"][feats], tol)
    assert _close(s["dB"], full["dB"][:, feats], tol)
    assert _close(s["db"], full["db"], tol)


# ------------------------------------------------------------------ sharding
def test_sharded_backward_identity_activation_is_exact_on_integers():
    """With the identity activation and small-integer inputs every product
    is exact in fp64: the shards' weight gradients tile the full ones, the N
    input-gradient partials sum to the full dX, and db = column sums of dY."""
    rng = np.random.default_rng(5)
    T, H, F = 5, 6, 16
    X = rng.integers(-3, 4, (T, H)).astype(float)
    A = rng.integers(-3, 4, (H, F)).astype(float)
    a = rng.integers(-3, 4, F).astype(float)
    B = rng.integers(-3, 4, (F, H)).astype(float)
    dY = rng.integers(-3, 4, (T, H)).astype(float)
    full = O.mlp_backward(X, A, a, B, dY, act="none")
    # closed forms of the linear case
    assert np.array_equal(full["dX"], dY @ B.T @ A.T)
    assert np.array_equal(full["dB"], (X @ A + a).T @ dY)
    for N in (1, 2, 4, 8):
        sh = O.mlp_backward_sharded(X, A, a, B, dY, N, act="none")
        for k in ("dX", "dA", "da", "dB", "db"):
            assert np.array_equal(sh[k], full[k]), (N, k)
        assert len(sh["dX_parts"]) == N
        assert np.array_equal(sh["db"], dY.sum(axis=0))  # once, not N times


def test_sharded_gelu_backward_equals_unsharded():
    X, A, a, B, b, dY = _tiny(3, T=6, H=8, F=16)
    full = O.mlp_backward(X, A, a, B, dY)
    for N in (1, 2, 4, 8):
        sh = O.mlp_backward_sharded(X, A, a, B, dY, N)
        for k in ("dX", "dA", "da", "dB", "db"):
            assert _close(sh[k], full[k], 1e-12), (N, k)


def test_input_gradient_needs_the_reduction():
    """No single shard's partial is the input gradient; their sum is."""
    X, A, a, B, b, dY = _tiny(4, T=5, H=6, F=12)
    sh = O.mlp_backward_sharded(X, A, a, B, dY, 3)
    for p in sh["dX_parts"]:
        assert not _close(p, sh["dX"], 1e-3)
    assert _close(sum(sh["dX_parts"][1:], sh["dX_parts"][0]), sh["dX"], 1e-14)


# ------------------------------------------------------------------ planted mistakes
def _mutant(kind, X, A, a, B, dY, N=2):
    g = dict(O.mlp_backward_sharded(X, A, a, B, dY, N))
    Z = X @ A + a
    dH = dY @ B.T
    if kind == "gelu_grad_without_density_term":
        dZ = dH * 0.5 * (1.0 + np.vectorize(math.erf)(Z / math.sqrt(2.0)))
        g.update(dX=dZ @ A.T, dA=X.T @ dZ, da=dZ.sum(0))
    elif kind == "activation_value_for_slope":
        dZ = dH * O.gelu(Z)
        g.update(dX=dZ @ A.T, dA=X.T @ dZ, da=dZ.sum(0))
    elif kind == "no_input_gradient_reduction":
        g["dX"] = g["dX_parts"][0]
    elif kind == "row_bias_gradient_per_shard":
        g["db"] = N * dY.sum(axis=0)
    elif kind == "pre_activation_for_row_gradient":
        g["dB"] = Z.T @ dY
    elif kind == "column_bias_gradient_from_dH":
        g["da"] = dH.sum(axis=0)
    else:
        raise ValueError(kind)
    return g


@pytest.mark.parametrize("kind", [
    "gelu_grad_without_density_term", "activation_value_for_slope", "no_input_gradient_reduction",
    "row_bias_gradient_per_shard", "pre_activation_for_row_gradient", "column_bias_gradient_from_dH",
])
def test_planted_backward_mistakes_are_caught(kind):
    X, A, a, B, b, dY = _tiny(9)
    fd = _fd_grads(X, A, a, B, b, dY)
    assert _matches_fd(O.mlp_backward_sharded(X, A, a, B, dY, 2), fd)
    assert not _matches_fd(_mutant(kind, X, A, a, B, dY), fd)


# ------------------------------------------------------------------ SwiGLU
def _swiglu_loss(dY, X, Wg, Wu, Wd):
    Y = brute.mlp_swiglu(X.tolist(), Wg.tolist(), Wu.tolist(), Wd.tolist())
    return sum(dy * y for dr, yr in zip(dY.tolist(), Y) for dy, y in zip(dr, yr))


def _swiglu_fd(X, Wg, Wu, Wd, dY, h=1e-5):
    args = {"X": X, "Wg": Wg, "Wu": Wu, "Wd": Wd}
    out = {}
    for name, arr in args.items():
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = _swiglu_loss(dY, **args)
            arr[idx] = keep - h
            lm = _swiglu_loss(dY, **args)
            arr[idx] = keep
            g[idx] = (lp - lm) / (2 * h)
        out["d" + name] = g
    return out


def _swiglu_tiny(seed, T=3, H=4, I=6):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, H)), rng.standard_normal((H, I)) * 0.7, rng.standard_normal((H, I)) * 0.7,
            rng.standard_normal((I, H)) * 0.7, rng.standard_normal((T, H)))


def test_silu_grad_matches_finite_differences_of_brute_silu():
    h = 1e-5
    for g in np.linspace(-8.0, 8.0, 81):
        fd = (brute.silu(g + h) - brute.silu(g - h)) / (2 * h)
        assert abs(O.silu_grad(g) - fd) <= 1e-9
    assert O.silu_grad(0.0) == 0.5
    # SiLU(g) - SiLU(-g) = g  =>  SiLU'(g) + SiLU'(-g) = 1
    z = np.linspace(-10, 10, 101)
    assert np.max(np.abs(O.silu_grad(z) + O.silu_grad(-z) - 1.0)) <= 1e-15


@pytest.mark.parametrize("seed", [0, 1])
def test_swiglu_backward_matches_finite_differences(seed):
    X, Wg, Wu, Wd, dY = _swiglu_tiny(seed)
    fd = _swiglu_fd(X, Wg, Wu, Wd, dY)
    g = O.mlp_swiglu_backward(X, Wg, Wu, Wd, dY)
    for k in ("dX", "dWg", "dWu", "dWd"):
        assert _close(g[k], fd[k], 1e-7), k


def test_swiglu_sharded_backward_equals_unsharded():
    X, Wg, Wu, Wd, dY = _swiglu_tiny(2, T=5, H=6, I=8)
    full = O.mlp_swiglu_backward(X, Wg, Wu, Wd, dY)
    for N in (1, 2, 4):
        blocks = O.swiglu_fused_blocks(Wg, Wu, N)
        sh = O.mlp_swiglu_backward_sharded(X, blocks, Wd, dY, N)
        s = Wg.shape[1] // N
        for i in range(N):  # block i's gradient is [dWg columns i | dWu columns i]
            want = np.concatenate([full["dWg"][:, i * s:(i + 1) * s], full["dWu"][:, i * s:(i + 1) * s]], axis=1)
            assert _close(sh["dF"][i], want, 1e-12)
        assert _close(sh["dX"], full["dX"], 1e-12) and _close(sh["dWd"], full["dWd"], 1e-12)


def test_swiglu_storage_and_sampled_forms():
    X, Wg, Wu, Wd, dY = _swiglu_tiny(3, T=12, H=8, I=10)
    full = O.mlp_swiglu_backward(X, Wg, Wu, Wd, dY)
    st = R.mlp_swiglu_backward(X, Wg.T.copy(), Wu.T.copy(), Wd.T.copy(), dY)
    assert _close(st["dWg"], full["dWg"].T, 1e-14) and _close(st["dWd"], full["dWd"].T, 1e-14)
    rows, feats = [0, 7, 11], [0, 3, 9]
    sm = R.mlp_swiglu_backward_sample(X, Wg.T.copy(), Wu.T.copy(), Wd.T.copy(), dY, rows, feats)
    assert _close(sm["dX"], st["dX"][rows], 1e-12)
    assert _close(sm["dWg"], st["dWg"][feats], 1e-12) and _close(sm["dWu"], st["dWu"][feats], 1e-12)
    assert _close(sm["dWd"], st["dWd"][:, feats], 1e-12)


@pytest.mark.parametrize("kind", ["gate_slope_without_up", "up_gradient_with_slope", "naive_block_split"])
def test_planted_swiglu_backward_mistakes_are_caught(kind):
    X, Wg, Wu, Wd, dY = _swiglu_tiny(4)
    fd = _swiglu_fd(X, Wg, Wu, Wd, dY)
    G, U = X @ Wg, X @ Wu
    dH = dY @ Wd.T
    if kind == "gate_slope_without_up":
        dG, dU = dH * O.silu_grad(G), dH * O.silu(G)
        got = {"dWg": X.T @ dG}
        key = "dWg"
    elif kind == "up_gradient_with_slope":
        dU = dH * O.silu_grad(G)
        got = {"dWu": X.T @ dU}
        key = "dWu"
    else:  # splitting [Wg | Wu] into N column blocks hands gate-only columns to shard 0
        N = 2
        naive = [np.concatenate([Wg, Wu], axis=1)[:, i * Wg.shape[1]:(i + 1) * Wg.shape[1]] for i in range(N)]
        sh = O.mlp_swiglu_backward_sharded(X, naive, Wd, dY, N)
        got = {"dX": sh["dX"]}
        key = "dX"
    assert not _close(got[key], fd[key], 1e-3)
