"""Pins of the oracle's vocab-parallel output head and cross-entropy.

Checked against a pure-Python loop cross-entropy (tests/_brute.py), closed
forms (uniform logits give log V, a single dominant logit gives
log(1 + (V-1) e^-L)), the shift invariance of softmax, and the sharded form
against the unsharded one for vocab sizes the shard count does not divide.
Planted mistakes must fail.
"""
import math

import numpy as np
import pytest

from oracle import tp_oracle as O
from tests import _brute as brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(seed, T=6, H=8, V=37, pad_to=None):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, H))
    rows = V if pad_to is None else pad_to
    E = rng.standard_normal((rows, H)) * 0.5
    labels = rng.integers(0, V, T)
    return X, E, labels


def test_padded_vocab():
    assert O.padded_vocab(150000, 8) == (150016, 18752)
    assert O.padded_vocab(64, 8) == (64, 8)
    assert O.padded_vocab(37, 4) == (64, 16)
    for V in (1, 7, 37, 1000, 50257):
        for N in (1, 2, 3, 8):
            Vp, Vs = O.padded_vocab(V, N)
            assert Vp == N * Vs and Vp >= V and Vs % 8 == 0 and Vp - V < N * 8 + N


def test_cross_entropy_matches_brute_force():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((5, 11)) * 3
    y = rng.integers(0, 11, 5)
    want = brute.cross_entropy(L.tolist(), y.tolist())
    assert np.max(np.abs(O.cross_entropy(L, y) - want)) <= 1e-12


def test_uniform_logits_give_log_vocab():
    """E = 0 makes every real logit 0: the loss is log V exactly, whatever the
    labels and however the vocab is padded and split."""
    T, H, V = 4, 8, 37
    X = np.random.default_rng(2).standard_normal((T, H))
    for N in (1, 2, 4, 8):
        Vp, _ = O.padded_vocab(V, N)
        E = np.zeros((Vp, H))
        loss, _ = O.vocab_parallel_ce(X, E, np.array([0, 5, 36, 17]), V, N)
        assert np.max(np.abs(loss - math.log(V))) <= 1e-14


def test_dominant_logit_closed_form():
    """Logits L at the label and 0 elsewhere: loss = log(1 + (V-1) e^-L)."""
    V, Lval = 20, 3.5
    labels = np.array([0, 7, 19])
    logits = np.zeros((3, V))
    logits[np.arange(3), labels] = Lval
    want = math.log(1.0 + (V - 1) * math.exp(-Lval))
    assert np.max(np.abs(O.cross_entropy(logits, labels) - want)) <= 1e-14


def test_shift_invariance():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((4, 9))
    y = rng.integers(0, 9, 4)
    assert np.max(np.abs(O.cross_entropy(L + 123.0, y) - O.cross_entropy(L, y))) <= 1e-12


@pytest.mark.parametrize("V,N", [(37, 1), (37, 2), (37, 4), (37, 3), (64, 8), (9, 8)])
def test_vocab_parallel_equals_unsharded(V, N):
    """Including splits where the last shards hold only padding (V=9, N=8)."""
    Vp, _ = O.padded_vocab(V, N)
    X, E, labels = _case(10 + V + N, V=V, pad_to=Vp)
    E[V:] = 7.0  # padding rows hold values that must not leak into the loss
    loss, _ = O.vocab_parallel_ce(X, E, labels, V, N)
    want = O.lm_head_ce(X, E, labels, V)
    assert np.max(np.abs(loss - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))
    brute_loss = brute.cross_entropy((X @ E[:V].T).tolist(), labels.tolist())
    assert np.max(np.abs(loss - brute_loss)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_each_label_has_exactly_one_owner():
    V, N = 37, 4
    Vp, Vs = O.padded_vocab(V, N)
    X, E, labels = _case(5, V=V, pad_to=Vp)
    labels = np.arange(V)[: X.shape[0]]
    _, (ms, ss, zs) = O.vocab_parallel_ce(X, E, labels, V, N)
    owners = np.stack([(labels >= i * Vs) & (labels < min((i + 1) * Vs, V)) for i in range(N)])
    assert np.all(owners.sum(axis=0) == 1)
    for i in range(N):
        assert np.all(zs[i][~owners[i]] == 0.0)


# ------------------------------------------------------------------ planted mistakes
def _mutant(kind, X, E, labels, V, N):
    Vp, Vs = O.padded_vocab(V, N)
    if kind == "padding_not_dropped":
        return O.cross_entropy(X @ E[:Vp].T, labels)
    if kind == "no_rescale_in_combine":
        _, (ms, ss, zs) = O.vocab_parallel_ce(X, E, labels, V, N)
        M = np.max(np.stack(ms), axis=0)
        return np.log(np.sum(np.stack(ss), axis=0)) + M - np.sum(np.stack(zs), axis=0)
    if kind == "target_from_every_shard":
        L = X @ E[:V].T
        lse = O.cross_entropy(L, labels) + L[np.arange(len(labels)), labels]
        return lse - N * L[np.arange(len(labels)), labels]
    if kind == "local_loss_summed":
        _, (ms, ss, zs) = O.vocab_parallel_ce(X, E, labels, V, N)
        return sum(np.log(s_) + m - z for m, s_, z in zip(ms, ss, zs))
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["padding_not_dropped", "no_rescale_in_combine", "target_from_every_shard",
                                  "local_loss_summed"])
def test_planted_vocab_mistakes_are_caught(kind):
    V, N = 37, 4
    Vp, _ = O.padded_vocab(V, N)
    X, E, labels = _case(21, V=V, pad_to=Vp)
    E[V:] = 0.0
    want = O.lm_head_ce(X, E, labels, V)
    assert np.max(np.abs(O.vocab_parallel_ce(X, E, labels, V, N)[0] - want)) <= 1e-12
    assert np.max(np.abs(_mutant(kind, X, E, labels, V, N) - want)) > 1e-3


# ------------------------------------------------------------------ embedding (input side)
@pytest.mark.parametrize("V,N", [(37, 4), (64, 8), (9, 8), (1000, 3)])
def test_vocab_parallel_embedding_is_the_plain_lookup(V, N):
    rng = np.random.default_rng(V + N)
    Vp, Vs = O.padded_vocab(V, N)
    E = rng.standard_normal((Vp, 6))
    E[V:] = np.nan  # padding rows must never be read
    ids = rng.integers(0, V, 50)
    Y, parts = O.vocab_parallel_embedding(ids, E, V, N)
    assert np.array_equal(Y, E[ids])  # exact: one nonzero term per element
    nonzero = np.stack([np.any(p != 0, axis=1) for p in parts])
    assert np.all(nonzero.sum(axis=0) == 1)  # exactly one owner per token


def test_vocab_parallel_embedding_keeps_signed_zeros():
    """The lookup returns the table's bits, signed zeros included: a stored
    -0.0 comes back as -0.0 and +0.0 as +0.0 (the non-owning shards' rows
    are -0.0, the additive identity, so the fold adds nothing to either)."""
    V, N = 37, 4
    Vp, _ = O.padded_vocab(V, N)
    E = np.random.default_rng(5).standard_normal((Vp, 4))
    E[3] = [-0.0, 0.0, -0.0, 1.5]
    E[30] = [0.0, -0.0, 2.0, -0.0]
    ids = np.array([3, 30, 3, 12])
    Y, _ = O.vocab_parallel_embedding(ids, E, V, N)
    assert np.array_equal(Y.view(np.uint64), E[ids].view(np.uint64))
    # the plainer fold from +0.0 would lose the sign of every stored -0.0
    plus = np.zeros_like(Y) + Y
    assert not np.array_equal(plus.view(np.uint64), E[ids].view(np.uint64))


def test_vocab_parallel_embedding_out_of_range_ids_give_zero_rows():
    V, N = 20, 4
    Vp, _ = O.padded_vocab(V, N)
    E = np.arange(Vp * 3, dtype=float).reshape(Vp, 3) + 1.0
    Y, _ = O.vocab_parallel_embedding(np.array([-1, 0, 19, 20, Vp + 5]), E, V, N)
    assert np.array_equal(Y[[0, 3, 4]], np.zeros((3, 3)))
    assert np.array_equal(Y[[1, 2]], E[[0, 19]])


def test_planted_embedding_mistake_padding_owned():
    """A shard that also owns the padding rows of its range would read them."""
    V, N = 37, 4
    Vp, Vs = O.padded_vocab(V, N)
    E = np.ones((Vp, 2))
    E[V:] = np.nan
    ids = np.array([V + 1])  # a padding id, as a buggy tokenizer could emit
    Y, _ = O.vocab_parallel_embedding(ids, E, V, N)
    assert np.all(Y == 0)
    wrong = E[ids]  # looking up without the range check
    assert np.isnan(wrong).all()
