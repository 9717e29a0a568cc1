"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

Every check here is independent of the oracle's own code: sharding identities
on integer inputs (exact in fp64), closed forms, textbook values, IEEE
rounding worked by hand, and a pure-Python brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import tp_oracle as O
from tests import _brute as brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _ints(rng, shape, lo=-4, hi=5):
    return rng.integers(lo, hi, size=shape).astype(np.float64)


# ---------------------------------------------------------------- identities
def test_I1_column_concat_is_full_product_bitwise():
    """Concatenating the column shards' outputs gives X A exactly
    (column-split equation of the wiki page)."""
    rng = np.random.default_rng(1)
    for N in (1, 2, 4, 8):
        X = _ints(rng, (7, 12))
        A = _ints(rng, (12, 8 * 3))
        a = _ints(rng, (8 * 3,))
        parts = O.column_linear_sharded(X, A, a, N)
        assert np.array_equal(np.concatenate(parts, axis=1), X @ A + a)


def test_I2_row_partials_sum_to_full_product_bitwise():
    """Sum of the row partials X_i B_i is X B exactly (row-split equation)."""
    rng = np.random.default_rng(2)
    for N in (1, 2, 4, 8):
        H = _ints(rng, (5, 8 * 2))
        B = _ints(rng, (8 * 2, 9))
        parts = O.row_partials(H, B, N)
        assert all(p.shape == (5, 9) for p in parts)  # every partial is full-shape
        assert np.array_equal(sum(parts[1:], parts[0]), H @ B)


def test_I3_sharded_gelu_mlp_equals_unsharded():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((6, 16))
    A = rng.standard_normal((16, 32)) * 0.3
    a = rng.standard_normal(32) * 0.1
    B = rng.standard_normal((32, 16)) * 0.3
    b = rng.standard_normal(16) * 0.1
    Y = O.mlp_gelu(X, A, a, B, b)
    for N in (1, 2, 4, 8):
        Ys = O.mlp_gelu_sharded(X, A, a, B, b, N)
        assert np.max(np.abs(Ys - Y)) <= 1e-12 * np.max(np.abs(Y))


def test_I4_bias_counted_once():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((5, 8))
    A = rng.standard_normal((8, 16))
    a = rng.standard_normal(16)
    b = rng.standard_normal(8)
    for N in (2, 4):
        # B = 0  =>  Y == b exactly (not N * b)
        Y0 = O.mlp_gelu_sharded(X, A, a, np.zeros((16, 8)), b, N)
        assert np.array_equal(Y0, np.broadcast_to(b, Y0.shape))
        # adding b moves every output by b, not by N * b
        B = rng.standard_normal((16, 8))
        diff = O.mlp_gelu_sharded(X, A, a, B, b, N) - O.mlp_gelu_sharded(X, A, a, B, None, N)
        assert np.max(np.abs(diff - b[None, :])) < 1e-12


def test_hand_worked_two_shard_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_worked_split.json")))
    X, A, B, b = (np.array(g[k], dtype=np.float64) for k in ("X", "A", "B", "b"))
    cols = O.column_linear_sharded(X, A, None, g["N"])
    assert np.array_equal(cols[0], g["XA_shard0"])
    assert np.array_equal(cols[1], g["XA_shard1"])
    assert np.array_equal(O.linear(X, A), g["XA"])
    P = O.row_partials(np.array(g["XA"], dtype=np.float64), B, g["N"])
    assert np.array_equal(P[0], g["P_shard0"])
    assert np.array_equal(P[1], g["P_shard1"])
    assert np.array_equal(O.reduce_partials_fp32(P, b, out="f32"), np.array(g["Y"], np.float32))


# ---------------------------------------------------------------- activations
def test_gelu_textbook_values(golden_dir):
    tab = json.load(open(os.path.join(golden_dir, "normal_cdf_table.json")))["values"]
    for x, phi in tab:
        assert O.gelu(x) == pytest.approx(x * phi, abs=1e-15, rel=1e-13)


def test_gelu_invariants():
    x = np.linspace(-8, 8, 2001)
    assert O.gelu(0.0) == 0.0
    # GELU(x) - GELU(-x) = x Phi(x) + x Phi(-x) ... = x  (Phi(x) + Phi(-x) = 1)
    assert np.max(np.abs(O.gelu(x) - O.gelu(-x) - x)) < 1e-14
    assert O.gelu(40.0) == 40.0 and abs(O.gelu(-40.0)) < 1e-300
    # the tanh approximation is NOT what the oracle computes (it differs by ~1e-4 somewhere)
    tanh = 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))
    assert np.max(np.abs(O.gelu(x) - tanh)) > 1e-4


def test_silu_closed_forms():
    assert O.silu(0.0) == 0.0
    # sigmoid(ln 3) = 3/4
    assert O.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    # sigmoid(-ln 3) = 1/4
    assert O.silu(-math.log(3.0)) == pytest.approx(-0.25 * math.log(3.0), rel=1e-15)
    x = np.linspace(-30, 30, 601)
    assert np.max(np.abs(O.silu(x) - O.silu(-x) - x)) < 1e-13
    assert O.silu(800.0) == 800.0 and O.silu(-800.0) == 0.0


# ---------------------------------------------------------------- brute force
def test_mlp_gelu_matches_brute_force():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((3, 4))
    A = rng.standard_normal((4, 8))
    a = rng.standard_normal(8)
    B = rng.standard_normal((8, 4))
    b = rng.standard_normal(4)
    ref = np.array(brute.mlp_gelu(X.tolist(), A.tolist(), a.tolist(), B.tolist(), b.tolist()))
    assert np.max(np.abs(O.mlp_gelu(X, A, a, B, b) - ref)) < 1e-13
    assert np.max(np.abs(O.mlp_gelu_sharded(X, A, a, B, b, 2) - ref)) < 1e-13


def test_mlp_swiglu_matches_brute_force_and_sharded():
    rng = np.random.default_rng(6)
    X = rng.standard_normal((3, 4))
    Wg = rng.standard_normal((4, 8))
    Wu = rng.standard_normal((4, 8))
    Wd = rng.standard_normal((8, 4))
    ref = np.array(brute.mlp_swiglu(X.tolist(), Wg.tolist(), Wu.tolist(), Wd.tolist()))
    assert np.max(np.abs(O.mlp_swiglu(X, Wg, Wu, Wd) - ref)) < 1e-13
    for N in (1, 2, 4):
        blocks = O.swiglu_fused_blocks(Wg, Wu, N)
        Ys = O.mlp_swiglu_sharded(X, blocks, Wd, N)
        assert np.max(np.abs(Ys - ref)) < 1e-13


def test_swiglu_fused_block_layout():
    """Block i = [gate columns of shard i | up columns of shard i]."""
    Wg = np.arange(4 * 12, dtype=np.float64).reshape(4, 12)
    Wu = -np.arange(4 * 12, dtype=np.float64).reshape(4, 12) - 1
    blocks = O.swiglu_fused_blocks(Wg, Wu, 3)
    for i, blk in enumerate(blocks):
        assert blk.shape == (4, 8)
        assert np.array_equal(blk[:, :4], Wg[:, 4 * i:4 * i + 4])
        assert np.array_equal(blk[:, 4:], Wu[:, 4 * i:4 * i + 4])


def test_attention_block_matches_brute_force():
    rng = np.random.default_rng(7)
    batch, seq, heads, d = 1, 5, 4, 2
    H = heads * d
    X = rng.standard_normal((batch * seq, H))
    Ws = [rng.standard_normal((H, H)) * 0.7 for _ in range(4)]
    ref = np.array(brute.attention_block(X.tolist(), *[w.tolist() for w in Ws], batch, seq, heads))
    assert np.max(np.abs(O.attention_block(X, *Ws, batch, seq, heads) - ref)) < 1e-12
    # two batches, two heads
    batch, seq, heads, d = 2, 4, 2, 3
    H = heads * d
    X = rng.standard_normal((batch * seq, H))
    Ws = [rng.standard_normal((H, H)) * 0.7 for _ in range(4)]
    ref = np.array(brute.attention_block(X.tolist(), *[w.tolist() for w in Ws], batch, seq, heads))
    assert np.max(np.abs(O.attention_block(X, *Ws, batch, seq, heads) - ref)) < 1e-12


# ---------------------------------------------------------------- attention closed forms
def test_attention_first_row_is_first_value():
    rng = np.random.default_rng(8)
    batch, seq, heads, d = 2, 6, 3, 4
    Q, K, V = (rng.standard_normal((batch * seq, heads * d)) for _ in range(3))
    Oa = O.causal_attention(Q, K, V, batch, seq, heads)
    for b in range(batch):
        assert np.array_equal(Oa[b * seq], V[b * seq])


def test_attention_zero_query_is_prefix_mean():
    rng = np.random.default_rng(9)
    batch, seq, heads, d = 2, 7, 2, 3
    Q = np.zeros((batch * seq, heads * d))
    K, V = (rng.standard_normal((batch * seq, heads * d)) for _ in range(2))
    Oa = O.causal_attention(Q, K, V, batch, seq, heads)
    for b in range(batch):
        for t in range(seq):
            ref = V[b * seq:b * seq + t + 1].mean(axis=0)
            assert np.max(np.abs(Oa[b * seq + t] - ref)) < 1e-14


def test_attention_scale_is_inverse_sqrt_head_dim():
    """Two keys with scores 0 and ln 3 after scaling by 1/sqrt(4) = 1/2:
    weights 1/4 and 3/4."""
    d = 4
    Q = np.zeros((2, d)); Q[1, 0] = 2.0 * math.log(3.0)
    K = np.zeros((2, d)); K[1, 0] = 1.0
    V = np.array([[1.0, 2.0, 3.0, 4.0], [-4.0, 0.0, 8.0, 2.0]])
    Oa = O.causal_attention(Q, K, V, 1, 2, 1)
    assert np.array_equal(Oa[0], V[0])
    assert np.max(np.abs(Oa[1] - np.array([-2.75, 0.5, 6.75, 2.5]))) < 1e-14


def test_attention_heads_are_independent_column_blocks():
    """Attention over h heads == attention on each head's columns alone."""
    rng = np.random.default_rng(10)
    batch, seq, heads, d = 2, 5, 4, 3
    Q, K, V = (rng.standard_normal((batch * seq, heads * d)) for _ in range(3))
    Oa = O.causal_attention(Q, K, V, batch, seq, heads)
    for h in range(heads):
        c = slice(h * d, (h + 1) * d)
        assert np.array_equal(Oa[:, c], O.causal_attention(Q[:, c], K[:, c], V[:, c], batch, seq, 1))


def test_sharded_attention_equals_unsharded():
    rng = np.random.default_rng(11)
    batch, seq, heads, d = 2, 6, 8, 2
    H = heads * d
    X = rng.standard_normal((batch * seq, H))
    Ws = [rng.standard_normal((H, H)) * 0.5 for _ in range(4)]
    bo = rng.standard_normal(H)
    Y = O.attention_block(X, *Ws, batch, seq, heads, bo=bo)
    for N in (1, 2, 4, 8):
        Ys = O.attention_block_sharded(X, *Ws, batch, seq, heads, N, bo=bo)
        assert np.max(np.abs(Ys - Y)) < 1e-12


def test_attention_rows_equals_full():
    rng = np.random.default_rng(12)
    batch, seq, heads, d = 2, 9, 2, 4
    H = heads * d
    X = rng.standard_normal((batch * seq, H))
    Ws = [rng.standard_normal((H, H)) * 0.5 for _ in range(4)]
    Y = O.attention_block(X, *Ws, batch, seq, heads)
    rows = np.array([0, 3, 8, 9, 10, 17])
    Yr = O.attention_block_rows(X, *Ws, batch, seq, heads, rows)
    assert np.max(np.abs(Yr - Y[rows])) < 1e-13


# ---------------------------------------------------------------- reduction / RS
def test_reduce_is_left_fold_in_shard_order():
    """fp32: (1e8 + 1) rounds to 1e8, so the left fold ((1e8 + 1) + -1e8) is 0,
    while the other order (1e8 + -1e8) + 1 would give 1."""
    p = [np.full((1, 1), 1e8, np.float32), np.full((1, 1), 1.0, np.float32),
         np.full((1, 1), -1e8, np.float32)]
    assert O.reduce_partials_fp32(p, out="f32")[0, 0] == 0.0
    assert O.reduce_partials_fp32([p[0], p[2], p[1]], out="f32")[0, 0] == 1.0


def test_reduce_exact_on_integer_partials_and_bias_once():
    rng = np.random.default_rng(13)
    parts = [rng.integers(-1000, 1000, size=(6, 5)).astype(np.float32) for _ in range(4)]
    bias = rng.integers(-50, 50, size=5).astype(np.float32)
    ref = sum(p.astype(np.int64) for p in parts) + bias.astype(np.int64)
    assert np.array_equal(O.reduce_partials_fp32(parts, bias, out="f32"), ref.astype(np.float32))


def test_bf16_rounding_hand_cases(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "bf16_rne_cases.json")))["cases"]
    bits = np.array([int(c[0], 16) for c in cases], dtype=np.uint32)
    want = np.array([int(c[1], 16) for c in cases], dtype=np.uint16)
    got = O.to_bf16(bits.view(np.float32).reshape(1, -1)).reshape(-1)
    assert np.array_equal(got, want), [(c, hex(g)) for c, g in zip(cases, got)]


def test_rs_slices_concatenate_to_full():
    rng = np.random.default_rng(14)
    parts = [rng.standard_normal((16, 3)).astype(np.float32) for _ in range(3)]
    bias = rng.standard_normal(3).astype(np.float32)
    full = O.reduce_partials_fp32(parts, bias, out="bf16")
    sl = [O.reduce_partials_fp32(parts, bias, out="bf16", n_slices=4, slice_=r) for r in range(4)]
    assert np.array_equal(np.concatenate(sl, axis=0), full)
    with pytest.raises(ValueError):
        O.rs_slice(full, 5, 0)


def test_divisibility_is_enforced():
    with pytest.raises(ValueError):
        O.column_shards(np.zeros((4, 10)), 4)
    with pytest.raises(ValueError):
        O.row_shards(np.zeros((10, 4)), 4)
    with pytest.raises(ValueError):
        O.attention_block_sharded(np.zeros((2, 6)), *[np.zeros((6, 6))] * 4, 1, 2, 6, 4)


# ------------------------------------------------- sequence-parallel entry side
def test_rmsnorm_hand_worked(golden_dir):
    """RMSNorm values worked by hand (tests/golden/rmsnorm_hand_worked.json)."""
    with open(os.path.join(golden_dir, "rmsnorm_hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        y = O.rmsnorm(np.array([c["x"]]), np.array(c["g"]), c["eps"])[0]
        assert np.allclose(y, c["y"], rtol=1e-14, atol=1e-15), c["work"]


def test_rmsnorm_invariants():
    """eps = 0, unit gain: every output row has mean square 1; the norm is
    odd and invariant to positive scaling of a row; a constant row maps to
    its sign times the gain."""
    rng = np.random.default_rng(11)
    X = rng.normal(size=(9, 24))
    one = np.ones(24)
    Y = O.rmsnorm(X, one, 0.0)
    assert np.allclose(np.mean(Y * Y, axis=1), 1.0, rtol=1e-14)
    assert np.allclose(O.rmsnorm(-X, one, 0.0), -Y, rtol=0, atol=1e-15)
    alpha = rng.uniform(0.1, 10.0, size=(9, 1))
    assert np.allclose(O.rmsnorm(alpha * X, one, 0.0), Y, rtol=1e-14)
    g = rng.normal(size=24)
    C = np.full((3, 24), -2.5)
    assert np.allclose(O.rmsnorm(C, g, 0.0), -g[None, :] * np.ones((3, 1)), rtol=1e-15)


def test_rmsnorm_matches_brute_force():
    rng = np.random.default_rng(12)
    X = rng.normal(size=(5, 7))
    g = rng.normal(size=7)
    ref = brute.rmsnorm(X.tolist(), g.tolist(), 1e-3)
    assert np.allclose(O.rmsnorm(X, g, 1e-3), ref, rtol=1e-13)


def test_sp_entry_equals_full_norm_bitwise():
    """Normalizing each sequence slice and gathering the slices gives the
    norm of the full tensor (the sequence split is exact for a row-wise op,
    blog post section 4.3); the gather keeps rank order."""
    rng = np.random.default_rng(13)
    X = rng.normal(size=(24, 16))
    g = rng.normal(size=16)
    full = O.rmsnorm(X, g, 1e-5)
    for n in (1, 2, 3, 4, 8):
        assert np.array_equal(O.sp_entry(X, g, 1e-5, n), full)
        sl = O.seq_slices(X, n)
        assert np.array_equal(O.all_gather_rows(sl), X)
        assert all(s.shape == (24 // n, 16) for s in sl)
    with pytest.raises(ValueError):
        O.sp_entry(X, g, 1e-5, 5)


def test_rmsnorm_hidden_split_equals_unsplit():
    """Blog post section 3.3: local sums of squares, one small reduction of the
    statistic, local scaling -- the parts concatenate to the unsplit norm.
    On integer inputs the statistic is exact, so the match is to rounding of
    the final products only."""
    rng = np.random.default_rng(14)
    X = _ints(rng, (6, 32))
    g = _ints(rng, (32,))
    full = O.rmsnorm(X, g, 0.5)
    for N in (1, 2, 4, 8):
        parts = O.rmsnorm_hidden_split(np.split(X, N, axis=1), np.split(g, N), 0.5)
        assert np.allclose(np.concatenate(parts, axis=1), full, rtol=1e-15, atol=0)


# ------------------------------------------------- LayerNorm and the hidden-split norms
def test_layernorm_hand_worked(golden_dir):
    """LayerNorm values worked by hand (tests/golden/layernorm_hand_worked.json)."""
    with open(os.path.join(golden_dir, "layernorm_hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        y = O.layernorm(np.array([c["x"]]), np.array(c["g"]), np.array(c["b"]), c["eps"])[0]
        assert np.allclose(y, c["y"], rtol=1e-14, atol=1e-15), c["work"]


def test_layernorm_invariants():
    """eps = 0, unit gain, no shift: every output row has mean 0 and mean
    square 1; the norm is invariant to adding a constant to a row and to
    positive scaling; negating a row negates the output; b shifts it."""
    rng = np.random.default_rng(21)
    X = rng.normal(size=(9, 24)) * 3.0 + 7.0
    one = np.ones(24)
    Y = O.layernorm(X, one, None, 0.0)
    assert np.allclose(np.mean(Y, axis=1), 0.0, atol=1e-14)
    assert np.allclose(np.mean(Y * Y, axis=1), 1.0, rtol=1e-13)
    shift = rng.normal(size=(9, 1)) * 100.0
    assert np.allclose(O.layernorm(X + shift, one, None, 0.0), Y, atol=1e-11)
    alpha = rng.uniform(0.1, 10.0, size=(9, 1))
    assert np.allclose(O.layernorm(alpha * X, one, None, 0.0), Y, atol=1e-12)
    assert np.allclose(O.layernorm(-X, one, None, 0.0), -Y, atol=1e-14)
    b = rng.normal(size=24)
    assert np.allclose(O.layernorm(X, one, b, 0.0), Y + b[None, :], atol=1e-14)
    # eps only rescales: mean square var / (var + eps)
    var = np.var(X, axis=1)
    Ye = O.layernorm(X, one, None, 2.0)
    assert np.allclose(np.mean(Ye * Ye, axis=1), var / (var + 2.0), rtol=1e-13)


def test_layernorm_matches_brute_force():
    rng = np.random.default_rng(22)
    X = rng.normal(size=(5, 7)) + 3.0
    g, b = rng.normal(size=7), rng.normal(size=7)
    ref = brute.layernorm(X.tolist(), g.tolist(), b.tolist(), 1e-3)
    assert np.allclose(O.layernorm(X, g, b, 1e-3), ref, rtol=1e-13, atol=1e-14)


def test_merge_moments_is_the_statistic_of_the_union():
    """The pairwise update gives the count, mean and sum of squared
    deviations of the concatenation, for unequal parts and any split point."""
    rng = np.random.default_rng(23)
    x = rng.normal(size=37) * 4.0 + 10.0
    for cut in (1, 5, 18, 36):
        a, b = x[:cut], x[cut:]
        n, m, q = O.merge_moments((len(a), a.mean(), np.sum((a - a.mean()) ** 2)),
                                  (len(b), b.mean(), np.sum((b - b.mean()) ** 2)))
        assert n == len(x)
        assert np.isclose(m, x.mean(), rtol=1e-14)
        assert np.isclose(q, np.sum((x - x.mean()) ** 2), rtol=1e-12)
    # on small integers every quantity is exact: the merge of [1, 2] and [4, 7]
    n, m, q = O.merge_moments((2, 1.5, 0.5), (2, 5.5, 4.5))
    assert (n, m, q) == (4, 3.5, 21.0)  # mean 14/4; deviations -2.5, -1.5, 0.5, 3.5 -> 6.25+2.25+0.25+12.25


def test_sp_entry_layernorm_equals_full_norm_bitwise():
    rng = np.random.default_rng(24)
    X = rng.normal(size=(24, 16))
    g, b = rng.normal(size=16), rng.normal(size=16)
    full = O.layernorm(X, g, b, 1e-5)
    for n in (1, 2, 3, 4, 8):
        assert np.array_equal(O.sp_entry_layernorm(X, g, b, 1e-5, n), full)


def test_layernorm_hidden_split_equals_unsplit():
    """Blog post section 3.3: local statistics, one small reduction of them,
    local normalization -- the parts concatenate to the unsplit norm, for
    equal and unequal parts, with and without a shift."""
    rng = np.random.default_rng(25)
    X = rng.normal(size=(6, 48)) * 2.0 + 5.0
    g, b = rng.normal(size=48), rng.normal(size=48)
    full = O.layernorm(X, g, b, 0.25)
    for N in (1, 2, 3, 4, 8):
        parts = O.layernorm_hidden_split(np.split(X, N, axis=1), np.split(g, N), np.split(b, N), 0.25)
        assert np.allclose(np.concatenate(parts, axis=1), full, rtol=0, atol=1e-13)
    cuts = [5, 17, 40]
    parts = O.layernorm_hidden_split(np.split(X, cuts, axis=1), np.split(g, cuts), None, 0.25)
    assert np.allclose(np.concatenate(parts, axis=1), O.layernorm(X, g, None, 0.25), rtol=0, atol=1e-13)


def test_planted_hidden_split_norm_mistakes():
    """What the split norm must not do: normalize each part with its own
    statistics (the mistake the blog post warns of in section 3.3), merge
    without the deviation-of-means term, or sum squares about each part's
    own mean and forget the parts' spread."""
    rng = np.random.default_rng(26)
    X = rng.normal(size=(4, 32))
    X[:, 16:] += 3.0  # the two halves have different means
    g, b = np.ones(32), np.zeros(32)
    want = O.layernorm(X, g, b, 1e-6)
    Xp = np.split(X, 2, axis=1)
    local = np.concatenate([O.layernorm(x, np.ones(16), None, 1e-6) for x in Xp], axis=1)
    assert np.max(np.abs(local - want)) > 0.5

    saved = O.merge_moments

    def no_spread(a, c):  # drops the d^2 n_a n_b / n term
        n, m, q = saved(a, c)
        d = c[1] - a[1]
        return n, m, q - d * d * (a[0] * c[0] / n)

    try:
        O.merge_moments = no_spread
        wrong = np.concatenate(O.layernorm_hidden_split(Xp, [np.ones(16)] * 2, None, 1e-6), axis=1)
    finally:
        O.merge_moments = saved
    assert np.max(np.abs(wrong - want)) > 0.5
    right = np.concatenate(O.layernorm_hidden_split(Xp, [np.ones(16)] * 2, None, 1e-6), axis=1)
    assert np.allclose(right, want, atol=1e-13)
