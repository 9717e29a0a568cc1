"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch each one.  A pin that a mistake slips through is not pinning anything.
"""
import math

import numpy as np
import pytest

import oracle.tp_oracle as T
from tests import test_oracle_pins as pins


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_tanh_gelu_is_caught(monkeypatch, golden_dir):
    def tanh_gelu(z):
        z = np.asarray(z, dtype=np.float64)
        return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    monkeypatch.setattr(T, "gelu", tanh_gelu)
    _fails(pins.test_gelu_textbook_values, golden_dir)


def test_bias_added_per_shard_is_caught(monkeypatch):
    def bad(X, A, a, B, b, N):
        Hs = [T.gelu(z) for z in T.column_linear_sharded(X, A, a, N)]
        P = T.row_partials(Hs, B, N)
        if b is not None:
            P = [p + np.asarray(b)[None, :] for p in P]   # bias on every shard
        return T._fold(P)
    monkeypatch.setattr(T, "mlp_gelu_sharded", bad)
    _fails(pins.test_I4_bias_counted_once)
    _fails(pins.test_I3_sharded_gelu_mlp_equals_unsharded)


def test_dropped_column_bias_is_caught(monkeypatch):
    orig = T.linear

    def no_bias(X, W, bias=None):
        return orig(X, W)
    monkeypatch.setattr(T, "linear", no_bias)
    _fails(pins.test_I1_column_concat_is_full_product_bitwise)


def test_wrong_row_block_is_caught(monkeypatch):
    orig = T.row_shards

    def reversed_shards(W, N):
        return orig(W, N)[::-1]
    monkeypatch.setattr(T, "row_shards", reversed_shards)
    _fails(pins.test_I2_row_partials_sum_to_full_product_bitwise)


def _attn_variant(scale_fn=None, keep_diag=True, transpose_v=False):
    def attn(Q, K, V, batch, seq, heads):
        Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
        d = Q.shape[1] // heads
        out = np.empty_like(Q)
        k = 1 if keep_diag else 0
        mask = np.triu(np.ones((seq, seq), dtype=bool), k=k)
        scale = scale_fn(d) if scale_fn else 1 / math.sqrt(d)
        for b in range(batch):
            r = slice(b * seq, (b + 1) * seq)
            for h in range(heads):
                c = slice(h * d, (h + 1) * d)
                S = Q[r, c] @ K[r, c].T * scale
                S[mask] = -np.inf
                S -= np.nanmax(np.where(np.isinf(S), np.nan, S), axis=1, keepdims=True) if not keep_diag else S.max(1, keepdims=True)
                P = np.exp(S)
                P /= P.sum(1, keepdims=True)
                out[r, c] = P @ V[r, c]
        return out
    return attn


def test_attention_scale_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(T, "causal_attention", _attn_variant(scale_fn=lambda d: 1.0 / d))
    _fails(pins.test_attention_scale_is_inverse_sqrt_head_dim)


def test_attention_mask_without_diagonal_is_caught(monkeypatch):
    monkeypatch.setattr(T, "causal_attention", _attn_variant(keep_diag=False))
    with np.errstate(all="ignore"):
        _fails(pins.test_attention_first_row_is_first_value)


def test_reduce_pairwise_order_is_caught(monkeypatch):
    def tree(parts, bias=None, out="f32", n_slices=1, slice_=-1):
        ps = [np.asarray(p, np.float32) for p in parts]
        while len(ps) > 1:
            nxt = [ps[i] + ps[i + 1] for i in range(0, len(ps) - 1, 2)]
            if len(ps) % 2:
                nxt.append(ps[-1])
            ps = nxt
        acc = ps[0]
        if bias is not None:
            acc = acc + np.asarray(bias, np.float32)[None, :]
        return acc
    # (1e8 + -1e8) is formed first by a reversed pairing; emulate a reversed-order fold
    def reversed_fold(parts, bias=None, out="f32", n_slices=1, slice_=-1):
        return tree(list(parts)[::-1], bias, out, n_slices, slice_)
    monkeypatch.setattr(T, "reduce_partials_fp32", reversed_fold)
    _fails(pins.test_reduce_is_left_fold_in_shard_order)


def test_naive_swiglu_split_is_caught(monkeypatch):
    def naive(Wg, Wu, N):
        full = np.concatenate([np.asarray(Wg, float), np.asarray(Wu, float)], axis=1)
        return T.column_shards(full, N)
    monkeypatch.setattr(T, "swiglu_fused_blocks", naive)
    _fails(pins.test_swiglu_fused_block_layout)


def test_local_statistic_rmsnorm_is_caught(monkeypatch):
    """The mistake the blog post (section 3.3) warns about: each hidden part
    normalized with its own local statistic instead of the reduced one."""
    def local_only(X_parts, g_parts, eps):
        return [T.rmsnorm(x, gp, eps) for x, gp in zip(X_parts, g_parts)]
    monkeypatch.setattr(T, "rmsnorm_hidden_split", local_only)
    _fails(pins.test_rmsnorm_hidden_split_equals_unsplit)


def test_rmsnorm_mean_abs_instead_of_mean_square_is_caught(monkeypatch):
    def bad(X, g, eps):
        X = np.asarray(X, dtype=np.float64)
        return X / (np.mean(np.abs(X), axis=-1, keepdims=True) + eps) * np.asarray(g)[None, :]
    monkeypatch.setattr(T, "rmsnorm", bad)
    _fails(pins.test_rmsnorm_invariants)


def test_rmsnorm_eps_outside_sqrt_is_caught(monkeypatch, golden_dir):
    def bad(X, g, eps):
        X = np.asarray(X, dtype=np.float64)
        return X / (np.sqrt(np.mean(X * X, axis=-1, keepdims=True)) + eps) * np.asarray(g)[None, :]
    monkeypatch.setattr(T, "rmsnorm", bad)
    _fails(pins.test_rmsnorm_hand_worked, golden_dir)


def test_sp_gather_out_of_rank_order_is_caught(monkeypatch):
    def bad(slices):
        return np.concatenate([np.asarray(s, dtype=np.float64) for s in slices[::-1]], axis=0)
    monkeypatch.setattr(T, "all_gather_rows", bad)
    _fails(pins.test_sp_entry_equals_full_norm_bitwise)
