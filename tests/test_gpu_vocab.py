"""Vocab-parallel output head and cross-entropy: HIP path vs the fp64 CPU
oracle, through the C ABI (gfx950 GPU required).

The loss is computed in fp32 from bf16 inputs (fp32 logits, fp32 statistics),
so it is held to the fp32 bound: max|loss - O| / max|O| <= 1e-4, and must be
bit-identical run to run.
"""
import math
import sys

import numpy as np
import pytest

from oracle import reference as R
from oracle import tp_oracle as O
from tensor_transformer_layers_amd import configs, inputs, tp, workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

DEV = "cuda"
TOL = 1e-4


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def _case(T, H, V, N, seed, pad_value=0.0):
    rng = np.random.default_rng(seed)
    Vp = tp.tp_vocab_padded(V, N)
    X = inputs.round_to_dtype(rng.standard_normal((T, H)).astype(np.float32), "bf16")
    E = np.full((Vp, H), pad_value, dtype=np.float32)
    E[:V] = inputs.round_to_dtype((rng.standard_normal((V, H)) * 0.05).astype(np.float32), "bf16")
    labels = rng.integers(0, V, T).astype(np.int32)
    return X, E, labels


def _dev(X, E, labels):
    return (torch.from_numpy(X).to(DEV, torch.bfloat16), torch.from_numpy(E).to(DEV, torch.bfloat16),
            torch.from_numpy(labels).to(DEV))


@pytest.mark.parametrize("T,H,V,N", [
    (100, 64, 1000, 8),
    (257, 136, 37, 4),      # the last shard holds only padding
    (64, 64, 9, 8),         # six shards hold only padding
    (1000, 512, 50257, 8),
    (300, 256, 4096, 1),
    (1, 64, 3, 8),          # one token, V < N: seven shards hold only padding
])
def test_vocab_ce_vs_oracle(T, H, V, N):
    say(f"vocab_ce T={T} H={H} V={V} N={N}")
    X, E, labels = _case(T, H, V, N, seed=T + H + V + N)
    Xd, Ed, Ld = _dev(X, E, labels)
    loss, mean, _ = tp.vocab_ce_forward(Xd, Ed, Ld, V, N)
    loss2, mean2, _ = tp.vocab_ce_forward(Xd, Ed, Ld, V, N)
    torch.cuda.synchronize()
    ref = O.lm_head_ce(X, E, labels, V)
    e = err(loss.cpu().numpy(), ref)
    say(f"  loss err={e:.3e}")
    assert e <= TOL
    assert abs(mean.item() - ref.mean()) <= TOL * np.max(np.abs(ref))
    assert torch.equal(loss, loss2) and torch.equal(mean, mean2), "not bit-identical run to run"


def test_padding_rows_do_not_reach_the_loss():
    T, H, V, N = 128, 64, 1003, 8
    X, E0, labels = _case(T, H, V, N, seed=5)
    _, E7, _ = _case(T, H, V, N, seed=5, pad_value=7.0)
    a, _, _ = tp.vocab_ce_forward(*_dev(X, E0, labels), V, N)
    b, _, _ = tp.vocab_ce_forward(*_dev(X, E7, labels), V, N)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_uniform_logits_give_log_vocab():
    T, H, V, N = 64, 64, 777, 4
    X, E, labels = _case(T, H, V, N, seed=6)
    E[:] = 0.0
    loss, mean, _ = tp.vocab_ce_forward(*_dev(X, E, labels), V, N)
    torch.cuda.synchronize()
    assert np.max(np.abs(loss.cpu().numpy() - math.log(V))) <= 1e-5 * math.log(V)


def test_one_shard_range_statistics():
    T, H, V, N, r = 200, 128, 1000, 8, 3
    X, E, labels = _case(T, H, V, N, seed=7)
    Xd, Ed, Ld = _dev(X, E, labels)
    loss, mean, ws = tp.vocab_ce_forward(Xd, Ed, Ld, V, N, shard_begin=r, shard_count=1)
    torch.cuda.synchronize()
    assert loss is None and mean is None
    Vs = tp.tp_vocab_padded(V, N) // N
    m, s, z = (a[r].cpu().numpy() for a in tp.vocab_ce_stats(ws, N, T, Vs, 1))
    _, (ms, ss, zs) = O.vocab_parallel_ce(X, E, labels, V, N)
    assert err(m, ms[r]) <= TOL and err(s, ss[r]) <= TOL
    owned = zs[r] != 0
    assert owned.any() and np.array_equal(z == 0, ~owned)
    assert err(z[owned], zs[r][owned]) <= TOL


def test_empty_tokens_is_noop():
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    E = torch.zeros((tp.tp_vocab_padded(100, 2), 64), dtype=torch.bfloat16, device=DEV)
    L = torch.empty((0,), dtype=torch.int32, device=DEV)
    loss, mean, ws = tp.vocab_ce_forward(X, E, L, 100, 2)
    torch.cuda.synchronize()
    assert ws is None and loss.shape == (0,)


def test_vocab_ce_full_size():
    """The 150k-vocab head at 8 x 2048 tokens, hidden 4096, 8 shards, on
    sampled token rows (the loss is token-wise)."""
    w = configs.workload(6)
    say(f"vocab config {w.name}: generating inputs")
    host = inputs.make_inputs(w)
    d = workloads.device_inputs(w, host)
    say("vocab config: all 8 shards")
    loss, _ = workloads.forward(w, d)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(w.T, 64, w.seed, [0, w.T - 1])
    say(f"vocab config: oracle on {len(rows)} rows")
    ref = R.workload("vocab_ce", host, rows=rows)
    got = loss[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    e = err(got, ref)
    say(f"vocab config: loss err={e:.3e}")
    assert e <= TOL


def test_labels_at_an_element_offset():
    """labels need only int32 alignment: a view starting one element in."""
    T, H, V, N = 130, 64, 1000, 4
    X, E, labels = _case(T, H, V, N, seed=17)
    Xd, Ed, _ = _dev(X, E, labels)
    Lbig = torch.from_numpy(np.concatenate([[0], labels]).astype(np.int32)).to(DEV)
    view = Lbig[1:]
    assert view.data_ptr() % 16 == 4
    loss, _, _ = tp.vocab_ce_forward(Xd, Ed, view, V, N)
    torch.cuda.synchronize()
    ref = O.lm_head_ce(X, E, labels, V)
    assert err(loss.cpu().numpy(), ref) <= TOL
