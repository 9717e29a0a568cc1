"""Vocab-parallel embedding lookup (the input side of the vocab split): HIP
path vs the fp64 CPU oracle, through the C ABI (gfx950 GPU required).

Every output element is the fp32 fold, from -0.0, of N partials (in the
table's type) of which at most one is not -0.0, and that one is a table
entry, so the result must equal the oracle bit for bit (bf16 and fp32 tables,
signed zeros included: the comparisons are on bit patterns).
"""
import sys

import numpy as np
import pytest

from oracle import tp_oracle as O
from tensor_transformer_layers_amd import inputs, tp

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

DEV = "cuda"
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def _case(T, H, V, N, seed, dt, pad_value=np.nan):
    rng = np.random.default_rng(seed)
    Vp = tp.tp_vocab_padded(V, N)
    E = np.full((Vp, H), pad_value, dtype=np.float32)  # padding rows must never be read
    E[:V] = rng.standard_normal((V, H)).astype(np.float32)
    if dt == "bf16":
        E[:V] = inputs.round_to_dtype(E[:V], "bf16")
    # signed zeros in the real rows: the lookup must return their bits
    z = rng.random((V, H)) < 0.02
    E[:V][z] = np.where(rng.random(int(z.sum())) < 0.5, -0.0, 0.0).astype(np.float32)
    ids = rng.integers(0, V, T).astype(np.int32)
    return E, ids


def _bits(x):
    """float64 bit patterns: equal values with different signs of zero differ."""
    return np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)


def _dev(E, ids, dt):
    return torch.from_numpy(E).to(DEV, TDT[dt]), torch.from_numpy(ids).to(DEV)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,H,V,N", [
    (100, 64, 1000, 8),
    (257, 136, 37, 4),      # the last shard holds only padding
    (64, 520, 9, 8),        # six shards hold only padding; H not a multiple of 512
    (1000, 1024, 50257, 8),
    (300, 256, 4096, 1),
    (1, 8, 3, 8),           # one token, the smallest hidden size, V < N
    (5, 8, 1, 1),           # a one-entry vocab on one shard
])
def test_vocab_embed_vs_oracle(T, H, V, N, dt):
    say(f"vocab_embed dt={dt} T={T} H={H} V={V} N={N}")
    E, ids = _case(T, H, V, N, seed=T + H + V + N, dt=dt)
    Ed, Id = _dev(E, ids, dt)
    Y, _ = tp.vocab_embed_forward(Id, Ed, V, N)
    torch.cuda.synchronize()
    ref, _ = O.vocab_parallel_embedding(ids, E.astype(np.float64), V, N)
    got = Y.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(_bits(got), _bits(ref)), f"max diff {np.nanmax(np.abs(got - ref))}"
    assert np.signbit(got).sum() == np.signbit(ref).sum()


def test_out_of_range_ids_give_zero_rows():
    T, H, V, N = 64, 64, 1003, 8
    E, ids = _case(T, H, V, N, seed=3, dt="bf16")
    Vp = E.shape[0]
    ids[:6] = [-1, V, V + 3, Vp, Vp + 100, -(1 << 30)]
    Ed, Id = _dev(E, ids, "bf16")
    Y, _ = tp.vocab_embed_forward(Id, Ed, V, N)
    torch.cuda.synchronize()
    ref, _ = O.vocab_parallel_embedding(ids, E.astype(np.float64), V, N)
    got = Y.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(_bits(got), _bits(ref))
    assert not got[:6].any()


def test_one_shard_range_partials():
    """A shard range writes only its slots of the partial slab, each the
    oracle's masked lookup for that shard."""
    T, H, V, N = 200, 128, 1000, 8
    E, ids = _case(T, H, V, N, seed=11, dt="bf16")
    Ed, Id = _dev(E, ids, "bf16")
    _, ws = tp.vocab_embed_forward(Id, Ed, V, N)  # fills every slot
    parts = tp.vocab_embed_partials(ws, N, T, H, torch.bfloat16)
    parts.fill_(-5.0)
    Y, ws = tp.vocab_embed_forward(Id, Ed, V, N, shard_begin=2, shard_count=3, ws=ws)
    torch.cuda.synchronize()
    assert Y is None
    _, ref_parts = O.vocab_parallel_embedding(ids, E.astype(np.float64), V, N)
    got = parts.float().cpu().numpy().astype(np.float64)
    for i in range(N):
        if 2 <= i < 5:
            assert np.array_equal(_bits(got[i]), _bits(ref_parts[i])), i
        else:
            assert np.all(got[i] == -5.0), i


def test_empty_tokens_is_noop():
    E, _ = _case(1, 64, 100, 4, seed=1, dt="bf16")
    Ed = torch.from_numpy(E).to(DEV, torch.bfloat16)
    Y, ws = tp.vocab_embed_forward(torch.zeros(0, dtype=torch.int32, device=DEV), Ed, 100, 4)
    torch.cuda.synchronize()
    assert Y.shape == (0, 64) and ws is None


def test_vocab_embed_full_size():
    """The 150k-token vocab at H=4096, 16384 tokens, 8 shards: every output
    row checked against the table (the lookup is exact)."""
    T, H, V, N = 16384, 4096, 150000, 8
    say(f"vocab_embed full T={T} H={H} V={V} N={N}")
    g = torch.Generator(device=DEV).manual_seed(7)
    Vp = tp.tp_vocab_padded(V, N)
    Ed = torch.randn((Vp, H), device=DEV, generator=g).to(torch.bfloat16)
    Ed[V:] = float("nan")
    Id = torch.randint(0, V, (T,), device=DEV, generator=g, dtype=torch.int32)
    Y, ws = tp.vocab_embed_forward(Id, Ed, V, N)
    Y2, _ = tp.vocab_embed_forward(Id, Ed, V, N, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Ed[Id.long()].view(torch.int16))
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))
    # sampled tokens against the fp64 oracle on the CPU (the whole table,
    # so the shard ranges are the real ones)
    rows = np.random.default_rng(0).choice(T, 64, replace=False)
    E = Ed.float().cpu().numpy()
    ref, _ = O.vocab_parallel_embedding(Id.cpu().numpy()[rows], E, V, N)
    got = Y[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
    assert np.array_equal(_bits(got), _bits(ref))


def test_ids_at_an_element_offset():
    """ids need only int32 alignment: a view starting one element in."""
    T, H, V, N = 99, 128, 500, 4
    E, ids = _case(T + 1, H, V, N, seed=21, dt="bf16")
    Ed, Id = _dev(E, ids, "bf16")
    view = Id[1:]
    assert view.data_ptr() % 16 == 4
    Y, _ = tp.vocab_embed_forward(view, Ed, V, N)
    torch.cuda.synchronize()
    ref, _ = O.vocab_parallel_embedding(ids[1:], E.astype(np.float64), V, N)
    assert np.array_equal(_bits(Y.float().cpu().numpy()), _bits(ref))
