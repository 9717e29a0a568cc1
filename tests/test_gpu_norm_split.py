"""LayerNorm on sequence slices, the hidden-split norms (RMSNorm and
LayerNorm) and the sequence-parallel backward's reduce-scatter of dX, on the
GPU vs the fp64 oracle, through the C ABI (gfx950 GPU required).

Tolerances, elementwise against the oracle's fp64 value (the norms are
elementwise after a few row statistics).  bf16 output: one round-to-nearest-
even step, under 2^-8 relative; fp32 output: 1e-5 relative.  The statistics
are fp32 sums of H terms, whose error is at most H * 2^-24 of the sum of the
terms' magnitudes (the standard bound for recursive summation); through the
mean and the scale it reaches every output as an absolute error below
4 H 2^-24 of the largest output, the floor added to the relative bound.
"""
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


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def _draw(seed, shape, sigma, dt, mean=0.0):
    ss = np.random.SeedSequence(seed)
    x = inputs.draw(ss, shape, sigma) + np.float32(mean)
    return inputs.round_to_dtype(x.astype(np.float32), dt)


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV, _tdt(dt))


def _check(y_dev, ref, dt, H):
    y = y_dev.float().cpu().numpy().astype(np.float64)
    rel = 2.0 ** -8 if dt == "bf16" else 1e-5
    floor = 4.0 * H * 2.0 ** -24 * float(np.max(np.abs(ref)))
    bad = np.abs(y - ref) > rel * np.abs(ref) + floor
    assert not bad.any(), f"{int(bad.sum())} elements off, worst |d| = {float(np.max(np.abs(y - ref))):.3e}"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


# ------------------------------------------------------------ LayerNorm on sequence slices
@pytest.mark.parametrize("dt,n,T,H,eps,sl,beta", [
    ("bf16", 4, 64, 512, 1e-5, -1, True),
    ("bf16", 8, 96, 12288, 1e-5, -1, True),    # the 175B-shaped hidden size: rows split over 8 waves
    ("bf16", 2, 10, 8, 1e-5, -1, False),       # one 16-byte piece
    ("bf16", 3, 33, 520, 1e-6, 1, True),       # ragged hidden (a partial piece), one slice only
    ("bf16", 1, 7, 16384, 1e-5, -1, True),     # largest hidden
    ("f32", 2, 128, 512, 1e-5, -1, True),
    ("f32", 4, 20, 8192, 0.0, -1, False),      # largest fp32 hidden, eps = 0
])
def test_layernorm_gather_vs_oracle(dt, n, T, H, eps, sl, beta):
    say(f"layernorm_gather dt={dt} n={n} T={T} H={H} eps={eps} slice={sl} beta={beta}")
    seed = 8000 + T + H + n
    X = _draw(seed, (T, H), 2.0, dt, mean=3.0)   # a mean far from 0: the deviations must be taken about it
    g = inputs.round_to_dtype((1.0 + _draw(seed + 1, (H,), 0.1, "f32")).astype(np.float32), dt)
    b = _draw(seed + 2, (H,), 0.1, dt) if beta else None
    Y = torch.full((T, H), 7.0, dtype=_tdt(dt), device=DEV)
    tp.layernorm_gather(_dev(X, dt), _dev(g, dt), None if b is None else _dev(b, dt), eps, n, out=Y, slice=sl)
    Y2 = tp.layernorm_gather(_dev(X, dt), _dev(g, dt), None if b is None else _dev(b, dt), eps, n)
    torch.cuda.synchronize()
    ref = O.sp_entry_layernorm(X, g, b, eps, n)
    per = T // n
    rows = slice(None) if sl < 0 else slice(sl * per, (sl + 1) * per)
    _check(Y[rows], ref[rows], dt, H)
    assert torch.equal(_bits(Y[rows]), _bits(Y2[rows])), "one slice differs from the same rows of the full call"
    if sl >= 0:
        rest = torch.ones(T, dtype=torch.bool, device=DEV)
        rest[rows] = False
        assert bool((Y[rest] == 7.0).all()), "rows outside the slice were written"


# ------------------------------------------------------------ hidden-split norms
SPLIT = [
    ("bf16", "layer", 64, 4096, 8, True),
    ("bf16", "rms", 64, 4096, 8, False),
    ("bf16", "layer", 40, 12288, 8, True),    # the 175B-shaped hidden size, 1536 per shard
    ("bf16", "layer", 9, 64, 8, False),       # 8 features per shard: one piece, most lanes idle
    ("bf16", "layer", 16, 16384 * 2, 2, True),  # the widest shard (16384): 8 waves per slice
    ("bf16", "rms", 33, 520, 5, False),       # an odd shard count
    ("bf16", "rms", 24, 4096, 2, False),      # 2048 per shard: four 1 KB pieces per lane in the scale pass
    ("bf16", "layer", 12, 1152, 9, True),     # more than 8 shards: the statistics folded in a loop
    ("f32", "layer", 50, 2048, 4, True),
    ("f32", "rms", 50, 2048, 1, False),
]


def _split_case(dt, kind, T, H, N, beta, seed):
    X = _draw(seed, (T, H), 1.5, dt)
    # each shard's features get a different offset: the shards' means differ,
    # so the merge's spread term matters
    X = inputs.round_to_dtype((X + np.repeat(np.arange(N, dtype=np.float32) * 0.75, H // N)[None, :]).astype(np.float32), dt)
    g = inputs.round_to_dtype((1.0 + _draw(seed + 1, (H,), 0.1, "f32")).astype(np.float32), dt)
    b = _draw(seed + 2, (H,), 0.1, dt) if beta else None
    return X, g, b


def _split_ref(X, g, b, eps, N, kind):
    parts = np.split(X.astype(np.float64), N, axis=1)
    gp = np.split(g.astype(np.float64), N)
    if kind == "layer":
        bp = None if b is None else np.split(b.astype(np.float64), N)
        return np.concatenate(O.layernorm_hidden_split(parts, gp, bp, eps), axis=1)
    return np.concatenate(O.rmsnorm_hidden_split(parts, gp, eps), axis=1)


@pytest.mark.parametrize("dt,kind,T,H,N,beta", SPLIT)
def test_norm_hidden_split_vs_oracle(dt, kind, T, H, N, beta):
    say(f"norm_hidden_split dt={dt} kind={kind} T={T} H={H} N={N} beta={beta}")
    X, g, b = _split_case(dt, kind, T, H, N, beta, seed=8100 + T + H + N)
    eps = 1e-5
    k = tp.TP_NORM_LAYER if kind == "layer" else tp.TP_NORM_RMS
    Y, ws = tp.norm_hidden_split(_dev(X, dt), _dev(g, dt), None if b is None else _dev(b, dt), eps, N, kind=k)
    Y2, _ = tp.norm_hidden_split(_dev(X, dt), _dev(g, dt), None if b is None else _dev(b, dt), eps, N, kind=k)
    torch.cuda.synchronize()
    ref = _split_ref(X, g, b, eps, N, kind)
    _check(Y, ref, dt, H)
    # the unsplit norm is the same function (blog post 3.3): both oracles agree
    full = O.layernorm(X, g, b, eps) if kind == "layer" else O.rmsnorm(X, g, eps)
    assert np.allclose(ref, full, rtol=0, atol=1e-12 * np.max(np.abs(full)))
    assert torch.equal(_bits(Y), _bits(Y2)), "not bit-identical run to run"
    # each shard's local statistic in the slab, against the oracle's
    st = tp.norm_split_stats(ws, N, T).cpu().numpy().astype(np.float64)
    Hs = H // N
    for i in range(N):
        part = X[:, i * Hs:(i + 1) * Hs].astype(np.float64)
        if kind == "layer":
            m = part.mean(axis=1)
            q = np.sum((part - m[:, None]) ** 2, axis=1)
            assert np.allclose(st[i, :, 0], m, rtol=1e-5, atol=4 * Hs * 2.0 ** -24 * np.max(np.abs(part)))
            assert np.allclose(st[i, :, 1], q, rtol=1e-4, atol=1e-6 * np.max(q))
        else:
            assert np.allclose(st[i, :, 0], np.sum(part * part, axis=1), rtol=1e-5)


@pytest.mark.parametrize("kind", ["layer", "rms"])
def test_norm_hidden_split_one_rank_share(kind):
    """Rank r alone: its own statistic into its slot of a slab holding the
    others' (left by an earlier call), the fold, and its own columns only --
    bit-identical to those columns of the all-shards call."""
    T, H, N, dt = 48, 2048, 8, "bf16"
    X, g, b = _split_case(dt, kind, T, H, N, kind == "layer", seed=8200)
    k = tp.TP_NORM_LAYER if kind == "layer" else tp.TP_NORM_RMS
    bd = None if b is None else _dev(b, dt)
    Y, ws = tp.norm_hidden_split(_dev(X, dt), _dev(g, dt), bd, 1e-5, N, kind=k)
    torch.cuda.synchronize()
    Hs = H // N
    for r in (0, 5, N - 1):
        Yr = torch.full((T, H), 7.0, dtype=torch.bfloat16, device=DEV)
        tp.norm_hidden_split(_dev(X, dt), _dev(g, dt), bd, 1e-5, N, kind=k, shard_begin=r, shard_count=1, out=Yr,
                             ws=ws)
        torch.cuda.synchronize()
        cols = slice(r * Hs, (r + 1) * Hs)
        assert torch.equal(_bits(Yr[:, cols]), _bits(Y[:, cols])), r
        rest = torch.ones(H, dtype=torch.bool, device=DEV)
        rest[cols] = False
        assert bool((Yr[:, rest] == 7.0).all()), "columns of other shards were written"


@pytest.mark.parametrize("kind,dt", [("layer", "bf16"), ("rms", "bf16"), ("layer", "f32")])
def test_norm_hidden_split_one_shard_equals_gather(kind, dt):
    """With N = 1 the split norm is the whole-row norm: the same sums in the
    same order, so the same bits as the sequence-slice kernel."""
    T, H = 24, 4096
    X, g, b = _split_case(dt, kind, T, H, 1, kind == "layer", seed=8300)
    k = tp.TP_NORM_LAYER if kind == "layer" else tp.TP_NORM_RMS
    bd = None if b is None else _dev(b, dt)
    Ys, _ = tp.norm_hidden_split(_dev(X, dt), _dev(g, dt), bd, 1e-5, 1, kind=k)
    Yg = (tp.layernorm_gather(_dev(X, dt), _dev(g, dt), bd, 1e-5, 1) if kind == "layer"
          else tp.rmsnorm_gather(_dev(X, dt), _dev(g, dt), 1e-5, 1))
    torch.cuda.synchronize()
    assert torch.equal(_bits(Ys), _bits(Yg))


def test_norm_hidden_split_full_size_sampled():
    """The 175B-shaped layer's hidden size split over 8 shards at the full
    token count (T = 16384, H = 12288, 1536 features per shard), the launch
    bench.py --config 8 times; sampled rows checked one by one."""
    w = configs.workload(8)
    say(f"hidden-split norm full size: {w.name}")
    host = inputs.make_inputs(w)
    d = workloads.device_inputs(w, host)
    Y, ws = workloads.forward(w, d)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(w.T, 256, w.seed, must=[0, w.T - 1])
    ref = R.workload(w.kind, host, rows=rows, N=w.N)
    _check(Y[torch.from_numpy(rows).to(DEV)], ref, "bf16", w.H)


# ------------------------------------------------------------ sequence-parallel backward
@pytest.mark.parametrize("act", [tp.TP_ACT_GELU, tp.TP_ACT_SWIGLU])
def test_backward_dx_reduce_scatter_slices(act):
    """The SP layout of the backward: rank r's reduce-scatter slice of dX is
    bit-identical to rows r*T/n .. of the all-reduced dX, and all slices
    together equal it (the backward of the sequence all-gather)."""
    kind = "mlp_swiglu" if act == tp.TP_ACT_SWIGLU else "mlp_gelu"
    base = configs.CONFIGS[3] if kind == "mlp_swiglu" else configs.CONFIGS[5]
    w = configs.scaled(base, batch=4, seq=128, H=512, F=8 * 64, n_slices=4, seed=8400)
    say(f"backward dX reduce-scatter {kind}: T={w.T} H={w.H} slices={w.n_slices}")
    host = inputs.make_inputs(w)
    d = workloads.device_inputs(w, host)
    dY = workloads.to_device(inputs.grad_output(w), d["X"].dtype)
    g, ws = workloads.backward(w, d, dY)
    full = g["dX"].clone()
    per = w.T // w.n_slices
    parts = []
    for r in range(w.n_slices):
        gr, ws = tp.mlp_backward(d["X"], d["A"], d["a"], d["B"], dY, w.N, act=act, ws=ws, need_da=d["a"] is not None,
                                 need_db=d["b"] is not None, n_slices=w.n_slices, slice=r)
        parts.append(gr["dX"])
        assert gr["dX"].shape == (per, w.H)
    torch.cuda.synchronize()
    for r in range(w.n_slices):
        assert torch.equal(_bits(parts[r]), _bits(full[r * per:(r + 1) * per])), r
    assert torch.equal(_bits(torch.cat(parts)), _bits(full))
    # and the slices against the oracle's input gradient
    if kind == "mlp_gelu":
        ref = R.mlp_gelu_backward(host["X"], host["A"], host["a"], host["B"], inputs.grad_output(w))["dX"]
    else:
        ref = R.mlp_swiglu_backward(host["X"], host["Wg"], host["Wu"], host["Wd"], inputs.grad_output(w))["dX"]
    got = torch.cat(parts).float().cpu().numpy()
    e = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    assert e <= 2e-2, e
