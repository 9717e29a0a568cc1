"""Backward of the MLP pair: HIP path vs the fp64 CPU oracle, through the C ABI
(gfx950 GPU required).

Every gradient (dX, dA, da, dB, db) is held to the bf16 bound of the forward,
max|G - O| / max|O| <= 2e-2 over the compared entries, and must be
bit-identical run to run (no atomics; fixed-order folds).
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
BF16_TOL = 2e-2
KEYS = ("dX", "dA", "da", "dB", "db")


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def dev(x, dtype=torch.bfloat16):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(DEV, dtype)


def err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def _host(T, H, F, bias, seed):
    rng = np.random.default_rng(seed)
    r = lambda shape, s: inputs.round_to_dtype((rng.standard_normal(shape) * s).astype(np.float32), "bf16")
    return {"X": r((T, H), 1.0), "A": r((F, H), 0.05), "a": r((F,), 0.05) if bias else None,
            "B": r((H, F), 0.05), "dY": r((T, H), 1.0)}


def _run(h, N, act=tp.TP_ACT_GELU, shard_begin=0, shard_count=None):
    X, A, a, B, dY = (dev(h[k]) for k in ("X", "A", "a", "B", "dY"))
    g, ws = tp.mlp_backward(X, A, a, B, dY, N, act=act, shard_begin=shard_begin, shard_count=shard_count,
                            need_da=a is not None)
    torch.cuda.synchronize()
    return g, ws


def _np(t):
    return t.float().cpu().numpy()


# T, H and the shard width all multiples of 64 (bf16): the GEMMs read every
# operand as stored (K-outer) and the bias gradients are column sums; any
# other shape transposes the operands first.
@pytest.mark.parametrize("T,H,F,N,act,bias", [
    (264, 136, 4 * 72, 4, tp.TP_ACT_GELU, True),     # transposed: ragged tiles in every dimension
    (64, 64, 2 * 64, 2, tp.TP_ACT_NONE, False),      # as stored: one 64-row k-tile
    (2048, 520, 8 * 40, 8, tp.TP_ACT_GELU, True),    # transposed: split-K weight gradients (2 splits)
    (4096, 256, 4 * 256, 4, tp.TP_ACT_GELU, False),  # as stored: two-pass dZ kernel, split-K
    (1024, 192, 4 * 320, 4, tp.TP_ACT_GELU, True),   # as stored: split-K, hidden narrower than a tile
    (512, 128, 192, 1, tp.TP_ACT_GELU, True),        # as stored: shard width ragged against the tile
    (8, 8, 8, 1, tp.TP_ACT_GELU, True),              # transposed: one shard, smallest sizes
])
def test_backward_vs_oracle(T, H, F, N, act, bias):
    say(f"mlp_backward T={T} H={H} F={F} N={N} act={act} bias={bias}")
    h = _host(T, H, F, bias, seed=T + H + F + N)
    g, _ = _run(h, N, act)
    g2, _ = _run(h, N, act)
    ref = R.mlp_gelu_backward(h["X"], h["A"], h["a"], h["B"], h["dY"],
                              act="gelu" if act == tp.TP_ACT_GELU else "none")
    for k in KEYS:
        if k == "da" and not bias:
            assert g["da"] is None
            continue
        e = err(_np(g[k]), ref[k])
        say(f"  {k}: err={e:.3e}")
        assert e <= BF16_TOL, k
        assert torch.equal(g[k], g2[k]), f"{k} not bit-identical run to run"


def test_bias_sums_alone_equal_shared():
    """On the as-stored path the two bias gradients (column sums of dZ and of
    dY) share their launches; each sum alone gives the same bits."""
    T, H, F, N = 1024, 192, 4 * 320, 4
    say(f"mlp_backward bias sums alone and shared T={T} H={H} F={F} N={N}")
    h = _host(T, H, F, True, seed=91)
    X, A, a, B, dY = (dev(h[k]) for k in ("X", "A", "a", "B", "dY"))
    both, _ = tp.mlp_backward(X, A, a, B, dY, N, need_da=True, need_db=True)
    only_a, _ = tp.mlp_backward(X, A, a, B, dY, N, need_da=True, need_db=False)
    only_b, _ = tp.mlp_backward(X, A, a, B, dY, N, need_da=False, need_db=True)
    torch.cuda.synchronize()
    assert only_a["db"] is None and only_b["da"] is None
    assert torch.equal(both["da"], only_a["da"])
    assert torch.equal(both["db"], only_b["db"])
    ref = R.mlp_gelu_backward(h["X"], h["A"], h["a"], h["B"], h["dY"], act="gelu")
    assert err(_np(both["da"]), ref["da"]) <= BF16_TOL
    assert err(_np(both["db"]), ref["db"]) <= BF16_TOL


def test_one_shard_range_matches_oracle_shard():
    """A one-shard range writes only that shard's rows of dA, columns of dB and
    entries of da, and leaves its dX partial in its slab slot."""
    T, H, F, N, r = 520, 264, 4 * 96, 4, 2
    say(f"mlp_backward one shard r={r} of N={N}")
    h = _host(T, H, F, True, seed=77)
    g, ws = _run(h, N, shard_begin=r, shard_count=1)
    assert g["dX"] is None
    sh = O.mlp_backward_sharded(h["X"], h["A"].T, h["a"], h["B"].T, h["dY"], N)
    Fs = F // N
    sl = slice(r * Fs, (r + 1) * Fs)
    dA, da, dB = _np(g["dA"]), _np(g["da"]), _np(g["dB"])
    assert err(dA[sl], sh["dA"][:, sl].T) <= BF16_TOL
    assert err(da[sl], sh["da"][sl]) <= BF16_TOL
    assert err(dB[:, sl], sh["dB"][sl].T) <= BF16_TOL
    assert err(_np(g["db"]), sh["db"]) <= BF16_TOL
    outside = np.ones(F, dtype=bool)
    outside[sl] = False
    assert not dA[outside].any() and not da[outside].any() and not dB[:, outside].any()
    P = tp.mlp_partials(ws, N, T, H)[r]
    assert err(_np(P), sh["dX_parts"][r]) <= BF16_TOL


def test_shard_ranges_compose_to_full_run():
    """Two half ranges plus the reduction over the slab give the full run's
    bits (each shard's work does not depend on which range launched it)."""
    T, H, F, N = 256, 128, 4 * 64, 4
    h = _host(T, H, F, True, seed=78)
    full, _ = _run(h, N)
    X, A, a, B, dY = (dev(h[k]) for k in ("X", "A", "a", "B", "dY"))
    g, ws = tp.mlp_backward(X, A, a, B, dY, N, shard_begin=0, shard_count=2)
    g, ws = tp.mlp_backward(X, A, a, B, dY, N, shard_begin=2, shard_count=2, grads=g, ws=ws)
    dX = tp.reduce_partials(tp.mlp_partials(ws, N, T, H), None, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(dX.view(torch.int16), full["dX"].view(torch.int16))
    for k in ("dA", "da", "dB", "db"):
        assert torch.equal(g[k], full[k]), k


def test_zero_upstream_gradient_gives_zero_gradients():
    T, H, F, N = 128, 64, 2 * 64, 2
    h = _host(T, H, F, True, seed=79)
    h["dY"] = np.zeros_like(h["dY"])
    g, _ = _run(h, N)
    for k in KEYS:
        assert not g[k].float().abs().sum().item(), k


def test_empty_tokens_is_noop():
    h = _host(8, 64, 128, True, seed=80)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    g, ws = tp.mlp_backward(X, dev(h["A"]), dev(h["a"]), dev(h["B"]), torch.empty_like(X), 2)
    torch.cuda.synchronize()
    assert ws is None and g["dX"].shape == (0, 64)
    assert not g["dA"].any() and not g["dB"].any()


@pytest.mark.parametrize("k", [2, 5])
def test_backward_full_size(k):
    """The GELU workloads at full size: all of workload 2 against the full
    oracle; workload 5 on sampled token rows (dX) and features (dA, da, dB)
    plus the whole db."""
    w = configs.CONFIGS[k]
    say(f"backward config {k} {w.name}: generating inputs")
    host = inputs.make_inputs(w)
    dY_h = inputs.grad_output(w)
    d = workloads.device_inputs(w, host)
    dY = dev(dY_h)
    say(f"backward config {k}: all {w.N} shards")
    g, ws = workloads.backward(w, d, dY)
    torch.cuda.synchronize()
    del ws
    if k == 2:
        say("backward config 2: full oracle")
        ref = R.mlp_gelu_backward(host["X"], host["A"], host["a"], host["B"], dY_h)
        got = {key: _np(g[key]) for key in KEYS}
    else:
        rows = inputs.sample_rows(w.T, 32, w.seed, [0, w.T - 1])
        feats = inputs.sample_rows(w.F, 16, w.seed + 1, [0, w.F - 1])
        say(f"backward config {k}: oracle on {len(rows)} rows and {len(feats)} features")
        ref = R.mlp_gelu_backward_sample(host["X"], host["A"], host["a"], host["B"], dY_h, rows, feats)
        ri = torch.from_numpy(rows).to(DEV)
        fi = torch.from_numpy(feats).to(DEV)
        got = {"dX": _np(g["dX"][ri]), "dA": _np(g["dA"][fi]), "da": _np(g["da"][fi]),
               "dB": _np(g["dB"][:, fi]), "db": _np(g["db"])}
    for key in KEYS:
        e = err(got[key], ref[key])
        say(f"backward config {k}: {key} err={e:.3e}")
        assert e <= BF16_TOL, key


# ------------------------------------------------------------------ SwiGLU
def _swiglu_host(T, H, I, seed):
    rng = np.random.default_rng(seed)
    r = lambda shape, s: inputs.round_to_dtype((rng.standard_normal(shape) * s).astype(np.float32), "bf16")
    return {"X": r((T, H), 1.0), "Wg": r((I, H), 0.05), "Wu": r((I, H), 0.05), "Wd": r((H, I), 0.05),
            "dY": r((T, H), 1.0)}


def _fused(Wg, Wu, N):
    """Per-shard [gate | up] row blocks, as the forward takes them."""
    I, H = Wg.shape
    s = I // N
    return np.concatenate([np.concatenate([Wg[i * s:(i + 1) * s], Wu[i * s:(i + 1) * s]]) for i in range(N)])


def _unfuse(dA, N):
    """Fused-block gradient [2I x H] back to (dWg, dWu), each [I x H]."""
    blocks = dA.reshape(N, 2, -1, dA.shape[1])
    return blocks[:, 0].reshape(-1, dA.shape[1]), blocks[:, 1].reshape(-1, dA.shape[1])


@pytest.mark.parametrize("T,H,I,N", [
    (264, 136, 4 * 40, 4),     # transposed operands: ragged tiles
    (2048, 512, 8 * 48, 8),    # transposed operands (shard's [gate | up] width 96): split-K
    (304, 256, 2 * 64, 2),
    (1024, 256, 4 * 96, 4),    # operands as stored: [gate | up] width 192, shard width ragged, split-K
])
def test_swiglu_backward_vs_oracle(T, H, I, N):
    say(f"swiglu backward T={T} H={H} I={I} N={N}")
    h = _swiglu_host(T, H, I, seed=T + H + I)
    A = dev(_fused(h["Wg"], h["Wu"], N))
    X, Wd, dY = dev(h["X"]), dev(h["Wd"]), dev(h["dY"])
    g, _ = tp.mlp_backward(X, A, None, Wd, dY, N, act=tp.TP_ACT_SWIGLU, need_db=True)
    g2, _ = tp.mlp_backward(X, A, None, Wd, dY, N, act=tp.TP_ACT_SWIGLU, need_db=True)
    torch.cuda.synchronize()
    ref = R.mlp_swiglu_backward(h["X"], h["Wg"], h["Wu"], h["Wd"], h["dY"])
    assert g["da"] is None
    dWg, dWu = _unfuse(_np(g["dA"]), N)
    got = {"dX": _np(g["dX"]), "dWg": dWg, "dWu": dWu, "dWd": _np(g["dB"]), "db": _np(g["db"])}
    for k in ("dX", "dWg", "dWu", "dWd", "db"):
        e = err(got[k], ref[k])
        say(f"  {k}: err={e:.3e}")
        assert e <= BF16_TOL, k
    for k in ("dX", "dA", "dB", "db"):
        assert torch.equal(g[k], g2[k]), f"{k} not bit-identical run to run"


def test_swiglu_backward_full_size():
    """The SwiGLU workload (T=32768, H=4096, I=11008, N=8) on sampled token
    rows (dX) and intermediate features (dWg, dWu, dWd)."""
    w = configs.CONFIGS[3]
    say(f"backward config 3 {w.name}: generating inputs")
    host = inputs.make_inputs(w)
    dY_h = inputs.grad_output(w)
    d = workloads.device_inputs(w, host)
    say("backward config 3: all 8 shards")
    g, ws = workloads.backward(w, d, dev(dY_h))
    torch.cuda.synchronize()
    del ws
    rows = inputs.sample_rows(w.T, 16, w.seed, [0, w.T - 1])
    feats = inputs.sample_rows(w.F, 12, w.seed + 1, [0, w.F - 1])
    say(f"backward config 3: oracle on {len(rows)} rows and {len(feats)} features")
    ref = R.mlp_swiglu_backward_sample(host["X"], host["Wg"], host["Wu"], host["Wd"], dY_h, rows, feats)
    Fs = w.F // w.N
    blk, off = feats // Fs, feats % Fs
    gate_rows = torch.from_numpy(blk * 2 * Fs + off).to(DEV)
    up_rows = torch.from_numpy(blk * 2 * Fs + Fs + off).to(DEV)
    got = {"dX": _np(g["dX"][torch.from_numpy(rows).to(DEV)]), "dWg": _np(g["dA"][gate_rows]),
           "dWu": _np(g["dA"][up_rows]), "dWd": _np(g["dB"][:, torch.from_numpy(feats).to(DEV)])}
    for key in ("dX", "dWg", "dWu", "dWd"):
        e = err(got[key], ref[key])
        say(f"backward config 3: {key} err={e:.3e}")
        assert e <= BF16_TOL, key


# ------------------------------------------------------------------ fp32
F32_TOL = 1e-4


@pytest.mark.parametrize("T,H,F,N,bias", [
    (136, 72, 2 * 48, 2, True),     # ragged tiles
    (512, 256, 4 * 64, 4, False),
])
def test_backward_f32_vs_oracle(T, H, F, N, bias):
    say(f"mlp_backward fp32 T={T} H={H} F={F} N={N} bias={bias}")
    rng = np.random.default_rng(T + H + F)
    h = {"X": rng.standard_normal((T, H)).astype(np.float32),
         "A": (rng.standard_normal((F, H)) * 0.05).astype(np.float32),
         "a": (rng.standard_normal(F) * 0.05).astype(np.float32) if bias else None,
         "B": (rng.standard_normal((H, F)) * 0.05).astype(np.float32),
         "dY": rng.standard_normal((T, H)).astype(np.float32)}
    X, A, a, B, dY = (dev(h[k], torch.float32) for k in ("X", "A", "a", "B", "dY"))
    g, _ = tp.mlp_backward(X, A, a, B, dY, N, need_da=bias)
    torch.cuda.synchronize()
    ref = R.mlp_gelu_backward(h["X"], h["A"], h["a"], h["B"], h["dY"])
    for k in KEYS:
        if k == "da" and not bias:
            continue
        e = err(_np(g[k]), ref[k])
        say(f"  {k}: err={e:.3e}")
        assert e <= F32_TOL, k


def test_backward_f32_full_size_workload_1():
    """The fp32 workload (T=128, H=512, F=2048, N=2) against the full oracle."""
    w = configs.CONFIGS[1]
    host = inputs.make_inputs(w)
    dY_h = inputs.grad_output(w)
    d = workloads.device_inputs(w, host)
    g, _ = workloads.backward(w, d, dev(dY_h, torch.float32))
    torch.cuda.synchronize()
    ref = R.mlp_gelu_backward(host["X"], host["A"], host["a"], host["B"], dY_h)
    for k in KEYS:
        e = err(_np(g[k]), ref[k])
        say(f"backward config 1: {k} err={e:.3e}")
        assert e <= F32_TOL, k
