"""Sequence-parallel entry side on the GPU vs the fp64 oracle, through the C ABI:
RMSNorm of each sequence slice into the gathered buffer (the all-gather
stand-in), alone and feeding the MLP sublayer with a reduce-scatter.

Tolerances.  The norm is elementwise after one row statistic, so each output
element is compared with the oracle's fp64 value.  bf16 output: the device
rounds its fp32 value once (round-to-nearest-even: under 2^-8 relative), and
that fp32 value carries a few fp32 ulps of evaluation error, so the bound is
2^-8 + 2^-20 relative.  fp32 output: 1e-5 relative (fp32 sum of squares and
the hardware reciprocal square root).  A small absolute floor (2^-20 of the
row-set maximum) covers outputs that round to zero.  The MLP
built on top keeps the suite's bf16 bound (normwise 2e-2).
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


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def _draw(seed, shape, sigma, dt):
    ss = np.random.SeedSequence(seed)
    return inputs.round_to_dtype(inputs.draw(ss, shape, sigma), dt)


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _check_norm(y_dev, ref, dt):
    y = y_dev.float().cpu().numpy().astype(np.float64)
    rel = 2.0 ** -8 + 2.0 ** -20 if dt == "bf16" else 1e-5
    floor = 2.0 ** -20 * float(np.max(np.abs(ref)))
    bad = np.abs(y - ref) > rel * np.abs(ref) + floor
    assert not bad.any(), f"{int(bad.sum())} elements off, worst |d| = {float(np.max(np.abs(y - ref))):.3e}"


@pytest.mark.parametrize("dt,n,T,H,eps,sl,separate", [
    ("bf16", 4, 64, 512, 1e-6, -1, False),
    ("bf16", 8, 96, 12288, 1e-6, -1, False),   # workload-5 hidden size
    ("bf16", 2, 10, 8, 1e-5, -1, False),       # one 16-byte piece, most lanes idle
    ("bf16", 3, 33, 520, 1e-6, 1, False),      # ragged hidden, one slice only
    ("bf16", 1, 7, 16384, 1e-6, -1, False),    # largest hidden
    ("bf16", 4, 64, 512, 1e-6, 2, True),       # slices in separate buffers
    ("f32", 2, 128, 512, 1e-5, -1, False),
    ("f32", 4, 20, 8192, 0.0, -1, True),       # largest fp32 hidden, eps = 0
])
def test_rmsnorm_gather_vs_oracle(dt, n, T, H, eps, sl, separate):
    say(f"rmsnorm_gather dt={dt} n={n} T={T} H={H} eps={eps} slice={sl} separate={separate}")
    seed = 7000 + T + H + n
    X = _draw(seed, (T, H), 1.0, dt)
    g = 1.0 + _draw(seed + 1, (H,), 0.1, "f32")
    g = inputs.round_to_dtype(g.astype(np.float32), dt)
    per = T // n
    tdt = _tdt(dt)
    gd = torch.from_numpy(g).to(DEV, tdt)
    Y = torch.full((T, H), 7.0, dtype=tdt, device=DEV)  # sentinel for rows a one-slice call must not touch
    if separate:
        # slice r lives at slot r of a padded slab: slots 2*per*H elements apart
        slab = torch.zeros((n, 2 * per, H), dtype=tdt, device=DEV)
        for r in range(n):
            slab[r, :per] = torch.from_numpy(X[r * per:(r + 1) * per]).to(DEV, tdt)
        tp.rmsnorm_gather(slab[0, :per], gd, eps, n, out=Y, slice=sl, slice_stride=2 * per * H)
    else:
        tp.rmsnorm_gather(torch.from_numpy(X).to(DEV, tdt), gd, eps, n, out=Y, slice=sl)
    torch.cuda.synchronize()
    ref = O.sp_entry(X, g, eps, n)
    rows = slice(None) if sl < 0 else slice(sl * per, (sl + 1) * per)
    _check_norm(Y[rows], ref[rows], dt)
    if sl >= 0:
        rest = torch.ones(T, dtype=torch.bool, device=DEV)
        rest[rows] = False
        assert bool((Y[rest] == 7.0).all()), "rows outside the slice were written"


def test_rmsnorm_gather_is_bit_identical_run_to_run():
    X = torch.from_numpy(_draw(7100, (256, 4096), 3.0, "bf16")).to(DEV, torch.bfloat16)
    g = torch.from_numpy(_draw(7101, (4096,), 1.0, "bf16")).to(DEV, torch.bfloat16)
    a = tp.rmsnorm_gather(X, g, 1e-6, 8)
    b = tp.rmsnorm_gather(X, g, 1e-6, 8)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_rmsnorm_gather_zero_rows_and_extreme_scale():
    """A zero row with eps > 0 stays zero; rows scaled by 2^+-40 normalize like
    the unscaled row (the statistic stays in fp32 range)."""
    H = 1024
    base = _draw(7200, (1, H), 1.0, "f32")
    X = np.concatenate([np.zeros((1, H)), base, base * 2.0 ** 40, base * 2.0 ** -40], axis=0).astype(np.float32)
    g = np.ones(H, dtype=np.float32)
    Y = tp.rmsnorm_gather(torch.from_numpy(X).to(DEV), torch.from_numpy(g).to(DEV), 1e-30, 2)
    torch.cuda.synchronize()
    y = Y.cpu().numpy().astype(np.float64)
    assert np.all(y[0] == 0.0)
    ref = O.rmsnorm(X.astype(np.float64), g, 1e-30)
    _check_norm(Y, ref, "f32")
    assert np.allclose(y[2], y[1], rtol=1e-5) and np.allclose(y[3], y[1], rtol=1e-5)


@pytest.mark.parametrize("T,H,F,N,ns", [(256, 512, 2048, 4, 4), (192, 1024, 1536, 2, 8)])
def test_sp_round_trip_vs_oracle(T, H, F, N, ns):
    """The whole sequence-parallel MLP sublayer: norm of each sequence slice,
    all-gather, column -> GELU -> row partials on N shards, then the
    reduce-scatter back to sequence slices (blog post section 4.3)."""
    say(f"sp round trip T={T} H={H} F={F} N={N} slices={ns}")
    seed = 7300 + T + H
    X = _draw(seed, (T, H), 1.0, "bf16")
    g = inputs.round_to_dtype((1.0 + _draw(seed + 1, (H,), 0.1, "f32")).astype(np.float32), "bf16")
    A = _draw(seed + 2, (F, H), 0.02, "bf16")     # [out x in] storage
    a = _draw(seed + 3, (F,), 0.02, "bf16")
    B = _draw(seed + 4, (H, F), 0.02, "bf16")
    b = _draw(seed + 5, (H,), 0.02, "bf16")
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV, torch.bfloat16)
    Xn = tp.rmsnorm_gather(d(X), d(g), 1e-6, ns)
    per = T // ns
    outs = []
    ws = None
    for r in range(ns):
        Yr = torch.empty((per, H), dtype=torch.bfloat16, device=DEV)
        _, ws = tp.mlp_forward(Xn, d(A), d(a), d(B), d(b), N, act=tp.TP_ACT_GELU, Y=Yr, ws=ws, n_slices=ns, slice=r)
        outs.append(Yr)
    torch.cuda.synchronize()
    xn64 = O.sp_entry(X, g, 1e-6, ns)
    # the normalized input crosses into the column GEMM as bf16, as on the device
    xn_b = inputs.round_to_dtype(xn64.astype(np.float32), "bf16").astype(np.float64)
    Yo = O.mlp_gelu(xn_b, A.T, a, B.T, b)
    for r in range(ns):
        ref = O.rs_slice(Yo, ns, r)
        y = outs[r].float().cpu().numpy()
        e = float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))
        assert e <= 2e-2, f"slice {r}: normwise error {e:.3e}"
    # the gathered normalized input itself
    _check_norm(Xn, xn64, "bf16")


def test_sp_entry_full_size_workload5_sampled():
    """Workload 5 at full size (T = 16384, H = 12288, 8 sequence slices), the
    launch bench.py --sp-entry times; the norm is row-wise, so sampled rows --
    including the first and last row of every slice -- are checked one by one
    against the oracle."""
    from tensor_transformer_layers_amd import configs
    w = configs.CONFIGS[5]
    say(f"sp entry full size: {w.name}")
    X = inputs.make_x(w)
    g = inputs.norm_gain(w)
    per = w.T // w.n_slices
    Xn = tp.rmsnorm_gather(torch.from_numpy(X).to(DEV, torch.bfloat16), torch.from_numpy(g).to(DEV, torch.bfloat16),
                           inputs.NORM_EPS, w.n_slices)
    torch.cuda.synchronize()
    must = [r * per for r in range(w.n_slices)] + [r * per + per - 1 for r in range(w.n_slices)]
    rows = inputs.sample_rows(w.T, 512, w.seed + 5, must=must)
    ref = O.rmsnorm(X[rows].astype(np.float64), g, inputs.NORM_EPS)
    _check_norm(Xn[torch.from_numpy(rows).to(DEV)], ref, "bf16")
