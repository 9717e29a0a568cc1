"""The forward's stored pre-activation (tp_mlp_desc.Z) and the backward that
takes it (tp_mlp_bwd_desc.Z) instead of recomputing X A^T + a, through the C
ABI (gfx950 GPU required).

  * Z against the fp64 definition X A^T + a: one bf16 rounding, so
    max|Z - O| / max|O| <= 1e-2.
  * Asking for Z leaves the forward's output as it was: bit for bit where
    both runs take the two-GEMM path, within the bf16 bound of the oracle
    where the narrow-hidden fused kernel served the run without Z.
  * The backward with the stored Z against the fp64 oracle (bf16 bound 2e-2,
    as for the recomputing backward), and bit for bit equal to the
    recomputing backward where that one also runs the GEMM path (H > 2048, or
    no activation): the forward's column product and the recomputation
    accumulate the same products in the same order and round once.
  * A shard range writes its own columns of Z and no others.
  * SwiGLU: Z holds each shard's [gate | up] pre-activations; the same
    checks, with the backward bit for bit equal to the recomputing one.
  * The stored activation (tp_mlp_desc.Hact / tp_mlp_bwd_desc.Hact): the
    forward's output and Z keep their bits, H against the fp64 activation of
    the fp64 pre-activation (one bf16 rounding), and a GELU backward that
    reads it for dB keeps every other gradient's bits.
"""
import sys

import numpy as np
import pytest

from oracle import reference as R
from oracle import tp_oracle as O
from tensor_transformer_layers_amd import inputs, tp

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

DEV = "cuda"
BF16_TOL = 2e-2
Z_TOL = 1e-2
KEYS = ("dX", "dA", "da", "dB", "db")


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def dev(x, dtype=torch.bfloat16):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(DEV, dtype)


def err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def _np(t):
    return t.float().cpu().numpy()


def _host(T, H, F, bias, seed):
    rng = np.random.default_rng(seed)
    r = lambda shape, s: inputs.round_to_dtype((rng.standard_normal(shape) * s).astype(np.float32), "bf16")
    return {"X": r((T, H), 1.0), "A": r((F, H), 0.05), "a": r((F,), 0.05) if bias else None,
            "B": r((H, F), 0.05), "dY": r((T, H), 1.0)}


def _zref(h):
    z = h["X"].astype(np.float64) @ h["A"].astype(np.float64).T
    return z if h["a"] is None else z + h["a"].astype(np.float64)


@pytest.mark.parametrize("T,H,F,N,act,bias", [
    (264, 136, 4 * 72, 4, tp.TP_ACT_GELU, True),     # narrow: fused forward, two-pass backward otherwise
    (256, 2304, 4 * 64, 4, tp.TP_ACT_GELU, True),    # GEMM path both ways
    (128, 2304, 2 * 64, 2, tp.TP_ACT_NONE, False),
    (2048, 520, 8 * 40, 8, tp.TP_ACT_GELU, True),    # split-K weight gradients
    (2048, 256, 4 * 128, 4, tp.TP_ACT_GELU, True),   # operands as stored: GELU(Z) written by the dZ GEMM
])
def test_stored_preactivation(T, H, F, N, act, bias):
    say(f"stored Z T={T} H={H} F={F} N={N} act={act} bias={bias}")
    h = _host(T, H, F, bias, seed=7 * T + H + F + N)
    X, A, a, B, dY = (dev(h[k]) for k in ("X", "A", "a", "B", "dY"))
    Z = torch.empty((T, F), dtype=torch.bfloat16, device=DEV)
    Y0, _ = tp.mlp_forward(X, A, a, B, None, N, act=act)
    Y1, _ = tp.mlp_forward(X, A, a, B, None, N, act=act, Z=Z)
    torch.cuda.synchronize()
    e = err(_np(Z), _zref(h))
    say(f"  Z err={e:.3e}")
    assert e <= Z_TOL
    yref = O.mlp_gelu(h["X"], h["A"].T, h["a"], h["B"].T, None) if act == tp.TP_ACT_GELU else \
        O.linear(O.linear(h["X"], h["A"].T, h["a"]), h["B"].T, None)
    e0, e1 = err(_np(Y0), yref), err(_np(Y1), yref)
    say(f"  Y err without Z {e0:.3e}, with Z {e1:.3e}")
    assert e0 <= BF16_TOL and e1 <= BF16_TOL
    fused = H in (256, 512) and (F // N) % 32 == 0
    if not fused:
        assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))

    g0, _ = tp.mlp_backward(X, A, a, B, dY, N, act=act, need_da=bias)
    g1, _ = tp.mlp_backward(X, A, a, B, dY, N, act=act, need_da=bias, Z=Z)
    torch.cuda.synchronize()
    ref = R.mlp_gelu_backward(h["X"], h["A"], h["a"], h["B"], h["dY"],
                              act="gelu" if act == tp.TP_ACT_GELU else "none")
    same_path = H > 2048 or act == tp.TP_ACT_NONE
    for k in KEYS:
        if k == "da" and not bias:
            assert g1["da"] is None
            continue
        e = err(_np(g1[k]), ref[k])
        say(f"  {k}: err={e:.3e}")
        assert e <= BF16_TOL, k
        if same_path:
            assert torch.equal(g0[k], g1[k]), f"{k}: stored Z differs from the recomputation"


def test_stored_preactivation_shard_range():
    """Shards [1, 3) of 4 write their columns of Z and leave the rest alone;
    a backward over the same range with that Z equals the recomputing one."""
    T, H, F, N = 256, 2304, 4 * 64, 4
    h = _host(T, H, F, True, seed=11)
    X, A, a, B, dY = (dev(h[k]) for k in ("X", "A", "a", "B", "dY"))
    Fs = F // N
    Zfull = torch.empty((T, F), dtype=torch.bfloat16, device=DEV)
    tp.mlp_forward(X, A, a, B, None, N, Z=Zfull)
    Z = torch.full((T, F), float("nan"), dtype=torch.bfloat16, device=DEV)
    tp.mlp_forward(X, A, a, B, None, N, shard_begin=1, shard_count=2, Z=Z)
    torch.cuda.synchronize()
    cols = slice(Fs, 3 * Fs)
    assert torch.equal(Z[:, cols].view(torch.int16), Zfull[:, cols].view(torch.int16))
    assert torch.isnan(Z[:, :Fs].float()).all() and torch.isnan(Z[:, 3 * Fs:].float()).all()
    g0, _ = tp.mlp_backward(X, A, a, B, dY, N, shard_begin=1, shard_count=2)
    g1, _ = tp.mlp_backward(X, A, a, B, dY, N, shard_begin=1, shard_count=2, Z=Z)
    torch.cuda.synchronize()
    for k in ("dA", "da", "dB", "db"):
        assert torch.equal(g0[k], g1[k]), k


# ------------------------------------------------------------------ SwiGLU
def _swiglu_host(T, H, I, seed):
    rng = np.random.default_rng(seed)
    r = lambda shape, s: inputs.round_to_dtype((rng.standard_normal(shape) * s).astype(np.float32), "bf16")
    return {"X": r((T, H), 1.0), "Wg": r((I, H), 0.05), "Wu": r((I, H), 0.05), "Wd": r((H, I), 0.05),
            "dY": r((T, H), 1.0)}


def _fused_blocks(Wg, Wu, N):
    """Per-shard [gate | up] row blocks, as the forward takes them."""
    s = Wg.shape[0] // N
    return np.concatenate([np.concatenate([Wg[i * s:(i + 1) * s], Wu[i * s:(i + 1) * s]]) for i in range(N)])


@pytest.mark.parametrize("T,H,I,N", [
    (264, 136, 4 * 40, 4),     # the backward transposes its operands
    (1024, 256, 4 * 96, 4),    # the backward reads its operands as stored
])
def test_stored_preactivation_swiglu(T, H, I, N):
    """SwiGLU: the forward writes each shard's [gate | up] pre-activations
    (against the fp64 products, one bf16 rounding), asking for them leaves Y
    unchanged bit for bit, and the backward that takes them equals the
    recomputing one bit for bit (the recomputation runs the same products in
    the same k order) and the oracle within the bf16 bound."""
    say(f"stored Z swiglu T={T} H={H} I={I} N={N}")
    h = _swiglu_host(T, H, I, seed=3 * T + H + I)
    A = dev(_fused_blocks(h["Wg"], h["Wu"], N))
    X, Wd, dY = dev(h["X"]), dev(h["Wd"]), dev(h["dY"])
    Z = torch.empty((T, 2 * I), dtype=torch.bfloat16, device=DEV)
    Y0, _ = tp.mlp_forward(X, A, None, Wd, None, N, act=tp.TP_ACT_SWIGLU)
    Y1, _ = tp.mlp_forward(X, A, None, Wd, None, N, act=tp.TP_ACT_SWIGLU, Z=Z)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
    Is = I // N
    x = h["X"].astype(np.float64)
    zref = np.concatenate([np.concatenate([x @ h["Wg"][i * Is:(i + 1) * Is].astype(np.float64).T,
                                           x @ h["Wu"][i * Is:(i + 1) * Is].astype(np.float64).T], axis=1)
                           for i in range(N)], axis=1)
    e = err(_np(Z), zref)
    say(f"  Z err={e:.3e}")
    assert e <= Z_TOL

    g0, _ = tp.mlp_backward(X, A, None, Wd, dY, N, act=tp.TP_ACT_SWIGLU, need_db=True)
    g1, _ = tp.mlp_backward(X, A, None, Wd, dY, N, act=tp.TP_ACT_SWIGLU, need_db=True, Z=Z)
    torch.cuda.synchronize()
    for k in ("dX", "dA", "dB", "db"):
        assert torch.equal(g0[k], g1[k]), f"{k}: stored Z differs from the recomputation"
    ref = R.mlp_swiglu_backward(h["X"], h["Wg"], h["Wu"], h["Wd"], h["dY"])
    blocks = _np(g1["dA"]).reshape(N, 2, Is, H)
    got = {"dX": _np(g1["dX"]), "dWg": blocks[:, 0].reshape(-1, H), "dWu": blocks[:, 1].reshape(-1, H),
           "dWd": _np(g1["dB"]), "db": _np(g1["db"])}
    for k in ("dX", "dWg", "dWu", "dWd", "db"):
        e = err(got[k], ref[k])
        say(f"  {k}: err={e:.3e}")
        assert e <= BF16_TOL, k


# ------------------------------------------------------- stored activation
@pytest.mark.parametrize("T,H,F,N,bias", [
    (2048, 256, 4 * 128, 4, True),   # operands as stored, 128x128 dZ tiles: dZ alone, dB reads H
    (256, 2304, 4 * 64, 4, True),    # operands as stored, 256x256 tiles
    (264, 136, 4 * 72, 4, False),    # the backward transposes its operands: H^T instead of GELU(Z)^T
])
def test_stored_activation(T, H, F, N, bias):
    """The forward also keeps its activated intermediate (tp_mlp_desc.Hact):
    Y and Z keep their bits, H is GELU of the fp32 pre-activation rounded
    once (against the fp64 GELU of X A^T + a), and the backward that takes it
    for dB (tp_mlp_bwd_desc.Hact) leaves dX, dA, da and db bit for bit as
    the Z-only backward has them, with dB within the bf16 bound."""
    say(f"stored H T={T} H={H} F={F} N={N} bias={bias}")
    h = _host(T, H, F, bias, seed=5 * T + H + F)
    X, A, a, B, dY = (dev(h[k]) for k in ("X", "A", "a", "B", "dY"))
    Z0 = torch.empty((T, F), dtype=torch.bfloat16, device=DEV)
    Z1 = torch.empty_like(Z0)
    Hh = torch.empty_like(Z0)
    Y0, _ = tp.mlp_forward(X, A, a, B, None, N, Z=Z0)
    Y1, _ = tp.mlp_forward(X, A, a, B, None, N, Z=Z1, Hact=Hh)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
    assert torch.equal(Z0.view(torch.int16), Z1.view(torch.int16))
    href = O.gelu(_zref(h))
    e = err(_np(Hh), href)
    say(f"  H err={e:.3e}")
    assert e <= Z_TOL

    g0, _ = tp.mlp_backward(X, A, a, B, dY, N, need_da=bias, Z=Z0)
    g1, _ = tp.mlp_backward(X, A, a, B, dY, N, need_da=bias, Z=Z0, Hact=Hh)
    torch.cuda.synchronize()
    for k in ("dX", "dA", "da", "db"):
        if g0[k] is None:
            assert g1[k] is None
            continue
        assert torch.equal(g0[k], g1[k]), f"{k}: changed by the stored activation"
    ref = R.mlp_gelu_backward(h["X"], h["A"], h["a"], h["B"], h["dY"], act="gelu")
    e = err(_np(g1["dB"]), ref["dB"])
    say(f"  dB err={e:.3e}")
    assert e <= BF16_TOL


def test_stored_activation_swiglu_forward():
    """SwiGLU forward with Hact: Y keeps its bits and H = SiLU(G) U (fp64
    oracle, one bf16 rounding)."""
    T, H, I, N = 264, 136, 4 * 40, 4
    say(f"stored H swiglu forward T={T} H={H} I={I} N={N}")
    h = _swiglu_host(T, H, I, seed=17)
    A = dev(_fused_blocks(h["Wg"], h["Wu"], N))
    X, Wd = dev(h["X"]), dev(h["Wd"])
    Hh = torch.empty((T, I), dtype=torch.bfloat16, device=DEV)
    Y0, _ = tp.mlp_forward(X, A, None, Wd, None, N, act=tp.TP_ACT_SWIGLU)
    Y1, _ = tp.mlp_forward(X, A, None, Wd, None, N, act=tp.TP_ACT_SWIGLU, Hact=Hh)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
    x = h["X"].astype(np.float64)
    g = x @ h["Wg"].astype(np.float64).T
    u = x @ h["Wu"].astype(np.float64).T
    e = err(_np(Hh), g / (1.0 + np.exp(-g)) * u)
    say(f"  H err={e:.3e}")
    assert e <= Z_TOL
