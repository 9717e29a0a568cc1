"""HIP path vs the fp64 CPU oracle, through the C ABI (gfx950 GPU required).

Tolerances: fp32 workloads max|Y - O| / max|O| <= 1e-4; bf16 workloads
max|Y - O| / max|O| <= 2e-2 (the oracle's max over the compared rows); the
fixed-order reduction is compared bit for bit with the oracle's fp32 fold.
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
F32_TOL = 1e-4


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV, dtype)


def err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def rng_bf16(rng, shape, sigma=1.0):
    return inputs.round_to_dtype((rng.standard_normal(shape) * sigma).astype(np.float32), "bf16")


# ------------------------------------------------------------------ reduction
@pytest.mark.parametrize("n,T,H,out,bias,ns,sl", [
    (1, 37, 64, "bf16", True, 1, -1),
    (2, 128, 512, "f32", True, 1, -1),
    (3, 50, 24, "bf16", False, 1, -1),
    (4, 1000, 520, "bf16", True, 1, -1),
    (8, 512, 1024, "bf16", True, 8, 3),
    (8, 512, 1024, "bf16", True, 8, 7),
    (5, 64, 8, "f32", False, 4, 0),
])
def test_reduce_bit_exact(n, T, H, out, bias, ns, sl):
    say(f"reduce n={n} T={T} H={H} out={out} bias={bias} slices={ns}/{sl}")
    rng = np.random.default_rng(100 + n * 7 + T)
    P = (rng.standard_normal((n, T, H)) * rng.choice([1e-3, 1.0, 300.0], size=(n, T, H))).astype(np.float32)
    b = inputs.round_to_dtype(rng.standard_normal(H).astype(np.float32), out) if bias else None
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    Pd = dev(P, torch.float32)
    bd = dev(b, odt) if bias else None
    y1 = tp.reduce_partials(Pd, bd, out_dtype=odt, n_slices=ns, slice=sl)
    y2 = tp.reduce_partials(Pd, bd, out_dtype=odt, n_slices=ns, slice=sl)
    torch.cuda.synchronize()
    want = O.reduce_partials_fp32(list(P), b, out=out, n_slices=ns, slice_=sl)
    if out == "bf16":
        got = y1.cpu().view(torch.int16).numpy().view(np.uint16)
        again = y2.cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        got, again = y1.cpu().numpy(), y2.cpu().numpy()
    assert np.array_equal(got, again), "reduction not bit-identical run to run"
    assert np.array_equal(got, want), "reduction differs from the fp32 left fold"


# ------------------------------------------------------------------ single linears
@pytest.mark.parametrize("T,K,Ns,act", [
    (333, 264, 200, tp.TP_ACT_GELU),
    (64, 64, 64, tp.TP_ACT_NONE),
    (257, 1376, 136, tp.TP_ACT_GELU),
    (4100, 136, 8200, tp.TP_ACT_GELU),     # 256x256 tiles, ragged M and N
    (300, 520, 96, tp.TP_ACT_SWIGLU),
    (4100, 72, 4104, tp.TP_ACT_SWIGLU),    # 256x256 tiles, ragged M and N
])
def test_column_linear_bf16(T, K, Ns, act):
    say(f"column_linear bf16 T={T} K={K} Ns={Ns} act={act}")
    rng = np.random.default_rng(T + K + Ns + act)
    X = rng_bf16(rng, (T, K))
    rows = 2 * Ns if act == tp.TP_ACT_SWIGLU else Ns
    W = rng_bf16(rng, (rows, K), 0.05)
    bias = rng_bf16(rng, (Ns,), 0.1) if act != tp.TP_ACT_SWIGLU else None
    Y = tp.column_linear(dev(X), dev(W), dev(bias) if bias is not None else None, act=act)
    torch.cuda.synchronize()
    Z = X.astype(np.float64) @ W.astype(np.float64).T
    if act == tp.TP_ACT_GELU:
        ref = O.gelu(Z + bias)
    elif act == tp.TP_ACT_NONE:
        ref = Z + bias
    else:
        ref = O.silu(Z[:, :Ns]) * Z[:, Ns:]
    e = err(Y.float().cpu().numpy(), ref)
    say(f"  err={e:.3e}")
    assert e <= BF16_TOL


@pytest.mark.parametrize("T,Ks,N", [(333, 264, 200), (257, 1376, 520), (4100, 200, 8200)])
def test_row_partial_bf16(T, Ks, N):
    say(f"row_linear_partial bf16 T={T} Ks={Ks} N={N}")
    rng = np.random.default_rng(T * 3 + Ks + N)
    X = rng_bf16(rng, (T, Ks))
    W = rng_bf16(rng, (N, Ks), 0.05)
    P = tp.row_linear_partial(dev(X), dev(W))
    torch.cuda.synchronize()
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    e = err(P.cpu().numpy(), ref)
    say(f"  err={e:.3e}")
    assert e <= 1e-5  # fp32 output of exact bf16 products, fp32 accumulation


@pytest.mark.parametrize("T,K,N", [(128, 512, 1024), (77, 36, 52)])
def test_linear_f32(T, K, N):
    say(f"linear f32 T={T} K={K} N={N}")
    rng = np.random.default_rng(T + K + N)
    X = rng.standard_normal((T, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    Y = tp.column_linear(dev(X, torch.float32), dev(W, torch.float32), dev(b, torch.float32), act=tp.TP_ACT_GELU)
    P = tp.row_linear_partial(dev(X, torch.float32), dev(W, torch.float32))
    torch.cuda.synchronize()
    Z = X.astype(np.float64) @ W.astype(np.float64).T
    assert err(Y.cpu().numpy(), O.gelu(Z + b)) <= F32_TOL
    assert err(P.cpu().numpy(), Z) <= F32_TOL


# ------------------------------------------------------------------ attention
def test_attn_local_vs_oracle():
    batch, seq, heads = 2, 384, 2
    say(f"attn_local batch={batch} seq={seq} heads={heads}")
    rng = np.random.default_rng(5)
    T, hd = batch * seq, heads * 128
    Q, K, V = (rng_bf16(rng, (T, hd)) for _ in range(3))
    QK = dev(np.concatenate([Q, K], axis=1))
    Vt = dev(V.T)
    Od = tp.attn_local(QK, hd, Vt, batch, seq, heads)
    torch.cuda.synchronize()
    ref = O.causal_attention(Q, K, V, batch, seq, heads)
    e = err(Od.float().cpu().numpy(), ref)
    say(f"  err={e:.3e}")
    assert e <= BF16_TOL
    # first row of every sequence is exactly (up to the bf16 cast) its first value row
    got = Od.float().cpu().numpy()
    for b in range(batch):
        assert np.array_equal(got[b * seq], V[b * seq])


# ------------------------------------------------------------------ whole sublayers
SMALL = {
    "gelu_bf16": configs.scaled(configs.CONFIGS[2], batch=1, seq=700, H=256, F=4 * 136, seed=11),
    "gelu_bf16_rs": configs.scaled(configs.CONFIGS[5], batch=4, seq=160, H=264, F=8 * 64, seed=12),
    "swiglu_bf16": configs.scaled(configs.CONFIGS[3], batch=1, seq=300, H=512, F=8 * 40, seed=13),
    "gelu_f32": configs.scaled(configs.CONFIGS[1], batch=1, seq=100, H=64, F=2 * 96, seed=14),
    "attn_bf16": configs.scaled(configs.CONFIGS[4], batch=2, seq=256, H=512, F=512, heads=4, N=2, seed=15),
}


def _run(w, host, **kw):
    d = workloads.device_inputs(w, host)
    Y, ws = workloads.forward(w, d, **kw)
    torch.cuda.synchronize()
    return d, Y, ws


@pytest.mark.parametrize("name", list(SMALL))
def test_sublayer_small_vs_oracle(name):
    w = SMALL[name]
    say(f"sublayer {name}: {w}")
    host = inputs.make_inputs(w)
    d, Y, ws = _run(w, host)
    ref = R.workload(w.kind, host, w.batch, w.seq, w.heads)
    e = err(Y.float().cpu().numpy(), ref)
    say(f"  err={e:.3e}")
    assert e <= (F32_TOL if w.dtype == "f32" else BF16_TOL)
    # run-to-run bit identity of the whole sublayer
    Y2, _ = workloads.forward(w, d, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16) if Y.dtype == torch.bfloat16 else Y,
                       Y2.view(torch.int16) if Y2.dtype == torch.bfloat16 else Y2)


@pytest.mark.parametrize("name", ["gelu_bf16", "attn_bf16", "swiglu_bf16"])
def test_one_rank_share_equals_full_run(name):
    """Shard r alone into a slab holding the other partials, then the
    reduction alone: bit-identical to the all-shards call."""
    w = SMALL[name]
    say(f"one-rank share {name}")
    host = inputs.make_inputs(w)
    d, Y, ws = _run(w, host)
    Y_full = Y.clone()
    P = tp.mlp_partials(ws, w.N, w.T, w.H)
    P.zero_()
    for r in range(w.N):
        workloads.forward(w, d, ws=ws, shard_begin=r, shard_count=1)
    Yr = workloads.reduce_slab(w, d, ws)
    torch.cuda.synchronize()
    assert torch.equal(Yr.view(torch.int16), Y_full.view(torch.int16))


def test_rs_slices_concatenate_to_full():
    w = SMALL["gelu_bf16_rs"]
    say("reduce-scatter slices")
    host = inputs.make_inputs(w)
    d, Y, ws = _run(w, host)
    parts = [workloads.reduce_slab(w, d, ws, slice=r) for r in range(w.n_slices)]
    Ys = [workloads.forward(w, d, ws=ws, slice=r)[0] for r in range(w.n_slices)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts).view(torch.int16), Y.view(torch.int16))
    assert torch.equal(torch.cat(Ys).view(torch.int16), Y.view(torch.int16))


def test_bias_counted_once_on_gpu():
    w = SMALL["gelu_bf16"]
    say("bias once")
    host = inputs.make_inputs(w)
    host = dict(host, B=np.zeros_like(host["B"]))
    d, Y, ws = _run(w, host)
    want = np.broadcast_to(host["b"], Y.shape)
    assert np.array_equal(Y.float().cpu().numpy(), want)


def test_empty_tokens_is_noop():
    say("T = 0")
    X = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((32, 64), dtype=torch.bfloat16, device=DEV)
    Y = tp.column_linear(X, W, None, act=tp.TP_ACT_NONE)
    assert Y.shape == (0, 32)


# ------------------------------------------------------------------ fused narrow-hidden MLP kernel
# (T, H, F, N, act, bias): ragged token blocks, H = 256 / 512, odd and single
# chunk counts per shard, no column bias, fewer tokens than one block
FUSED = [
    (1000, 512, 4 * 64, 4, "gelu", True),
    (300, 256, 2 * 96, 2, "none", True),
    (128, 512, 4 * 32, 4, "gelu", False),
    (77, 256, 8 * 32, 8, "gelu", True),
]


def _fused_inputs(T, H, F, seed):
    rng = np.random.default_rng(seed)
    X = rng_bf16(rng, (T, H))
    A = rng_bf16(rng, (F, H), 0.05)   # [out x in]; pre-activations ~N(0, 1.3)
    a = rng_bf16(rng, (F,), 0.1)
    B = rng_bf16(rng, (H, F), 0.05)
    b = rng_bf16(rng, (H,), 0.1)
    return X, A, a, B, b


@pytest.mark.parametrize("T,H,F,N,act,bias", FUSED)
def test_fused_mlp_vs_oracle(T, H, F, N, act, bias):
    say(f"fused mlp T={T} H={H} F={F} N={N} act={act} bias={bias}")
    X, A, a, B, b = _fused_inputs(T, H, F, seed=T + H + F + N)
    if not bias:
        a = None
    code = tp.TP_ACT_GELU if act == "gelu" else tp.TP_ACT_NONE
    Y, ws = tp.mlp_forward(dev(X), dev(A), None if a is None else dev(a), dev(B), dev(b), N, act=code)
    torch.cuda.synchronize()
    if act == "gelu":
        ref = O.mlp_gelu(X, A.T, a, B.T, b)
    else:
        ref = O.linear(O.linear(X, A.T, a), B.T, b)
    e = err(Y.float().cpu().numpy(), ref)
    say(f"  err={e:.3e}")
    assert e <= BF16_TOL


def test_fused_mlp_matches_separate_kernels():
    """The fused kernel's partials against the column kernel (GELU epilogue)
    followed by the row-partial kernel, shard by shard.  The products run in
    the same k order and the activation is the same arithmetic, but the fused
    kernel adds the bias before the products (as the accumulator's initial
    value) and the column kernel after, so a pre-activation can differ in its
    last fp32 bit and, rarely, round to a neighbouring bf16 intermediate: one
    such unit moves a partial by at most 2^-7 |h| |B|, under 4e-3 of max|P|
    here.  A wrong operand, index or missing term would be of order 1."""
    T, H, F, N = 640, 512, 4 * 64, 4
    Fs = F // N
    say("fused vs separate kernels")
    X, A, a, B, b = (dev(t) for t in _fused_inputs(T, H, F, seed=5))
    Y, ws = tp.mlp_forward(X, A, a, B, b, N, act=tp.TP_ACT_GELU)
    Pf = tp.mlp_partials(ws, N, T, H).clone()
    worst, same = 0.0, True
    for i in range(N):
        Hi = tp.column_linear(X, A[i * Fs:(i + 1) * Fs], a[i * Fs:(i + 1) * Fs], act=tp.TP_ACT_GELU)
        Pi = tp.row_linear_partial(Hi, B[:, i * Fs:(i + 1) * Fs])
        torch.cuda.synchronize()
        d = (Pi - Pf[i]).abs().max().item() / Pi.abs().max().item()
        worst = max(worst, d)
        same = same and torch.equal(Pi, Pf[i])
    say(f"  max rel diff {worst:.3e}, bit-identical: {same}")
    assert worst <= 4e-3


# ------------------------------------------------------------------ the five workloads at full size
def _sample_rows(w):
    """Token rows the full-size check compares: every row where the fp64
    oracle finishes in seconds (workloads 1, 2 and the attention block,
    whose rows need their whole causal prefix anyway), else 1024 seeded rows
    that include the first and last token and the first and last row of
    every reduce-scatter slice (the MLP is token-wise, so a row's oracle
    value needs no other row)."""
    if w.kind == "attn" or (w.T <= 16384 and w.kind == "mlp_gelu" and w.H <= 512):
        return None  # the full oracle
    must = [0, w.T - 1]
    if w.n_slices > 1:
        s = w.T // w.n_slices
        must += [r * s for r in range(w.n_slices)] + [r * s + s - 1 for r in range(w.n_slices)]
    return inputs.sample_rows(w.T, 1024, w.seed, must)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_config_full_size(k):
    w = configs.CONFIGS[k]
    say(f"config {k} {w.name}: generating inputs")
    host = inputs.make_inputs(w)
    d = workloads.device_inputs(w, host)
    say(f"config {k}: forward (all {w.N} shards)")
    Y, ws = workloads.forward(w, d)
    torch.cuda.synchronize()
    rows = _sample_rows(w)
    say(f"config {k}: oracle on {'all' if rows is None else len(rows)} rows")
    ref = R.workload(w.kind, host, w.batch, w.seq, w.heads, rows=rows)
    got = Y.float()[torch.from_numpy(rows).to(DEV)] if rows is not None else Y.float()
    e = err(got.cpu().numpy(), ref)
    say(f"config {k}: err={e:.3e}")
    assert e <= (F32_TOL if w.dtype == "f32" else BF16_TOL)
    if w.n_slices > 1:
        # rank r's reduce-scatter slice == rows of the full result
        r = w.n_slices - 1
        Ysl = workloads.reduce_slab(w, d, ws, slice=r)
        torch.cuda.synchronize()
        s = w.T // w.n_slices
        assert torch.equal(Ysl.view(torch.int16), Y[r * s:(r + 1) * s].view(torch.int16))
