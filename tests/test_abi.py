"""The C-ABI library loads, exports every symbol include/tp.h declares, and
rejects bad arguments before touching the GPU (no compute call here: every
call below fails validation or is a no-op, so none reaches HIP)."""
import ctypes
import os
import re
import subprocess

import pytest

from tensor_transformer_layers_amd import tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp.h")

FAKE = 0x100000  # 16-byte aligned, never dereferenced (validation fails first)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tp.LIB_PATH):
        pytest.skip("libtp.so not built")
    return tp.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", tp.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (tp_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(L, n)
        assert n in tp._SIGS, f"binding lacks {n}"


def test_version_and_status_strings(L):
    assert tp.lib().tp_version().decode().startswith("libtp")
    assert tp.status_string(tp.TP_ERR_DIVISIBILITY) == "TP_ERR_DIVISIBILITY"
    assert tp.status_string(99) == "TP_ERR_UNKNOWN"


def _mlp(**kw):
    d = tp.MlpDesc()
    d.dt, d.act = tp.TP_BF16, tp.TP_ACT_GELU
    d.T, d.H, d.F, d.N = 256, 512, 2048, 4
    d.shard_begin, d.shard_count = 0, 4
    d.X = d.A = d.a = d.B = d.b = d.Y = FAKE
    d.n_slices, d.slice = 1, -1
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_mlp_workspace_size_is_host_only(L):
    d = _mlp()
    need = tp.tp_mlp_workspace_size(d)
    p_bytes = 4 * 256 * 512 * 4
    h_bytes = 4 * 256 * 512 * 2
    assert need == p_bytes + h_bytes
    d.shard_count = 1
    assert tp.tp_mlp_workspace_size(d) == p_bytes + 256 * 512 * 2


@pytest.mark.parametrize("kw,status,needle", [
    (dict(F=2050), tp.TP_ERR_DIVISIBILITY, "not divisible by N=4"),
    (dict(N=3, shard_count=3, F=3 * 2044), tp.TP_ERR_ALIGN, "F/N=2044 is not a multiple of 8"),
    (dict(X=None), tp.TP_ERR_NULL, "X is NULL"),
    (dict(B=None), tp.TP_ERR_NULL, "B is NULL"),
    (dict(A=FAKE + 2), tp.TP_ERR_ALIGN, "A is not 16-byte aligned"),
    (dict(dt=7), tp.TP_ERR_DTYPE, "dtype"),
    (dict(act=9), tp.TP_ERR_DTYPE, "activation"),
    (dict(act=tp.TP_ACT_SWIGLU, dt=tp.TP_F32), tp.TP_ERR_DTYPE, "bf16-only"),
    (dict(act=tp.TP_ACT_SWIGLU), tp.TP_ERR_SHAPE, "bias must be NULL"),
    (dict(shard_begin=3, shard_count=2), tp.TP_ERR_SHAPE, "shard range"),
    (dict(n_slices=3), tp.TP_ERR_DIVISIBILITY, "sequence slices"),
    (dict(n_slices=4, slice=4), tp.TP_ERR_SHAPE, "slice 4"),
    (dict(H=500), tp.TP_ERR_ALIGN, "hidden H=500"),
    (dict(Y=None), tp.TP_ERR_NULL, "Y is NULL"),
    (dict(Z=FAKE, dt=tp.TP_F32), tp.TP_ERR_DTYPE, "bf16 path only"),
    (dict(Z=FAKE + 4, act=tp.TP_ACT_SWIGLU, a=None), tp.TP_ERR_ALIGN, "Z is not 16-byte aligned"),
    (dict(Z=FAKE + 8), tp.TP_ERR_ALIGN, "Z is not 16-byte aligned"),
    (dict(Hact=FAKE, dt=tp.TP_F32), tp.TP_ERR_DTYPE, "bf16 path only"),
    (dict(Hact=FAKE, act=tp.TP_ACT_NONE), tp.TP_ERR_SHAPE, "intermediate is the pre-activation"),
    (dict(Hact=FAKE + 8), tp.TP_ERR_ALIGN, "Hact is not 16-byte aligned"),
])
def test_mlp_validation(L, kw, status, needle):
    d = _mlp(**kw)
    s = tp.tp_mlp_forward(None, d, FAKE, 1 << 40)
    assert s == status, (tp.status_string(s), tp.last_error())
    assert needle in tp.last_error()
    assert tp.tp_mlp_workspace_size(d) == 0


def test_mlp_workspace_errors(L):
    d = _mlp()
    need = tp.tp_mlp_workspace_size(d)
    assert tp.tp_mlp_forward(None, d, None, need) == tp.TP_ERR_WORKSPACE
    assert tp.tp_mlp_forward(None, d, FAKE, need - 1) == tp.TP_ERR_WORKSPACE
    assert "needed" in tp.last_error()
    assert tp.tp_mlp_forward(None, d, FAKE + 8, need) == tp.TP_ERR_ALIGN


def _attn(**kw):
    d = tp.AttnDesc()
    d.dt = tp.TP_BF16
    d.batch, d.seq, d.hidden = 2, 256, 1024
    d.heads, d.head_dim, d.N = 8, 128, 4
    d.shard_begin, d.shard_count = 0, 4
    d.X = d.Wqkv = d.Wo = d.Y = FAKE
    d.bo = None
    d.n_slices, d.slice = 1, -1
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,status,needle", [
    (dict(N=3), tp.TP_ERR_DIVISIBILITY, "heads=8 are not divisible by N=3"),
    (dict(head_dim=64, hidden=512), tp.TP_ERR_SHAPE, "head_dim=64"),
    (dict(hidden=2048), tp.TP_ERR_SHAPE, "heads*head_dim"),
    (dict(seq=200), tp.TP_ERR_SHAPE, "multiple of 128"),
    (dict(dt=tp.TP_F32), tp.TP_ERR_DTYPE, "bf16-only"),
    (dict(Wqkv=None), tp.TP_ERR_NULL, "Wqkv is NULL"),
])
def test_attn_validation(L, kw, status, needle):
    d = _attn(**kw)
    s = tp.tp_attn_forward(None, d, FAKE, 1 << 40)
    assert s == status, (tp.status_string(s), tp.last_error())
    assert needle in tp.last_error()


def test_attn_workspace_size(L):
    d = _attn()
    T, hd = 512, 2 * 128
    want = 4 * T * 1024 * 4 + 4 * T * 2 * hd * 2 + 4 * hd * T * 2 + 4 * T * hd * 2
    assert tp.tp_attn_workspace_size(d) == want


def test_linear_and_reduce_validation(L):
    # K not a multiple of 8 (bf16)
    s = tp.tp_column_linear(None, tp.TP_BF16, tp.TP_ACT_GELU, 16, 12, 16, FAKE, 16, FAKE, 16, None, FAKE, 16)
    assert s == tp.TP_ERR_ALIGN and "K=12" in tp.last_error()
    # ld smaller than the row
    s = tp.tp_column_linear(None, tp.TP_BF16, tp.TP_ACT_GELU, 16, 64, 16, FAKE, 32, FAKE, 64, None, FAKE, 16)
    assert s == tp.TP_ERR_SHAPE and "leading dimension" in tp.last_error()
    s = tp.tp_row_linear_partial(None, tp.TP_F32, 16, 64, 16, FAKE, 64, None, 64, FAKE, 16)
    assert s == tp.TP_ERR_NULL
    # output leading dimensions must keep the vector stores aligned
    s = tp.tp_column_linear(None, tp.TP_BF16, tp.TP_ACT_GELU, 16, 64, 16, FAKE, 64, FAKE, 64, None, FAKE, 20)
    assert s == tp.TP_ERR_ALIGN and "ldy" in tp.last_error()
    s = tp.tp_row_linear_partial(None, tp.TP_BF16, 16, 64, 16, FAKE, 64, FAKE, 64, FAKE, 18)
    assert s == tp.TP_ERR_ALIGN and "ldp" in tp.last_error()
    # partials overlapping
    s = tp.tp_reduce_partials(None, tp.TP_BF16, 4, 8, 16, FAKE, 64, None, FAKE, 1, -1)
    assert s == tp.TP_ERR_SHAPE and "overlap" in tp.last_error()
    s = tp.tp_reduce_partials(None, tp.TP_BF16, 4, 8, 12, FAKE, 96, None, FAKE, 1, -1)
    assert s == tp.TP_ERR_ALIGN
    s = tp.tp_reduce_partials(None, tp.TP_BF16, 0, 8, 16, FAKE, 128, None, FAKE, 1, -1)
    assert s == tp.TP_ERR_SHAPE
    # empty inputs are a no-op that succeeds without any HIP call
    assert tp.tp_column_linear(None, tp.TP_BF16, tp.TP_ACT_GELU, 0, 64, 16, FAKE, 64, FAKE, 64, None, FAKE, 16) == tp.TP_OK
    assert tp.tp_reduce_partials(None, tp.TP_BF16, 4, 0, 16, FAKE, 0, None, FAKE, 1, -1) == tp.TP_OK
    assert tp.tp_attn_local(None, 0, 128, 2, 128, FAKE, 512, 256, FAKE, 8, FAKE, 256) == tp.TP_OK


def test_attn_local_validation(L):
    s = tp.tp_attn_local(None, 1, 128, 2, 128, FAKE, 512, 128, FAKE, 128, FAKE, 256)
    assert s == tp.TP_ERR_SHAPE and "k_col0" in tp.last_error()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(tp, "LIB_PATH", str(tmp_path / "libtp.so"))
    monkeypatch.setattr(tp, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        tp.lib()


def test_rmsnorm_gather_validation(L):
    f = tp.tp_rmsnorm_gather
    # args: stream, dt, n_slices, T, H, X, slice_stride, ldx, gamma, eps, Y, ldy, slice
    ok = dict(dt=tp.TP_BF16, n=4, T=64, H=512, X=FAKE, ss=16 * 512, ldx=512, g=FAKE, eps=1e-6, Y=FAKE, ldy=512, sl=-1)

    def call(**kw):
        a = {**ok, **kw}
        return f(None, a["dt"], a["n"], a["T"], a["H"], a["X"], a["ss"], a["ldx"], a["g"], a["eps"], a["Y"],
                 a["ldy"], a["sl"])
    assert call(T=0) == tp.TP_OK                        # empty: no HIP call
    assert call(T=66) == tp.TP_ERR_DIVISIBILITY         # T not a multiple of n_slices
    assert call(H=516) == tp.TP_ERR_ALIGN and "H=516" in tp.last_error()
    assert call(dt=tp.TP_F32, H=20000, ss=16 * 20000, ldx=20000, ldy=20000) == tp.TP_ERR_SHAPE
    assert "limit" in tp.last_error()
    assert call(H=16392, ss=16 * 16392, ldx=16392, ldy=16392) == tp.TP_ERR_SHAPE
    assert call(eps=-1.0) == tp.TP_ERR_SHAPE and "eps" in tp.last_error()
    assert call(eps=float("inf")) == tp.TP_ERR_SHAPE
    assert call(g=None) == tp.TP_ERR_NULL and "gamma" in tp.last_error()
    assert call(X=None) == tp.TP_ERR_NULL
    assert call(ldx=500) == tp.TP_ERR_SHAPE and "leading dimension" in tp.last_error()
    assert call(ss=15 * 512) == tp.TP_ERR_SHAPE and "overlap" in tp.last_error()
    assert call(ss=16 * 512 + 4) == tp.TP_ERR_ALIGN
    assert call(sl=4) == tp.TP_ERR_SHAPE
    assert call(Y=FAKE + 8) == tp.TP_ERR_ALIGN


# ------------------------------------------------------------ MLP backward
def _bwd(**kw):
    d = tp.MlpBwdDesc()
    d.dt, d.act = tp.TP_BF16, tp.TP_ACT_GELU
    d.T, d.H, d.F, d.N = 256, 512, 2048, 4
    d.shard_begin, d.shard_count = 0, 4
    d.X = d.A = d.a = d.B = d.dY = d.dX = d.dA = d.da = d.dB = d.db = FAKE
    d.n_slices, d.slice = 1, -1
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_mlp_backward_workspace_size_is_host_only(L):
    T, H, F, N = 256, 512, 2048, 4
    ws = tp.tp_mlp_backward_workspace_size
    # bf16, every contraction a multiple of 64: operands read as stored.  dX
    # partial slab, Z, dZ and act(Z) (the two-pass GELU kernel at H <= 2048
    # writes it), B^T for that kernel's second pass, and the column-sum
    # partials of the bias gradients (at most one row per 16 tokens)
    need = ws(_bwd())
    base = N * T * H * 4 + 3 * T * F * 2 + H * F * 2
    assert base < need <= base + 4 * (F + H) * (T // 16) + 2 * 256
    one = ws(_bwd(shard_count=1, shard_begin=3))
    assert one < need
    # with the forward's pre-activation supplied there is no recomputed Z and
    # no two-pass kernel (so no B^T); act(Z) is still written, by the dZ GEMM
    stored = ws(_bwd(Z=FAKE))
    assert stored == need - T * F * 2 - H * F * 2

    # a token count that is not a multiple of 64 (or fp32): the operands are
    # transposed first -- X, dY, act(Z), dZ, A and B -- and the bias
    # gradients are row sums of the transposes
    Tt = 264
    need_t = ws(_bwd(T=Tt))
    base_t = N * Tt * H * 4 + 3 * Tt * F * 2 + 2 * H * Tt * 2 + 2 * F * Tt * 2 + 2 * H * F * 2
    assert need_t >= base_t
    extra = need_t - base_t  # split-K partials of the weight gradients
    assert extra % (F * H * 4) == 0 and extra // (F * H * 4) in (0, 2, 4, 8, 16)
    assert ws(_bwd(T=Tt, Z=FAKE)) == need_t - 2 * Tt * F * 2
    f32 = ws(_bwd(dt=tp.TP_F32))
    assert f32 >= N * T * H * 4 + 2 * T * F * 4 + 2 * H * T * 4 + 2 * F * T * 4 + 2 * H * F * 4


@pytest.mark.parametrize("kw,status,needle", [
    (dict(F=2050), tp.TP_ERR_DIVISIBILITY, "not divisible by N=4"),
    (dict(T=260), tp.TP_ERR_ALIGN, "T=260 is not a multiple of 8"),
    (dict(dt=tp.TP_F32, act=tp.TP_ACT_SWIGLU, a=None, da=None), tp.TP_ERR_DTYPE, "SwiGLU backward is bf16-only"),
    (dict(act=tp.TP_ACT_SWIGLU), tp.TP_ERR_SHAPE, "a and da must be NULL"),
    (dict(act=9), tp.TP_ERR_DTYPE, "activation 9 unknown"),
    (dict(dY=None), tp.TP_ERR_NULL, "dY is NULL"),
    (dict(dA=None), tp.TP_ERR_NULL, "dA is NULL"),
    (dict(dX=None), tp.TP_ERR_NULL, "dX is NULL"),
    (dict(dB=FAKE + 4), tp.TP_ERR_ALIGN, "dB is not 16-byte aligned"),
    (dict(da=FAKE + 4), tp.TP_ERR_ALIGN, "da is not 16-byte aligned"),
    (dict(shard_begin=3, shard_count=2), tp.TP_ERR_SHAPE, "shard range"),
    (dict(Z=FAKE + 4, act=tp.TP_ACT_SWIGLU, a=None, da=None), tp.TP_ERR_ALIGN, "Z is not 16-byte aligned"),
    (dict(Z=FAKE + 4), tp.TP_ERR_ALIGN, "Z is not 16-byte aligned"),
    (dict(Hact=FAKE), tp.TP_ERR_SHAPE, "GELU and a stored Z only"),
    (dict(Hact=FAKE, Z=FAKE, act=tp.TP_ACT_NONE), tp.TP_ERR_SHAPE, "GELU and a stored Z only"),
    (dict(Hact=FAKE, Z=FAKE, act=tp.TP_ACT_SWIGLU, a=None, da=None), tp.TP_ERR_SHAPE, "GELU and a stored Z only"),
    (dict(Hact=FAKE + 8, Z=FAKE), tp.TP_ERR_ALIGN, "Hact is not 16-byte aligned"),
])
def test_mlp_backward_rejects_before_launch(L, kw, status, needle):
    d = _bwd(**kw)
    assert tp.tp_mlp_backward_workspace_size(d) == 0
    s = tp.tp_mlp_backward(None, d, FAKE, 1 << 40)
    assert s == status, tp.last_error()
    assert needle in tp.last_error()


def test_mlp_backward_swiglu_workspace(L):
    """SwiGLU keeps [gate | up] per shard (twice the columns of Z and dZ)
    plus SiLU(gate)*up, against GELU's dZ and GELU(Z) with a stored Z."""
    T, H, F, N = 256, 512, 2048, 4
    gelu = tp.tp_mlp_backward_workspace_size(_bwd(a=None, da=None, Z=FAKE))
    swi = tp.tp_mlp_backward_workspace_size(_bwd(act=tp.TP_ACT_SWIGLU, a=None, da=None))
    assert swi == gelu + 3 * T * F * 2
    # with the forward's [gate | up] pre-activation supplied, no recomputed Z slab
    swi_z = tp.tp_mlp_backward_workspace_size(_bwd(act=tp.TP_ACT_SWIGLU, a=None, da=None, Z=FAKE))
    assert swi_z == swi - T * 2 * F * 2


def test_mlp_backward_partial_range_needs_no_dx(L):
    d = _bwd(dX=None, shard_begin=1, shard_count=2)
    assert tp.tp_mlp_backward_workspace_size(d) > 0


def test_mlp_backward_small_workspace_and_empty_input(L):
    d = _bwd()
    need = tp.tp_mlp_backward_workspace_size(d)
    assert tp.tp_mlp_backward(None, d, FAKE, need - 1) == tp.TP_ERR_WORKSPACE
    assert tp.tp_mlp_backward(None, _bwd(T=0), None, 0) == tp.TP_OK


@pytest.mark.parametrize("T,H,F,N,c", [
    (16384, 512, 2048, 4, 4), (16384, 512, 2048, 4, 1), (16384, 12288, 49152, 8, 8),
    (2048, 520, 320, 8, 8), (4096, 256, 1024, 4, 4), (264, 136, 288, 4, 4), (1000, 64, 128, 2, 2),
])
def test_bench_split_rule_matches_library(L, T, H, F, N, c):
    """bench.py's copies of the backward's path and split-K rules (used to
    name kernels in profiler output) agree with the library's, read off the
    workspace."""
    import bench
    from tensor_transformer_layers_amd.configs import Workload

    d = _bwd(T=T, H=H, F=F, N=N, shard_count=c)
    Fc = F // N * c
    align = lambda x: (x + 255) // 256 * 256
    w = Workload(key=0, name="t", kind="mlp_gelu", dtype="bf16", batch=1, seq=T, H=H, F=F, N=N, sigma_bias=0.02)
    direct = bench.backward_direct(w)
    S = bench.backward_splits(T, Fc, H, direct)
    splitk = align(S * Fc * H * 4) if S > 1 else 0
    need = tp.tp_mlp_backward_workspace_size(d)
    if direct:
        # slab, Z, dZ, act(Z), B^T (two-pass kernel at H <= 2048), column-sum partials
        fused = H <= 2048
        base = align(N * T * H * 4) + 3 * align(T * Fc * 2) + (align(H * Fc * 2) if fused else 0)
        extra = need - base - splitk
        assert 0 < extra <= 4 * (Fc + H) * (T // 16) + 2 * 256
    else:
        fused_h = align(T * Fc * 2) if H <= 2048 else 0  # act(Z) of the two-pass GELU kernel
        base = align(N * T * H * 4) + 2 * align(T * Fc * 2) + fused_h + 2 * align(H * T * 2) \
            + 2 * align(Fc * T * 2) + 2 * align(H * Fc * 2)
        assert need - base == splitk


# ------------------------------------------------------------ vocab-parallel CE
def _vce(**kw):
    d = tp.VocabCeDesc()
    d.dt = tp.TP_BF16
    d.T, d.H, d.V, d.N = 256, 512, 1000, 8
    d.shard_begin, d.shard_count = 0, 8
    d.X = d.E = d.labels = d.loss = d.mean_loss = FAKE
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_vocab_padding_matches_oracle(L):
    from oracle import tp_oracle as O
    for V in (1, 7, 1000, 50257, 150000):
        for N in (1, 2, 3, 8):
            assert tp.tp_vocab_padded(V, N) == O.padded_vocab(V, N)[0]
    assert tp.tp_vocab_padded(0, 8) == 0


def test_vocab_ce_workspace_size_is_host_only(L):
    T, N = 256, 8
    cps = 2  # Vs = ceil(1000 / 8) = 125 -> 128 columns: two 64-column chunks
    align = lambda x: (x + 255) // 256 * 256
    assert tp.tp_vocab_ce_workspace_size(_vce()) == align(3 * N * cps * T * 4) + 3 * align(N * T * 4)
    assert tp.tp_vocab_ce_workspace_size(_vce(shard_count=1, loss=None)) == align(3 * cps * T * 4) + 3 * align(N * T * 4)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dt=tp.TP_F32), tp.TP_ERR_DTYPE, "bf16-only"),
    (dict(V=0), tp.TP_ERR_SHAPE, "V=0"),
    (dict(H=516), tp.TP_ERR_ALIGN, "H=516 is not a multiple of 8"),
    (dict(labels=None), tp.TP_ERR_NULL, "labels is NULL"),
    (dict(labels=FAKE + 2), tp.TP_ERR_ALIGN, "labels is not 4-byte aligned"),
    (dict(loss=None), tp.TP_ERR_NULL, "loss is NULL"),
    (dict(E=FAKE + 8), tp.TP_ERR_ALIGN, "E is not 16-byte aligned"),
    (dict(mean_loss=FAKE + 2), tp.TP_ERR_ALIGN, "mean_loss"),
    (dict(shard_begin=7, shard_count=2), tp.TP_ERR_SHAPE, "shard range"),
])
def test_vocab_ce_rejects_before_launch(L, kw, status, needle):
    d = _vce(**kw)
    assert tp.tp_vocab_ce_workspace_size(d) == 0
    assert tp.tp_vocab_ce_forward(None, d, FAKE, 1 << 40) == status, tp.last_error()
    assert needle in tp.last_error()


def test_vocab_ce_small_workspace_and_empty_input(L):
    d = _vce()
    need = tp.tp_vocab_ce_workspace_size(d)
    assert tp.tp_vocab_ce_forward(None, d, FAKE, need - 1) == tp.TP_ERR_WORKSPACE
    assert tp.tp_vocab_ce_forward(None, _vce(T=0), None, 0) == tp.TP_OK


def _vemb(**kw):
    d = tp.VocabEmbedDesc()
    d.dt = tp.TP_BF16
    d.T, d.H, d.V, d.N = 256, 512, 1000, 8
    d.shard_begin, d.shard_count = 0, 8
    d.ids = d.E = d.Y = FAKE
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_vocab_embed_workspace_size_is_host_only(L):
    align = lambda x: (x + 255) // 256 * 256
    # one partial per shard in the table's type
    for kw in ({}, dict(shard_count=1, Y=None)):
        assert tp.tp_vocab_embed_workspace_size(_vemb(**kw)) == align(8 * 256 * 512 * 2)
    assert tp.tp_vocab_embed_workspace_size(_vemb(dt=tp.TP_F32)) == align(8 * 256 * 512 * 4)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dt=7), tp.TP_ERR_DTYPE, ""),
    (dict(V=0), tp.TP_ERR_SHAPE, "V=0"),
    (dict(H=516), tp.TP_ERR_ALIGN, "H=516 is not a multiple of 8"),
    (dict(ids=None), tp.TP_ERR_NULL, "ids is NULL"),
    (dict(ids=FAKE + 2), tp.TP_ERR_ALIGN, "ids is not 4-byte aligned"),
    (dict(Y=None), tp.TP_ERR_NULL, "Y is NULL"),
    (dict(E=FAKE + 8), tp.TP_ERR_ALIGN, "E is not 16-byte aligned"),
    (dict(shard_begin=7, shard_count=2), tp.TP_ERR_SHAPE, "shard range"),
])
def test_vocab_embed_rejects_before_launch(L, kw, status, needle):
    d = _vemb(**kw)
    assert tp.tp_vocab_embed_workspace_size(d) == 0
    assert tp.tp_vocab_embed_forward(None, d, FAKE, 1 << 40) == status, tp.last_error()
    assert needle in tp.last_error()


def test_vocab_embed_small_workspace_and_empty_input(L):
    d = _vemb()
    need = tp.tp_vocab_embed_workspace_size(d)
    assert tp.tp_vocab_embed_forward(None, d, FAKE, need - 1) == tp.TP_ERR_WORKSPACE
    assert tp.tp_vocab_embed_forward(None, _vemb(T=0), None, 0) == tp.TP_OK
    # a partial shard range writes no Y, so Y may be NULL
    d = _vemb(shard_begin=2, shard_count=3, Y=None)
    assert tp.tp_vocab_embed_forward(None, d, FAKE, need - 1) == tp.TP_ERR_WORKSPACE


# ------------------------------------------------------------ overlapped forward
@pytest.mark.parametrize("kw,chunks,status,needle", [
    (dict(), 0, tp.TP_ERR_SHAPE, "chunks=0"),
    (dict(), 65, tp.TP_ERR_SHAPE, "chunks=65"),
    (dict(), 3, tp.TP_ERR_DIVISIBILITY, "do not split into 3 chunks"),
    (dict(shard_count=2), 2, tp.TP_ERR_SHAPE, "whole shard range"),
    (dict(n_slices=4, slice=1), 2, tp.TP_ERR_SHAPE, "slice must be -1"),
    (dict(F=2050), 2, tp.TP_ERR_DIVISIBILITY, "not divisible by N=4"),
])
def test_mlp_forward_overlap_rejects_before_launch(L, kw, chunks, status, needle):
    d = _mlp(**kw)
    s = tp.tp_mlp_forward_overlap(None, FAKE, d, chunks, FAKE, 1 << 40)
    assert s == status, tp.last_error()
    assert needle in tp.last_error()


def test_mlp_forward_overlap_needs_two_streams_and_workspace(L):
    d = _mlp()
    assert tp.tp_mlp_forward_overlap(FAKE, FAKE, d, 2, FAKE, 1 << 40) == tp.TP_ERR_SHAPE
    assert "stream2 must differ" in tp.last_error()
    need = tp.tp_mlp_workspace_size(d)
    assert tp.tp_mlp_forward_overlap(None, FAKE, d, 2, FAKE, need - 1) == tp.TP_ERR_WORKSPACE


# ------------------------------------------------------------ size limits
def test_leading_dimension_limit(L):
    """A 256-row tile of an operand is addressed with 32-bit byte offsets: a
    bf16 leading dimension of 2^23 is refused before any launch."""
    big = 1 << 23
    s = tp.tp_column_linear(None, tp.TP_BF16, tp.TP_ACT_NONE, 64, 64, 64, FAKE, big, FAKE, 64, None, FAKE, 64)
    assert s == tp.TP_ERR_SHAPE and "leading dimension" in tp.last_error()
    s = tp.tp_column_linear(None, tp.TP_BF16, tp.TP_ACT_NONE, 64, 64, 64, FAKE, big - 8, FAKE, 64, None, None, 64)
    assert s == tp.TP_ERR_NULL  # the largest accepted ld passes the size check


def test_attention_token_limit(L):
    d = tp.AttnDesc()
    d.dt = tp.TP_BF16
    d.batch, d.seq, d.hidden = 4097, 4096, 4096  # 16.8M tokens
    d.heads, d.head_dim, d.N, d.shard_begin, d.shard_count = 32, 128, 8, 0, 8
    d.X = d.Wqkv = d.Wo = d.Y = FAKE
    d.n_slices, d.slice = 1, -1
    assert tp.tp_attn_workspace_size(d) == 0
    assert "token limit" in tp.last_error()


def test_binding_has_every_helper_the_workloads_call():
    """workloads.py and bench.py reach the library through these helpers."""
    import inspect
    import re as _re

    from tensor_transformer_layers_amd import workloads

    src = inspect.getsource(workloads)
    called = set(_re.findall(r"\btp\.([a-z_0-9]+)\(", src))
    assert called, "no binding calls found"
    missing = sorted(n for n in called if not hasattr(tp, n))
    assert not missing, missing


def test_binding_rejects_mismatched_dtypes():
    """The ctypes layer checks dtypes before passing untyped pointers on."""
    import torch

    X = torch.zeros((16, 64), dtype=torch.bfloat16)
    A = torch.zeros((128, 64), dtype=torch.float32)
    B = torch.zeros((64, 128), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="A is torch.float32"):
        tp.mlp_backward(X, A, None, B, X.clone(), 2)
    with pytest.raises(TypeError, match="labels"):
        tp.vocab_ce_forward(X, torch.zeros((64, 64), dtype=torch.bfloat16), torch.zeros(16, dtype=torch.int64),
                            50, 2)
    with pytest.raises(TypeError, match="B is torch.float32"):
        tp.mlp_forward(X, B.t().contiguous(), None, B.float(), None, 2)
    with pytest.raises(TypeError, match="ids"):
        tp.vocab_embed_forward(torch.zeros(16, dtype=torch.int64), B, 50, 2)
    with pytest.raises(TypeError, match="Y is torch.float32"):
        tp.vocab_embed_forward(torch.zeros(16, dtype=torch.int32), B, 50, 2, Y=A)


def test_binding_rejects_wrong_shapes_before_the_c_call():
    """The C ABI sees only pointers and sizes, so a tensor smaller than the
    sizes it implies would be read or written out of bounds.  The binding
    checks every shape first (CPU tensors: nothing here reaches HIP)."""
    import torch

    bf = torch.bfloat16
    T, H, F, N = 16, 64, 128, 2
    X = torch.zeros((T, H), dtype=bf)
    A = torch.zeros((F, H), dtype=bf)
    B = torch.zeros((H, F), dtype=bf)
    # MLP: A must be [F x H] (GELU) or [2F x H] (SwiGLU), biases [F] and [H], Y [T x H]
    with pytest.raises(ValueError, match="A has shape"):
        tp.mlp_forward(X, A[:F - 8], None, B, None, N)
    with pytest.raises(ValueError, match="A has shape"):
        tp.mlp_forward(X, A, None, B, None, N, act=tp.TP_ACT_SWIGLU)
    with pytest.raises(ValueError, match="a has shape"):
        tp.mlp_forward(X, A, torch.zeros(F - 1, dtype=bf), B, None, N)
    with pytest.raises(ValueError, match="b has shape"):
        tp.mlp_forward(X, A, None, B, torch.zeros(H + 1, dtype=bf), N)
    with pytest.raises(ValueError, match="Y has shape"):
        tp.mlp_forward(X, A, None, B, None, N, Y=torch.zeros((T - 1, H), dtype=bf))
    with pytest.raises(ValueError, match="Y has shape"):  # one RS slice is T / n_slices rows
        tp.mlp_forward(X, A, None, B, None, N, Y=torch.zeros((T, H), dtype=bf), n_slices=2, slice=1)
    with pytest.raises(ValueError, match="B has shape"):
        tp.mlp_forward_overlap(X, A, None, B[:, :F - 8].contiguous()[:H - 8], None, N, 2, None)
    with pytest.raises(ValueError, match="contiguous"):
        tp.mlp_forward(X.t().contiguous().t(), A, None, B, None, N)
    # backward: dY [T x H], gradient buffers of the operands' shapes
    with pytest.raises(ValueError, match="dY has shape"):
        tp.mlp_backward(X, A, None, B, X[: T - 2], N)
    with pytest.raises(ValueError, match="dB has shape"):
        tp.mlp_backward(X, A, None, B, X.clone(), N, grads={"dB": torch.zeros((H, F - 8))})
    # vocab head: E must hold every padded row, labels 1-D int32 of length T
    Vp = tp.tp_vocab_padded(100, N)
    E = torch.zeros((Vp, H), dtype=bf)
    lab = torch.zeros(T, dtype=torch.int32)
    with pytest.raises(ValueError, match="E has shape"):
        tp.vocab_ce_forward(X, E[:100].contiguous(), lab, 100, N)
    with pytest.raises(ValueError, match="labels has shape"):
        tp.vocab_ce_forward(X, E, lab[: T - 1], 100, N)
    with pytest.raises(ValueError, match="labels has shape"):
        tp.vocab_ce_forward(X, E, lab.view(2, T // 2), 100, N)
    with pytest.raises(ValueError, match="labels must be contiguous"):
        tp.vocab_ce_forward(X, E, torch.zeros(2 * T, dtype=torch.int32)[::2], 100, N)
    # embedding: ids 1-D contiguous int32, E padded
    ids = torch.zeros(T, dtype=torch.int32)
    with pytest.raises(ValueError, match="ids must be 1-D"):
        tp.vocab_embed_forward(ids.view(2, T // 2), E, 100, N)
    with pytest.raises(ValueError, match="ids must be contiguous"):
        tp.vocab_embed_forward(torch.zeros(2 * T, dtype=torch.int32)[::2], E, 100, N)
    with pytest.raises(ValueError, match="E has shape"):
        tp.vocab_embed_forward(ids, E[: Vp - 8].contiguous(), 100, N)
    with pytest.raises(ValueError, match="Y has shape"):
        tp.vocab_embed_forward(ids, E, 100, N, Y=torch.zeros((T, H - 8), dtype=bf))
    # linear pieces, the reduction and the norm
    with pytest.raises(ValueError, match="W must be"):
        tp.column_linear(X, torch.zeros((F, H - 8), dtype=bf))
    with pytest.raises(ValueError, match="bias has shape"):
        tp.column_linear(X, A, bias=torch.zeros(F + 8, dtype=bf))
    with pytest.raises(ValueError, match="out has 15 rows"):
        tp.row_linear_partial(X, B.t().contiguous()[:, :H].contiguous(), out=torch.zeros((T - 1, F)))
    P = torch.zeros((N, T, H))
    with pytest.raises(ValueError, match="bias has shape"):
        tp.reduce_partials(P, bias=torch.zeros(H - 8, dtype=bf))
    with pytest.raises(ValueError, match="out has shape"):
        tp.reduce_partials(P, out=torch.zeros((T, H), dtype=bf), n_slices=2, slice=0)
    with pytest.raises(ValueError, match="n_parts"):
        tp.reduce_partials(P, n_parts=N + 1)
    with pytest.raises(ValueError, match="fp32"):
        tp.reduce_partials(P.to(bf))
    with pytest.raises(ValueError, match="gamma has shape"):
        tp.rmsnorm_gather(X, torch.zeros(H - 8, dtype=bf), 1e-6, 2)
    # attention: Wqkv [3*heads*128 x hidden], Wo [hidden x heads*128], X [batch*seq x hidden]
    hid, heads = 256, 2
    Xa = torch.zeros((2 * 8, hid), dtype=bf)
    Wqkv = torch.zeros((3 * heads * 128, hid), dtype=bf)
    Wo = torch.zeros((hid, heads * 128), dtype=bf)
    with pytest.raises(ValueError, match="batch\\*seq"):
        tp.attn_forward(Xa, Wqkv, Wo, None, 2, 9, heads, 2)
    with pytest.raises(ValueError, match="Wqkv has shape"):
        tp.attn_forward(Xa, Wqkv[:-8].contiguous(), Wo, None, 2, 8, heads, 2)
    with pytest.raises(ValueError, match="Wo has shape"):
        tp.attn_forward(Xa, Wqkv, Wo[:, :-8].contiguous(), None, 2, 8, heads, 2)
    with pytest.raises(ValueError, match="QK must be"):
        tp.attn_local(torch.zeros((16, 300), dtype=bf), 256, torch.zeros((256, 16), dtype=bf), 2, 8, 2)
    with pytest.raises(ValueError, match="Vt must be"):
        tp.attn_local(torch.zeros((16, 512), dtype=bf), 256, torch.zeros((256, 15), dtype=bf), 2, 8, 2)


def test_mlp_forward_noalloc_rejects_before_any_hip_call(L):
    """The allocation-free forward validates like tp_mlp_forward, then
    refuses a partial shard range and any problem whose workspace exceeds its
    static scratch -- all before touching the GPU."""
    assert tp.NOALLOC_SCRATCH_BYTES == 64 << 20
    hdr = open(HEADER).read()
    assert re.search(r"#define TP_NOALLOC_SCRATCH_BYTES \(\(size_t\)64 << 20\)", hdr)
    d = _mlp(F=2050)
    assert tp.tp_mlp_forward_noalloc(None, d) == tp.TP_ERR_DIVISIBILITY
    d = _mlp(shard_count=1)
    assert tp.tp_mlp_forward_noalloc(None, d) == tp.TP_ERR_SHAPE
    assert "whole shard range" in tp.last_error()
    d = _mlp(T=16384, H=512, F=2048, N=4, shard_count=4)  # 128 MiB of partials
    assert tp.tp_mlp_workspace_size(d) > tp.NOALLOC_SCRATCH_BYTES
    assert tp.tp_mlp_forward_noalloc(None, d) == tp.TP_ERR_WORKSPACE
    assert "static scratch" in tp.last_error()
    d = _mlp(T=0)
    assert tp.tp_mlp_forward_noalloc(None, d) == tp.TP_OK  # empty input: nothing to do


def test_layernorm_gather_validation(L):
    f = tp.tp_layernorm_gather
    ok = dict(dt=tp.TP_BF16, n=4, T=64, H=512, X=FAKE, ss=16 * 512, ldx=512, g=FAKE, b=FAKE, eps=1e-6, Y=FAKE,
              ldy=512, sl=-1)

    def call(**kw):
        a = {**ok, **kw}
        return f(None, a["dt"], a["n"], a["T"], a["H"], a["X"], a["ss"], a["ldx"], a["g"], a["b"], a["eps"], a["Y"],
                 a["ldy"], a["sl"])
    assert call(T=0) == tp.TP_OK
    assert call(T=66) == tp.TP_ERR_DIVISIBILITY
    assert call(H=516) == tp.TP_ERR_ALIGN
    assert call(H=16392, ss=16 * 16392, ldx=16392, ldy=16392) == tp.TP_ERR_SHAPE
    assert call(eps=-1.0) == tp.TP_ERR_SHAPE
    assert call(g=None) == tp.TP_ERR_NULL and "gamma" in tp.last_error()
    assert call(b=FAKE + 4) == tp.TP_ERR_ALIGN and "beta" in tp.last_error()
    assert call(sl=4) == tp.TP_ERR_SHAPE


def _nsplit(**kw):
    d = tp.NormSplitDesc()
    d.dt, d.kind = tp.TP_BF16, tp.TP_NORM_LAYER
    d.T, d.H, d.N, d.shard_begin, d.shard_count = 64, 4096, 8, 0, 8
    d.X = d.gamma = d.beta = d.Y = FAKE
    d.ldx = d.ldy = 4096
    d.eps = 1e-5
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_norm_hidden_split_workspace_and_validation(L):
    """The statistics slab is N x T x 2 fp32; every bad argument is refused
    before any HIP call."""
    assert tp.tp_norm_split_workspace_size(_nsplit()) == 8 * 64 * 2 * 4
    assert tp.tp_norm_split_workspace_size(_nsplit(T=0)) == 0

    def status(**kw):
        return tp.tp_norm_hidden_split(None, _nsplit(**kw), FAKE, 1 << 20)
    assert status(T=0) == tp.TP_OK
    assert status(H=4100) == tp.TP_ERR_DIVISIBILITY and "not divisible by N=8" in tp.last_error()
    assert status(H=8 * 12, ldx=96, ldy=96) == tp.TP_ERR_ALIGN and "shard width" in tp.last_error()
    assert status(kind=7) == tp.TP_ERR_DTYPE
    assert status(kind=tp.TP_NORM_RMS) == tp.TP_ERR_SHAPE and "beta" in tp.last_error()
    assert status(shard_begin=6, shard_count=3) == tp.TP_ERR_SHAPE
    assert status(N=1, shard_count=1, H=8 * 16392, ldx=8 * 16392, ldy=8 * 16392) == tp.TP_ERR_SHAPE
    assert status(eps=float("nan")) == tp.TP_ERR_SHAPE
    assert status(gamma=None) == tp.TP_ERR_NULL
    assert status(beta=FAKE + 2) == tp.TP_ERR_ALIGN
    assert status(Y=None) == tp.TP_ERR_NULL
    assert status(ldx=4000) == tp.TP_ERR_SHAPE
    assert tp.tp_norm_hidden_split(None, _nsplit(), FAKE, 100) == tp.TP_ERR_WORKSPACE
    assert tp.tp_norm_hidden_split(None, _nsplit(), None, 1 << 20) == tp.TP_ERR_WORKSPACE


def test_mlp_backward_slices_are_validated(L):
    ws = tp.tp_mlp_backward_workspace_size(_bwd())
    assert tp.tp_mlp_backward_workspace_size(_bwd(n_slices=4, slice=2)) == ws  # the fold's layout needs no space
    assert tp.tp_mlp_backward(None, _bwd(n_slices=3), FAKE, ws) == tp.TP_ERR_DIVISIBILITY
    assert tp.tp_mlp_backward(None, _bwd(n_slices=4, slice=4), FAKE, ws) == tp.TP_ERR_SHAPE
    assert tp.tp_mlp_backward(None, _bwd(n_slices=0), FAKE, ws) == tp.TP_ERR_SHAPE
