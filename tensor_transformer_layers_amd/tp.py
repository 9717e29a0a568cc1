"""ctypes binding of libtp.so (C ABI in include/tp.h).

Argument marshalling only: the raw functions below carry the C names and
signatures; the tensor helpers turn torch tensors into (pointer, shape, ld,
stream) and raise ``TPError`` on a non-OK status.  Every step of the path runs
in the HIP kernels of libtp; there is no fallback: if the library is missing,
``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtp.so")

TP_OK, TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_DIVISIBILITY, TP_ERR_DTYPE, TP_ERR_ALIGN, TP_ERR_WORKSPACE, TP_ERR_HIP = range(8)
TP_F32, TP_BF16 = 0, 1
TP_ACT_NONE, TP_ACT_GELU, TP_ACT_SWIGLU = 0, 1, 2
TP_NORM_RMS, TP_NORM_LAYER = 0, 1

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


class MlpDesc(ctypes.Structure):
    _fields_ = [
        ("dt", _int), ("act", _int),
        ("T", _i64), ("H", _i64), ("F", _i64),
        ("N", _int), ("shard_begin", _int), ("shard_count", _int),
        ("X", _vp), ("A", _vp), ("a", _vp), ("B", _vp), ("b", _vp),
        ("Y", _vp),
        ("n_slices", _int), ("slice", _int),
        ("Z", _vp),
        ("Hact", _vp),
    ]


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("dt", _int),
        ("batch", _i64), ("seq", _i64), ("hidden", _i64),
        ("heads", _int), ("head_dim", _int), ("N", _int), ("shard_begin", _int), ("shard_count", _int),
        ("X", _vp), ("Wqkv", _vp), ("Wo", _vp), ("bo", _vp),
        ("Y", _vp),
        ("n_slices", _int), ("slice", _int),
    ]


class MlpBwdDesc(ctypes.Structure):
    _fields_ = [
        ("dt", _int), ("act", _int),
        ("T", _i64), ("H", _i64), ("F", _i64),
        ("N", _int), ("shard_begin", _int), ("shard_count", _int),
        ("X", _vp), ("A", _vp), ("a", _vp), ("B", _vp), ("dY", _vp),
        ("dX", _vp), ("dA", _vp), ("da", _vp), ("dB", _vp), ("db", _vp),
        ("n_slices", _int), ("slice", _int),
        ("Z", _vp),
        ("Hact", _vp),
    ]


class NormSplitDesc(ctypes.Structure):
    _fields_ = [
        ("dt", _int), ("kind", _int),
        ("T", _i64), ("H", _i64),
        ("N", _int), ("shard_begin", _int), ("shard_count", _int),
        ("X", _vp), ("ldx", _i64), ("gamma", _vp), ("beta", _vp), ("eps", ctypes.c_float),
        ("Y", _vp), ("ldy", _i64),
    ]


class VocabCeDesc(ctypes.Structure):
    _fields_ = [
        ("dt", _int),
        ("T", _i64), ("H", _i64), ("V", _i64),
        ("N", _int), ("shard_begin", _int), ("shard_count", _int),
        ("X", _vp), ("E", _vp), ("labels", _vp), ("loss", _vp), ("mean_loss", _vp),
    ]


class VocabEmbedDesc(ctypes.Structure):
    _fields_ = [
        ("dt", _int),
        ("T", _i64), ("H", _i64), ("V", _i64),
        ("N", _int), ("shard_begin", _int), ("shard_count", _int),
        ("ids", _vp), ("E", _vp), ("Y", _vp),
    ]


_SIGS = {
    "tp_column_linear": (_int, [_vp, _int, _int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64]),
    "tp_row_linear_partial": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]),
    "tp_reduce_partials": (_int, [_vp, _int, _int, _i64, _i64, _vp, _i64, _vp, _vp, _int, _int]),
    "tp_rmsnorm_gather": (_int, [_vp, _int, _int, _i64, _i64, _vp, _i64, _i64, _vp, ctypes.c_float, _vp, _i64,
                                 _int]),
    "tp_layernorm_gather": (_int, [_vp, _int, _int, _i64, _i64, _vp, _i64, _i64, _vp, _vp, ctypes.c_float, _vp,
                                   _i64, _int]),
    "tp_norm_split_workspace_size": (_sz, [ctypes.POINTER(NormSplitDesc)]),
    "tp_norm_hidden_split": (_int, [_vp, ctypes.POINTER(NormSplitDesc), _vp, _sz]),
    "tp_mlp_workspace_size": (_sz, [ctypes.POINTER(MlpDesc)]),
    "tp_attn_workspace_size": (_sz, [ctypes.POINTER(AttnDesc)]),
    "tp_mlp_partials_offset": (_sz, [ctypes.POINTER(MlpDesc)]),
    "tp_attn_partials_offset": (_sz, [ctypes.POINTER(AttnDesc)]),
    "tp_mlp_forward": (_int, [_vp, ctypes.POINTER(MlpDesc), _vp, _sz]),
    "tp_mlp_forward_overlap": (_int, [_vp, _vp, ctypes.POINTER(MlpDesc), _int, _vp, _sz]),
    "tp_mlp_forward_noalloc": (_int, [_vp, ctypes.POINTER(MlpDesc)]),
    "tp_attn_forward": (_int, [_vp, ctypes.POINTER(AttnDesc), _vp, _sz]),
    "tp_mlp_backward_workspace_size": (_sz, [ctypes.POINTER(MlpBwdDesc)]),
    "tp_mlp_backward": (_int, [_vp, ctypes.POINTER(MlpBwdDesc), _vp, _sz]),
    "tp_vocab_padded": (_i64, [_i64, _int]),
    "tp_vocab_ce_workspace_size": (_sz, [ctypes.POINTER(VocabCeDesc)]),
    "tp_vocab_ce_forward": (_int, [_vp, ctypes.POINTER(VocabCeDesc), _vp, _sz]),
    "tp_vocab_embed_workspace_size": (_sz, [ctypes.POINTER(VocabEmbedDesc)]),
    "tp_vocab_embed_forward": (_int, [_vp, ctypes.POINTER(VocabEmbedDesc), _vp, _sz]),
    "tp_attn_local": (_int, [_vp, _i64, _i64, _int, _int, _vp, _i64, _i64, _vp, _i64, _vp, _i64]),
    "tp_timing_enable": (_int, [_int]),
    "tp_timing_read": (_int, [_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                              ctypes.POINTER(_i64)]),
    "tp_timing_reset": (None, []),
    "tp_status_string": (ctypes.c_char_p, [_int]),
    "tp_last_error": (ctypes.c_char_p, []),
    "tp_version": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libtp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -m tensor_transformer_layers_amd.build_lib)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class TPError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{status_string(status)}: {message}")


def status_string(s: int) -> str:
    return lib().tp_status_string(s).decode()


def last_error() -> str:
    return lib().tp_last_error().decode()


def check(status: int) -> None:
    if status != TP_OK:
        raise TPError(status, last_error())


# raw C entry points, same names and arguments as include/tp.h --------------
def tp_column_linear(*args) -> int:
    return lib().tp_column_linear(*args)


def tp_row_linear_partial(*args) -> int:
    return lib().tp_row_linear_partial(*args)


def tp_reduce_partials(*args) -> int:
    return lib().tp_reduce_partials(*args)


def tp_rmsnorm_gather(*args) -> int:
    return lib().tp_rmsnorm_gather(*args)


def tp_layernorm_gather(*args) -> int:
    return lib().tp_layernorm_gather(*args)


def tp_norm_split_workspace_size(desc: NormSplitDesc) -> int:
    return lib().tp_norm_split_workspace_size(ctypes.byref(desc))


def tp_norm_hidden_split(stream, desc: NormSplitDesc, ws, ws_bytes) -> int:
    return lib().tp_norm_hidden_split(stream, ctypes.byref(desc), ws, ws_bytes)


def tp_mlp_forward(stream, desc: MlpDesc, ws, ws_bytes) -> int:
    return lib().tp_mlp_forward(stream, ctypes.byref(desc), ws, ws_bytes)


def tp_mlp_forward_overlap(stream, stream2, desc: MlpDesc, chunks, ws, ws_bytes) -> int:
    return lib().tp_mlp_forward_overlap(stream, stream2, ctypes.byref(desc), chunks, ws, ws_bytes)


def tp_mlp_forward_noalloc(stream, desc: MlpDesc) -> int:
    return lib().tp_mlp_forward_noalloc(stream, ctypes.byref(desc))


# TP_NOALLOC_SCRATCH_BYTES of include/tp.h: the static scratch of tp_mlp_forward_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20


def tp_attn_forward(stream, desc: AttnDesc, ws, ws_bytes) -> int:
    return lib().tp_attn_forward(stream, ctypes.byref(desc), ws, ws_bytes)


def tp_mlp_backward(stream, desc: MlpBwdDesc, ws, ws_bytes) -> int:
    return lib().tp_mlp_backward(stream, ctypes.byref(desc), ws, ws_bytes)


def tp_mlp_backward_workspace_size(desc: MlpBwdDesc) -> int:
    return lib().tp_mlp_backward_workspace_size(ctypes.byref(desc))


def tp_vocab_padded(V: int, N: int) -> int:
    return lib().tp_vocab_padded(V, N)


def tp_vocab_ce_workspace_size(desc: VocabCeDesc) -> int:
    return lib().tp_vocab_ce_workspace_size(ctypes.byref(desc))


def tp_vocab_ce_forward(stream, desc: VocabCeDesc, ws, ws_bytes) -> int:
    return lib().tp_vocab_ce_forward(stream, ctypes.byref(desc), ws, ws_bytes)


def tp_vocab_embed_workspace_size(desc: VocabEmbedDesc) -> int:
    return lib().tp_vocab_embed_workspace_size(ctypes.byref(desc))


def tp_vocab_embed_forward(stream, desc: VocabEmbedDesc, ws, ws_bytes) -> int:
    return lib().tp_vocab_embed_forward(stream, ctypes.byref(desc), ws, ws_bytes)


def tp_attn_local(*args) -> int:
    return lib().tp_attn_local(*args)


def tp_mlp_workspace_size(desc: MlpDesc) -> int:
    return lib().tp_mlp_workspace_size(ctypes.byref(desc))


def tp_attn_workspace_size(desc: AttnDesc) -> int:
    return lib().tp_attn_workspace_size(ctypes.byref(desc))


def tp_timing_enable(on: int) -> int:
    return lib().tp_timing_enable(on)


def tp_timing_reset() -> None:
    lib().tp_timing_reset()


def tp_timing_read() -> dict:
    """{kernel name: (total ms, launches)} since the last reset."""
    L = lib()
    n = L.tp_timing_read(0, None, None, None)
    names = (ctypes.c_char_p * max(n, 1))()
    ms = (ctypes.c_double * max(n, 1))()
    cnt = (_i64 * max(n, 1))()
    n = L.tp_timing_read(n, names, ms, cnt)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(n)}


# torch tensor helpers (marshalling only) ------------------------------------
def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _same_dtype(ref, **named):
    """The C ABI takes untyped pointers: check here that every tensor has the
    dtype of ``ref`` (and is contiguous), so a mismatch fails loudly instead
    of being reinterpreted."""
    for name, t in named.items():
        if t is None:
            continue
        if t.dtype != ref.dtype:
            raise TypeError(f"{name} is {t.dtype}, expected {ref.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _expect(name, t, shape, dtype=None, device=None, contiguous=True):
    """The C ABI sees only pointers and the sizes the caller passes, so a
    tensor smaller than those sizes would be read or written out of bounds.
    Check here, before the C call, that ``t`` has exactly ``shape`` (a tuple
    of ints), the expected dtype and device, and, unless ``contiguous`` is
    False, a contiguous layout."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} is {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _rows_2d(name, t, cols, dtype=None, device=None):
    """``t`` is a 2-D row-major view with ``cols`` columns (a leading
    dimension of at least ``cols``, unit column stride)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dim() != 2 or t.shape[1] != cols or t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) < cols):
        raise ValueError(f"{name} must be a row-major [rows x {cols}] view, got shape {tuple(t.shape)} "
                         f"strides {tuple(t.stride())}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} is {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ld(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a row-major 2-D tensor (unit column stride)")
    return t.stride(0)


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def column_linear(X, W, bias=None, act=TP_ACT_GELU, out=None, stream=None):
    """Y_i = act(X W_i^T + bias_i); W is [Ns x K] ([2Ns x K] for SwiGLU)."""
    torch = _torch()
    if X.dim() != 2 or W.dim() != 2:
        raise ValueError("X and W must be 2-D")
    T, K = X.shape
    if act == TP_ACT_SWIGLU and W.shape[0] % 2:
        raise ValueError(f"SwiGLU W holds [gate | up] rows: an even row count, got {W.shape[0]}")
    Ns = W.shape[0] // 2 if act == TP_ACT_SWIGLU else W.shape[0]
    _rows_2d("X", X, K, device=X.device)
    _rows_2d("W", W, K, dtype=X.dtype, device=X.device)
    if bias is not None:
        _expect("bias", bias, (Ns,), X.dtype, X.device)
    if out is None:
        out = torch.empty((T, Ns), dtype=X.dtype, device=X.device)
    _rows_2d("out", out, Ns, dtype=X.dtype, device=X.device)
    if out.shape[0] != T:
        raise ValueError(f"out has {out.shape[0]} rows, expected {T}")
    check(tp_column_linear(_stream(stream), _dt(X), act, T, K, Ns, _ptr(X), _ld(X), _ptr(W), _ld(W),
                           _ptr(bias), _ptr(out), _ld(out)))
    return out


def row_linear_partial(X, W, out=None, stream=None):
    """P_i = X_i W_i^T in fp32; W is [Nout x Ks]."""
    torch = _torch()
    if X.dim() != 2 or W.dim() != 2:
        raise ValueError("X and W must be 2-D")
    T, Ks = X.shape
    Nout = W.shape[0]
    _rows_2d("X", X, Ks, device=X.device)
    _rows_2d("W", W, Ks, dtype=X.dtype, device=X.device)
    if out is None:
        out = torch.empty((T, Nout), dtype=torch.float32, device=X.device)
    _rows_2d("out", out, Nout, dtype=torch.float32, device=X.device)
    if out.shape[0] != T:
        raise ValueError(f"out has {out.shape[0]} rows, expected {T}")
    check(tp_row_linear_partial(_stream(stream), _dt(X), T, Ks, Nout, _ptr(X), _ld(X), _ptr(W), _ld(W),
                                _ptr(out), _ld(out)))
    return out


def reduce_partials(P, bias=None, out_dtype=None, n_slices=1, slice=-1, out=None, n_parts=None, stream=None):
    """Fixed-order sum of P[0..n) ([n x T x H] fp32) + bias, cast to out_dtype."""
    torch = _torch()
    if P.dim() != 3 or P.dtype != torch.float32:
        raise ValueError(f"P must be an fp32 [n x T x H] tensor, got {P.dtype} {tuple(P.shape)}")
    n, T, H = P.shape
    if not P[0].is_contiguous() or (n > 1 and P.stride(0) < T * H):
        raise ValueError("each partial P[k] must be a contiguous [T x H] block, the blocks not overlapping")
    if n_parts is not None and not 0 <= n_parts <= n:
        raise ValueError(f"n_parts = {n_parts} exceeds the {n} partials of P")
    n = n if n_parts is None else n_parts
    out_dtype = out_dtype or (bias.dtype if bias is not None else torch.bfloat16)
    if bias is not None:
        _expect("bias", bias, (H,), out_dtype, P.device)
    rows = T if slice < 0 else T // n_slices
    if out is None:
        out = torch.empty((rows, H), dtype=out_dtype, device=P.device)
    _expect("out", out, (rows, H), out_dtype, P.device)
    odt = TP_BF16 if out_dtype == torch.bfloat16 else TP_F32
    check(tp_reduce_partials(_stream(stream), odt, n, T, H, _ptr(P), P.stride(0), _ptr(bias), _ptr(out),
                             n_slices, slice))
    return out


def rmsnorm_gather(X, gamma, eps, n_slices, out=None, slice=-1, slice_stride=None, stream=None):
    """RMSNorm of each of the n_slices sequence slices of X ([T x H], slice r =
    rows r*T/n ..) into the gathered [T x H] buffer ``out`` (allocated when
    None).  With ``slice_stride`` the slices are read at X + r*slice_stride
    elements instead (X then holds the first slice's [T/n x H] rows)."""
    torch = _torch()
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    rows, H = X.shape
    _rows_2d("X", X, H, device=X.device)
    if slice_stride is not None and n_slices > 1 and slice_stride < rows * X.stride(0):
        raise ValueError(f"slice_stride {slice_stride} is shorter than one slice ({rows} rows)")
    T = rows if slice_stride is None else rows * n_slices
    stride = (T // n_slices) * X.stride(0) if slice_stride is None else slice_stride
    _expect("gamma", gamma, (H,), X.dtype, X.device)
    if out is None:
        out = torch.empty((T, H), dtype=X.dtype, device=X.device)
    _rows_2d("out", out, H, dtype=X.dtype, device=X.device)
    if out.shape[0] != T:
        raise ValueError(f"out has {out.shape[0]} rows, expected {T}")
    check(tp_rmsnorm_gather(_stream(stream), _dt(X), n_slices, T, H, _ptr(X), stride, _ld(X), _ptr(gamma),
                            float(eps), _ptr(out), _ld(out), slice))
    return out


def _check_mlp(X, A, a, B, b, act, Y=None, rows=None):
    """Shapes of the MLP operands in the ABI's storage: X [T x H]; A [F x H]
    ([2F x H] of per-shard [gate | up] blocks for SwiGLU); a [F] or None;
    B [H x F]; b [H] or None; Y [rows x H] when given.  Returns (T, H, F)."""
    if X.dim() != 2 or B.dim() != 2:
        raise ValueError("X and B must be 2-D")
    T, H = X.shape
    F = B.shape[1]
    _expect("X", X, (T, H))
    _expect("B", B, (H, F), X.dtype, X.device)
    _expect("A", A, ((2 * F if act == TP_ACT_SWIGLU else F), H), X.dtype, X.device)
    if a is not None:
        _expect("a", a, (F,), X.dtype, X.device)
    if b is not None:
        _expect("b", b, (H,), X.dtype, X.device)
    if Y is not None:
        _expect("Y", Y, (T if rows is None else rows, H), X.dtype, X.device)
    return T, H, F


def layernorm_gather(X, gamma, beta, eps, n_slices, out=None, slice=-1, slice_stride=None, stream=None):
    """LayerNorm of each of the n_slices sequence slices of X into the
    gathered [T x H] buffer ``out`` (arguments as rmsnorm_gather; beta [H]
    or None)."""
    torch = _torch()
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    rows, H = X.shape
    _rows_2d("X", X, H, device=X.device)
    if slice_stride is not None and n_slices > 1 and slice_stride < rows * X.stride(0):
        raise ValueError(f"slice_stride {slice_stride} is shorter than one slice ({rows} rows)")
    T = rows if slice_stride is None else rows * n_slices
    stride = (T // n_slices) * X.stride(0) if slice_stride is None else slice_stride
    _expect("gamma", gamma, (H,), X.dtype, X.device)
    if beta is not None:
        _expect("beta", beta, (H,), X.dtype, X.device)
    if out is None:
        out = torch.empty((T, H), dtype=X.dtype, device=X.device)
    _rows_2d("out", out, H, dtype=X.dtype, device=X.device)
    if out.shape[0] != T:
        raise ValueError(f"out has {out.shape[0]} rows, expected {T}")
    check(tp_layernorm_gather(_stream(stream), _dt(X), n_slices, T, H, _ptr(X), stride, _ld(X), _ptr(gamma),
                              _ptr(beta), float(eps), _ptr(out), _ld(out), slice))
    return out


def norm_hidden_split(X, gamma, beta, eps, N, kind=TP_NORM_LAYER, shard_begin=0, shard_count=None, out=None,
                      ws=None, stream=None):
    """Norm of X [T x H] split along hidden over N shards (shard i = columns
    [i H/N, (i+1) H/N)): local statistics, their fold in shard order, local
    scaling.  Returns (Y, workspace); the workspace holds the N x T x 2 fp32
    statistics slab (norm_split_stats)."""
    torch = _torch()
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    T, H = X.shape
    _rows_2d("X", X, H, device=X.device)
    _expect("gamma", gamma, (H,), X.dtype, X.device)
    if beta is not None:
        _expect("beta", beta, (H,), X.dtype, X.device)
    if out is None:
        out = torch.empty((T, H), dtype=X.dtype, device=X.device)
    _rows_2d("out", out, H, dtype=X.dtype, device=X.device)
    if out.shape[0] != T:
        raise ValueError(f"out has {out.shape[0]} rows, expected {T}")
    d = NormSplitDesc()
    d.dt, d.kind = _dt(X), kind
    d.T, d.H = T, H
    d.N, d.shard_begin = N, shard_begin
    d.shard_count = N if shard_count is None else shard_count
    d.X, d.ldx, d.gamma, d.beta, d.eps = _ptr(X), _ld(X), _ptr(gamma), _ptr(beta), float(eps)
    d.Y, d.ldy = _ptr(out), _ld(out)
    need = tp_norm_split_workspace_size(d)
    if need == 0:
        if T == 0:
            return out, ws
        raise TPError(TP_ERR_SHAPE, last_error())
    if ws is None or ws.numel() < need:
        ws = alloc_workspace(need, X.device)
    check(tp_norm_hidden_split(_stream(stream), d, _ptr(ws), ws.numel()))
    return out, ws


def norm_split_stats(ws, N, T):
    """View [N x T x 2] fp32 of the statistics slab of a hidden-split norm
    workspace (RMSNorm: sum of squares, 0; LayerNorm: mean, sum of squared
    deviations)."""
    torch = _torch()
    return ws[: N * T * 2 * 4].view(torch.float32).view(N, T, 2)


def mlp_desc(X, A, a, B, b, N, act, Y=None, shard_begin=0, shard_count=None, n_slices=1, slice=-1, F=None,
             Z=None, Hact=None):
    T, H = X.shape
    if F is None:
        F = B.shape[1]
    d = MlpDesc()
    d.dt = _dt(X)
    d.act = act
    d.T, d.H, d.F = T, H, F
    d.N = N
    d.shard_begin = shard_begin
    d.shard_count = N if shard_count is None else shard_count
    d.X, d.A, d.a, d.B, d.b = _ptr(X), _ptr(A), _ptr(a), _ptr(B), _ptr(b)
    d.Y = _ptr(Y)
    d.n_slices, d.slice = n_slices, slice
    d.Z = _ptr(Z)
    d.Hact = _ptr(Hact)
    return d


def alloc_workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def mlp_forward(X, A, a, B, b, N, act=TP_ACT_GELU, Y=None, ws=None, shard_begin=0, shard_count=None,
                n_slices=1, slice=-1, Z=None, Hact=None, stream=None):
    """Whole MLP sublayer; returns (Y, workspace).  Y is None for partial
    shard ranges (the partials are in the workspace slab).  Z ([T x F], or
    [T x 2F] for SwiGLU with shard i's [gate | up] in columns 2i*F/N..; X's
    dtype, bf16 only) or None: also write the range's pre-activation there,
    for mlp_backward(..., Z=Z).  Hact ([T x F], X's dtype, bf16 GELU or
    SwiGLU) or None: keep the range's activated intermediate there (the row
    layer's input), for mlp_backward(..., Hact=Hact)."""
    torch = _torch()
    _same_dtype(X, A=A, a=a, B=B, b=b, Y=Y)
    T, H, _ = _check_mlp(X, A, a, B, b, act)
    cnt = N if shard_count is None else shard_count
    rows = T if slice < 0 or n_slices < 1 else T // n_slices
    if Y is None and cnt == N:
        Y = torch.empty((rows, H), dtype=X.dtype, device=X.device)
    if Y is not None:
        _expect("Y", Y, (rows, H), X.dtype, X.device)
    if Z is not None:
        zw = B.shape[1] * (2 if act == TP_ACT_SWIGLU else 1)
        _expect("Z", Z, (T, zw), X.dtype, X.device)
    if Hact is not None:
        _expect("Hact", Hact, (T, B.shape[1]), X.dtype, X.device)
    d = mlp_desc(X, A, a, B, b, N, act, Y, shard_begin, cnt, n_slices, slice, Z=Z, Hact=Hact)
    need = tp_mlp_workspace_size(d)
    if need == 0:
        raise TPError(TP_ERR_SHAPE, last_error())
    if ws is None or ws.numel() < need:
        ws = alloc_workspace(need, X.device)
    check(tp_mlp_forward(_stream(stream), d, _ptr(ws), ws.numel()))
    return Y, ws


def mlp_forward_noalloc(X, A, a, B, b, N, act=TP_ACT_GELU, Y=None, n_slices=1, slice=-1, stream=None):
    """The whole MLP sublayer through tp_mlp_forward_noalloc: no workspace,
    the library's static per-GPU scratch instead (at most
    NOALLOC_SCRATCH_BYTES of workspace; calls that overlap on one GPU race).
    Allocates only Y, and only when it is None."""
    torch = _torch()
    _same_dtype(X, A=A, a=a, B=B, b=b, Y=Y)
    T, H, _ = _check_mlp(X, A, a, B, b, act)
    rows = T if slice < 0 or n_slices < 1 else T // n_slices
    if Y is None:
        Y = torch.empty((rows, H), dtype=X.dtype, device=X.device)
    _expect("Y", Y, (rows, H), X.dtype, X.device)
    d = mlp_desc(X, A, a, B, b, N, act, Y, 0, N, n_slices, slice)
    check(tp_mlp_forward_noalloc(_stream(stream), d))
    return Y


def mlp_backward(X, A, a, B, dY, N, act=TP_ACT_GELU, shard_begin=0, shard_count=None, grads=None, ws=None,
                 need_da=True, need_db=True, n_slices=1, slice=-1, Z=None, Hact=None, stream=None):
    """Backward of the MLP pair over a shard range; returns (grads, workspace).
    ``grads`` holds dX (bf16 [T x H], filled when the range covers all N
    shards; with n_slices > 1 and slice = r, rank r's reduce-scatter slice,
    [T/n_slices x H]), dA (fp32, A's shape: [F x H], or the [2F x H] fused
    blocks for SwiGLU), da (fp32 [F] or None; always None for SwiGLU), dB
    (fp32 [H x F]) and db (fp32 [H] or None); missing entries are allocated.
    Z: the forward's stored pre-activation ([T x F], SwiGLU [T x 2F]; X's
    dtype) to use instead of recomputing it, or None.  Hact: the forward's
    stored activation ([T x F], GELU with Z only), read for dB instead of
    GELU(Z), or None."""
    torch = _torch()
    _same_dtype(X, A=A, a=a, B=B, dY=dY)
    T, H, F = _check_mlp(X, A, a, B, None, act)
    _expect("dY", dY, (T, H), X.dtype, X.device)
    if act == TP_ACT_SWIGLU:
        need_da = False  # no column bias
    cnt = N if shard_count is None else shard_count
    g = dict(grads or {})
    dev = X.device
    f32 = torch.float32
    dx_rows = T if slice < 0 or n_slices < 1 else T // n_slices
    if "dX" not in g:
        g["dX"] = torch.empty((dx_rows, H), dtype=X.dtype, device=dev) if cnt == N else None
    if "dA" not in g:
        g["dA"] = torch.zeros(tuple(A.shape), dtype=f32, device=dev)
    if "da" not in g:
        g["da"] = torch.zeros((F,), dtype=f32, device=dev) if need_da else None
    if "dB" not in g:
        g["dB"] = torch.zeros((H, F), dtype=f32, device=dev)
    if "db" not in g:
        g["db"] = torch.zeros((H,), dtype=f32, device=dev) if need_db else None
    if g["dX"] is not None:
        _expect("dX", g["dX"], (dx_rows, H), X.dtype, dev)
    _expect("dA", g["dA"], tuple(A.shape), f32, dev)
    if g["da"] is not None:
        _expect("da", g["da"], (F,), f32, dev)
    _expect("dB", g["dB"], (H, F), f32, dev)
    if g["db"] is not None:
        _expect("db", g["db"], (H,), f32, dev)
    if Z is not None:
        _expect("Z", Z, (T, 2 * F if act == TP_ACT_SWIGLU else F), X.dtype, dev)
    if Hact is not None:
        _expect("Hact", Hact, (T, F), X.dtype, dev)
    d = MlpBwdDesc()
    d.dt = _dt(X)
    d.act = act
    d.T, d.H, d.F = T, H, F
    d.N, d.shard_begin, d.shard_count = N, shard_begin, cnt
    d.X, d.A, d.a, d.B, d.dY = _ptr(X), _ptr(A), _ptr(a), _ptr(B), _ptr(dY)
    d.dX, d.dA, d.da, d.dB, d.db = (_ptr(g[k]) for k in ("dX", "dA", "da", "dB", "db"))
    d.n_slices, d.slice = n_slices, slice
    d.Z = _ptr(Z)
    d.Hact = _ptr(Hact)
    need = tp_mlp_backward_workspace_size(d)
    if need == 0:
        if T == 0:
            return g, ws
        raise TPError(TP_ERR_SHAPE, last_error())
    if ws is None or ws.numel() < need:
        ws = alloc_workspace(need, dev)
    check(tp_mlp_backward(_stream(stream), d, _ptr(ws), ws.numel()))
    return g, ws


def vocab_ce_forward(X, E, labels, V, N, shard_begin=0, shard_count=None, loss=None, mean=None, ws=None,
                     stream=None):
    """Vocab-parallel output head and cross-entropy; returns (loss [T] fp32
    or None for a partial shard range, mean [1] fp32 or None, workspace).
    E must have tp_vocab_padded(V, N) rows; labels are int32."""
    torch = _torch()
    _same_dtype(X, E=E)
    if labels.dtype != torch.int32:
        raise TypeError(f"labels are {labels.dtype}, expected torch.int32")
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    T, H = X.shape
    if N >= 1 and V >= 1:
        # the head's product reads every padded row: E must hold them all
        _expect("E", E, (tp_vocab_padded(V, N), H), X.dtype, X.device)
    _expect("labels", labels, (T,), torch.int32, X.device)
    cnt = N if shard_count is None else shard_count
    if loss is None and cnt == N:
        loss = torch.empty((T,), dtype=torch.float32, device=X.device)
    if mean is None and cnt == N:
        mean = torch.empty((1,), dtype=torch.float32, device=X.device)
    if loss is not None:
        _expect("loss", loss, (T,), torch.float32, X.device)
    if mean is not None:
        _expect("mean", mean, (1,), torch.float32, X.device)
    d = VocabCeDesc()
    d.dt = _dt(X)
    d.T, d.H, d.V = T, H, V
    d.N, d.shard_begin, d.shard_count = N, shard_begin, cnt
    d.X, d.E, d.labels, d.loss, d.mean_loss = _ptr(X), _ptr(E), _ptr(labels), _ptr(loss), _ptr(mean)
    need = tp_vocab_ce_workspace_size(d)
    if need == 0:
        if T == 0:
            return loss, mean, ws
        raise TPError(TP_ERR_SHAPE, last_error())
    if ws is None or ws.numel() < need:
        ws = alloc_workspace(need, X.device)
    check(tp_vocab_ce_forward(_stream(stream), d, _ptr(ws), ws.numel()))
    return loss, mean, ws


def vocab_ce_stats(ws, N, T, Vs, shard_count):
    """Views (m, s, z), each [N x T] fp32, of the per-shard statistics in a
    vocab cross-entropy workspace (after the per-chunk statistics of the
    shard range)."""
    torch = _torch()
    align = lambda x: (x + 255) // 256 * 256
    cps = (Vs + 63) // 64
    off = align(3 * shard_count * cps * T * 4)
    step = align(N * T * 4)
    f = lambda o: ws[o:o + N * T * 4].view(torch.float32).view(N, T)
    return f(off), f(off + step), f(off + 2 * step)


def vocab_embed_forward(ids, E, V, N, shard_begin=0, shard_count=None, Y=None, ws=None, stream=None):
    """Vocab-parallel embedding lookup; returns (Y [T x H] or None for a
    partial shard range, workspace).  E must have tp_vocab_padded(V, N) rows;
    ids are int32.  The per-shard partials, in E's dtype, are slot i of the
    workspace (vocab_embed_partials)."""
    torch = _torch()
    if ids.dtype != torch.int32:
        raise TypeError(f"ids are {ids.dtype}, expected torch.int32")
    if ids.dim() != 1:
        raise ValueError(f"ids must be 1-D, got shape {tuple(ids.shape)}")
    if E.dim() != 2:
        raise ValueError("E must be 2-D")
    T, H = ids.shape[0], E.shape[1]
    _expect("ids", ids, (T,), torch.int32, E.device)
    if N >= 1 and V >= 1:
        _expect("E", E, (tp_vocab_padded(V, N), H), None, E.device)
    cnt = N if shard_count is None else shard_count
    if Y is None and cnt == N:
        Y = torch.empty((T, H), dtype=E.dtype, device=E.device)
    if Y is not None:
        _same_dtype(E, Y=Y)
        _expect("Y", Y, (T, H), E.dtype, E.device)
    d = VocabEmbedDesc()
    d.dt = _dt(E)
    d.T, d.H, d.V = T, H, V
    d.N, d.shard_begin, d.shard_count = N, shard_begin, cnt
    d.ids, d.E, d.Y = _ptr(ids), _ptr(E), _ptr(Y)
    need = tp_vocab_embed_workspace_size(d)
    if need == 0:
        if T == 0:
            check(tp_vocab_embed_forward(_stream(stream), d, None, 0))
            return Y, ws
        raise TPError(TP_ERR_SHAPE, last_error())
    if ws is None or ws.numel() < need:
        ws = alloc_workspace(need, E.device)
    check(tp_vocab_embed_forward(_stream(stream), d, _ptr(ws), ws.numel()))
    return Y, ws


def vocab_embed_partials(ws, N, T, H, dtype):
    """View [N x T x H] (``dtype``, the table's) of the per-shard partials in
    an embedding workspace."""
    es = _torch().empty((), dtype=dtype).element_size()
    return ws[:N * T * H * es].view(dtype).view(N, T, H)


def mlp_forward_overlap(X, A, a, B, b, N, chunks, stream2, act=TP_ACT_GELU, Y=None, ws=None, stream=None):
    """The whole MLP sublayer with the reduction of row block k overlapped
    with the products of block k+1 on ``stream2`` (a torch stream other than
    the current one); returns (Y, workspace)."""
    torch = _torch()
    _same_dtype(X, A=A, a=a, B=B, b=b, Y=Y)
    T, H, _ = _check_mlp(X, A, a, B, b, act)
    if Y is None:
        Y = torch.empty((T, H), dtype=X.dtype, device=X.device)
    _expect("Y", Y, (T, H), X.dtype, X.device)
    d = mlp_desc(X, A, a, B, b, N, act, Y)
    need = tp_mlp_workspace_size(d)
    if need == 0:
        if T == 0:
            return Y, ws
        raise TPError(TP_ERR_SHAPE, last_error())
    if ws is None or ws.numel() < need:
        ws = alloc_workspace(need, X.device)
    check(tp_mlp_forward_overlap(_stream(stream), stream2.cuda_stream, d, chunks, _ptr(ws), ws.numel()))
    return Y, ws


def mlp_partials(ws, N, T, H):
    """View of the fp32 partial slab at the start of an MLP/attention workspace."""
    torch = _torch()
    return ws[: N * T * H * 4].view(torch.float32).view(N, T, H)


def attn_desc(X, Wqkv, Wo, bo, batch, seq, heads, N, Y=None, shard_begin=0, shard_count=None, n_slices=1,
              slice=-1, head_dim=128):
    d = AttnDesc()
    d.dt = _dt(X)
    d.batch, d.seq, d.hidden = batch, seq, X.shape[1]
    d.heads, d.head_dim, d.N = heads, head_dim, N
    d.shard_begin = shard_begin
    d.shard_count = N if shard_count is None else shard_count
    d.X, d.Wqkv, d.Wo, d.bo = _ptr(X), _ptr(Wqkv), _ptr(Wo), _ptr(bo)
    d.Y = _ptr(Y)
    d.n_slices, d.slice = n_slices, slice
    return d


def attn_forward(X, Wqkv, Wo, bo, batch, seq, heads, N, Y=None, ws=None, shard_begin=0, shard_count=None,
                 n_slices=1, slice=-1, stream=None):
    torch = _torch()
    _same_dtype(X, Wqkv=Wqkv, Wo=Wo, bo=bo, Y=Y)
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    T, Hd = X.shape
    if T != batch * seq:
        raise ValueError(f"X has {T} rows, expected batch*seq = {batch * seq}")
    _expect("X", X, (T, Hd))
    _expect("Wqkv", Wqkv, (3 * heads * 128, Hd), X.dtype, X.device)
    _expect("Wo", Wo, (Hd, heads * 128), X.dtype, X.device)
    if bo is not None:
        _expect("bo", bo, (Hd,), X.dtype, X.device)
    cnt = N if shard_count is None else shard_count
    rows = T if slice < 0 or n_slices < 1 else T // n_slices
    if Y is None and cnt == N:
        Y = torch.empty((rows, Hd), dtype=X.dtype, device=X.device)
    if Y is not None:
        _expect("Y", Y, (rows, Hd), X.dtype, X.device)
    d = attn_desc(X, Wqkv, Wo, bo, batch, seq, heads, N, Y, shard_begin, cnt, n_slices, slice)
    need = tp_attn_workspace_size(d)
    if need == 0:
        raise TPError(TP_ERR_SHAPE, last_error())
    if ws is None or ws.numel() < need:
        ws = alloc_workspace(need, X.device)
    check(tp_attn_forward(_stream(stream), d, _ptr(ws), ws.numel()))
    return Y, ws


def attn_local(QK, k_col0, Vt, batch, seq, heads, out=None, stream=None):
    torch = _torch()
    T = batch * seq
    if QK.dim() != 2 or Vt.dim() != 2:
        raise ValueError("QK and Vt must be 2-D")
    _rows_2d("QK", QK, QK.shape[1], device=QK.device)
    _rows_2d("Vt", Vt, Vt.shape[1], dtype=QK.dtype, device=QK.device)
    if QK.shape[0] != T or k_col0 < heads * 128 or QK.shape[1] < k_col0 + heads * 128:
        raise ValueError(f"QK must be [batch*seq = {T} x >= k_col0 + heads*128] with Q in columns "
                         f"[0, heads*128) and K from column k_col0 >= heads*128, got {tuple(QK.shape)}, "
                         f"k_col0 = {k_col0}")
    if Vt.shape[0] != heads * 128 or Vt.shape[1] < T:
        raise ValueError(f"Vt must be [heads*128 = {heads * 128} x >= {T}], got {tuple(Vt.shape)}")
    if out is None:
        out = torch.empty((T, heads * 128), dtype=QK.dtype, device=QK.device)
    _rows_2d("out", out, heads * 128, dtype=QK.dtype, device=QK.device)
    if out.shape[0] != T:
        raise ValueError(f"out has {out.shape[0]} rows, expected {T}")
    check(tp_attn_local(_stream(stream), batch, seq, heads, 128, _ptr(QK), _ld(QK), k_col0, _ptr(Vt), _ld(Vt),
                        _ptr(out), _ld(out)))
    return out
