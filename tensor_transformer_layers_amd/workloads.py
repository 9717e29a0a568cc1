"""Device-side set-up and one forward pass of a workload through libtp.

Set-up (done once, outside any timed region) uploads the generator's arrays
and arranges weights in the layout the C ABI takes: per-shard fused
[gate | up] blocks for SwiGLU, per-shard [Q | K | V] row blocks of the shard's
heads for attention.  The forward pass itself is one call into libtp.
"""
from __future__ import annotations

import numpy as np

from . import tp
from .configs import Workload


def _torch():
    import torch
    return torch


def to_device(x, dtype, device="cuda"):
    torch = _torch()
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dtype)


def device_inputs(w: Workload, host: dict, device="cuda") -> dict:
    torch = _torch()
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = {}
    if w.kind == "mlp_gelu":
        for k in ("X", "A", "a", "B", "b"):
            d[k] = to_device(host[k], dt, device)
    elif w.kind == "mlp_swiglu":
        Fs = w.F // w.N
        d["X"] = to_device(host["X"], dt, device)
        Wg = to_device(host["Wg"], dt, device)
        Wu = to_device(host["Wu"], dt, device)
        # shard i: rows [gate i*Fs..(i+1)*Fs | up i*Fs..(i+1)*Fs]
        d["A"] = torch.cat([Wg.view(w.N, Fs, w.H), Wu.view(w.N, Fs, w.H)], dim=1).reshape(w.N * 2 * Fs, w.H).contiguous()
        del Wg, Wu
        d["a"] = None
        d["B"] = to_device(host["Wd"], dt, device)
        d["b"] = None
    elif w.kind == "attn":
        hd = (w.heads // w.N) * w.head_dim
        d["X"] = to_device(host["X"], dt, device)
        Wq, Wk, Wv = (to_device(host[k], dt, device).view(w.N, hd, w.H) for k in ("Wq", "Wk", "Wv"))
        d["Wqkv"] = torch.cat([Wq, Wk, Wv], dim=1).reshape(w.N * 3 * hd, w.H).contiguous()
        del Wq, Wk, Wv
        d["Wo"] = to_device(host["Wo"], dt, device)
        d["bo"] = None
    elif w.kind == "vocab_ce":
        d["X"] = to_device(host["X"], dt, device)
        # padding rows (zeros) added on the host: one upload, no device copy
        Vp = tp.tp_vocab_padded(w.F, w.N)
        E = np.zeros((Vp, w.H), dtype=np.float32)
        E[: w.F] = host["E"]
        d["E"] = to_device(E, dt, device)
        del E
        d["labels"] = torch.from_numpy(np.ascontiguousarray(host["labels"])).to(device)
    elif w.kind.startswith("norm_split"):
        for k in ("X", "g", "b"):
            d[k] = to_device(host[k], dt, device)
    elif w.kind == "vocab_embed":
        Vp = tp.tp_vocab_padded(w.F, w.N)
        E = np.zeros((Vp, w.H), dtype=np.float32)
        E[: w.F] = host["E"]
        d["E"] = to_device(E, dt, device)
        del E
        d["ids"] = torch.from_numpy(np.ascontiguousarray(host["ids"])).to(device)
    else:
        raise ValueError(w.kind)
    return d


def act_of(w: Workload) -> int:
    return tp.TP_ACT_SWIGLU if w.kind == "mlp_swiglu" else tp.TP_ACT_GELU


def forward(w: Workload, d: dict, Y=None, ws=None, shard_begin=0, shard_count=None, slice=-1, stream=None):
    """One pass of the sublayer over shards [shard_begin, shard_begin+count).
    For the vocab cross-entropy, Y is the per-token loss; for the embedding,
    the looked-up rows."""
    if w.kind.startswith("norm_split"):
        from .inputs import NORM_EPS
        kind = tp.TP_NORM_LAYER if w.kind == "norm_split_layer" else tp.TP_NORM_RMS
        return tp.norm_hidden_split(d["X"], d["g"], d["b"], NORM_EPS, w.N, kind=kind, shard_begin=shard_begin,
                                    shard_count=shard_count, out=Y, ws=ws, stream=stream)
    if w.kind == "vocab_embed":
        return tp.vocab_embed_forward(d["ids"], d["E"], w.F, w.N, shard_begin=shard_begin,
                                      shard_count=shard_count, Y=Y, ws=ws, stream=stream)
    if w.kind == "vocab_ce":
        loss, mean, ws = tp.vocab_ce_forward(d["X"], d["E"], d["labels"], w.F, w.N, shard_begin=shard_begin,
                                             shard_count=shard_count, loss=Y, mean=d.get("mean"), ws=ws,
                                             stream=stream)
        if mean is not None:
            d["mean"] = mean
        return loss, ws
    if w.kind == "attn":
        return tp.attn_forward(d["X"], d["Wqkv"], d["Wo"], d["bo"], w.batch, w.seq, w.heads, w.N, Y=Y, ws=ws,
                               shard_begin=shard_begin, shard_count=shard_count, n_slices=w.n_slices,
                               slice=slice, stream=stream)
    return tp.mlp_forward(d["X"], d["A"], d["a"], d["B"], d["b"], w.N, act=act_of(w), Y=Y, ws=ws,
                          shard_begin=shard_begin, shard_count=shard_count, n_slices=w.n_slices, slice=slice,
                          stream=stream)


def forward_overlap(w: Workload, d: dict, chunks, stream2, Y=None, ws=None, stream=None):
    """All shards of an MLP sublayer with the reduction of each row block
    overlapped with the next block's products on ``stream2``."""
    if w.kind not in ("mlp_gelu", "mlp_swiglu"):
        raise ValueError(f"the overlapped forward is built for the MLP sublayers, not {w.kind}")
    return tp.mlp_forward_overlap(d["X"], d["A"], d["a"], d["B"], d["b"], w.N, chunks, stream2, act=act_of(w), Y=Y,
                                  ws=ws, stream=stream)


def reduce_slab(w: Workload, d: dict, ws, Y=None, slice=-1, stream=None):
    """The reduction step alone over the partial slab of a workspace."""
    torch = _torch()
    P = tp.mlp_partials(ws, w.N, w.T, w.H)
    bias = d.get("b") if w.kind != "attn" else d.get("bo")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return tp.reduce_partials(P, bias, out_dtype=dt, n_slices=w.n_slices, slice=slice, out=Y, stream=stream)


def backward(w: Workload, d: dict, dY, grads=None, ws=None, shard_begin=0, shard_count=None, Z=None, Hact=None,
             stream=None):
    """One backward pass of the MLP sublayer (GELU or SwiGLU) over a shard
    range; Z: the forward's stored pre-activation ([T x F]) or None to
    recompute it; Hact: the forward's stored activation (GELU, with Z) or
    None."""
    if w.kind not in ("mlp_gelu", "mlp_swiglu"):
        raise ValueError(f"the backward is built for the MLP sublayers, not {w.kind}")
    return tp.mlp_backward(d["X"], d["A"], d["a"], d["B"], dY, w.N, act=act_of(w),
                           shard_begin=shard_begin, shard_count=shard_count, grads=grads, ws=ws,
                           need_da=d["a"] is not None, need_db=d["b"] is not None, Z=Z, Hact=Hact, stream=stream)
