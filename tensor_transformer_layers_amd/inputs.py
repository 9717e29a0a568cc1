"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no arithmetic of the method: it only draws normal numbers
and rounds them to the workload's storage dtype.  Both the CPU oracle and the
GPU path receive exactly the arrays returned here.

Recipe (one workload, seed s):
  * tensor j of the workload gets its own stream,
    ``SeedSequence(s).spawn(n_tensors)[j]``; the tensor's flat element range
    is cut into fixed 2**22-element chunks, chunk c drawing from
    ``child_j.spawn(n_chunks)[c]`` (so the values do not depend on the number
    of threads used to fill them);
  * values are ``standard_normal(float32) * sigma`` (sigma is a standard
    deviation), then rounded to bf16 with round-to-nearest-even for bf16
    workloads and returned widened back to float32 (exact), so one float32
    array carries the value both sides use.

Weights are drawn directly in [out x in] storage (the layout of the weight
chunks in the pages' PyTorch listing); the math-layout matrix is its
transpose.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Workload

CHUNK = 1 << 22

# tensor order per workload kind (fixed: it defines each tensor's stream)
TENSORS = {
    "mlp_gelu": ["X", "A", "a", "B", "b"],
    "mlp_swiglu": ["X", "Wg", "Wu", "Wd"],
    "attn": ["X", "Wq", "Wk", "Wv", "Wo"],
    "vocab_ce": ["X", "E"],
    "vocab_embed": ["E"],
    "norm_split_layer": ["X", "g", "b"],
    "norm_split_rms": ["X", "g", "b"],
}


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def draw(seed_seq: np.random.SeedSequence, shape, sigma: float) -> np.ndarray:
    """N(0, sigma^2) float32 array of ``shape`` from ``seed_seq``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, -(-n // CHUNK))
    kids = seed_seq.spawn(nchunks)

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        np.random.default_rng(kids[c]).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out.reshape(shape)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (bf16: RNE) and return them
    as float32 again (exactly representable)."""
    if dtype == "f32":
        return x
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(x)
        return t.to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


def shapes(w: Workload) -> dict:
    """Storage shapes ([out x in] for weights) of every input tensor."""
    T, H, F = w.T, w.H, w.F
    if w.kind == "mlp_gelu":
        return {"X": (T, H), "A": (F, H), "a": (F,), "B": (H, F), "b": (H,)}
    if w.kind == "mlp_swiglu":
        return {"X": (T, H), "Wg": (F, H), "Wu": (F, H), "Wd": (H, F)}
    if w.kind == "attn":
        return {"X": (T, H), "Wq": (H, H), "Wk": (H, H), "Wv": (H, H), "Wo": (H, H)}
    if w.kind == "vocab_ce":  # E: the output head over the real vocab, [V x H]
        return {"X": (T, H), "E": (F, H)}
    if w.kind == "vocab_embed":  # E: the embedding table over the real vocab, [V x H]
        return {"E": (F, H)}
    if w.kind.startswith("norm_split"):  # the norm's input, gain and shift
        return {"X": (T, H), "g": (H,), "b": (H,)}
    raise ValueError(w.kind)


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """All inputs of workload ``w`` as float32 numpy arrays (values already
    rounded to ``w.dtype``).  Weights are [out x in]; biases are absent when
    ``w.sigma_bias`` is None."""
    seed = w.seed if seed is None else seed
    names = TENSORS[w.kind]
    kids = np.random.SeedSequence(seed).spawn(len(names))
    shp = shapes(w)
    out = {}
    for name, ss in zip(names, kids):
        if name == "g":  # a norm gain: 1 + N(0, 0.1^2)
            g = np.float32(1.0) + draw(ss, shp[name], 0.1)
            out[name] = round_to_dtype(g.astype(np.float32), w.dtype)
            continue
        if name in ("a", "b"):
            if w.sigma_bias is None:
                out[name] = None
                continue
            sigma = w.sigma_bias
        elif name == "X":
            sigma = w.sigma_x
        else:
            sigma = w.sigma_w
        out[name] = round_to_dtype(draw(ss, shp[name], sigma), w.dtype)
    if w.kind == "vocab_ce":
        out["labels"] = labels(w) if seed == w.seed else \
            np.random.default_rng(np.random.SeedSequence([seed, 3])).integers(0, w.F, size=w.T).astype(np.int32)
    if w.kind == "vocab_embed":
        out["ids"] = token_ids(w, seed)
    return out


def make_x(w: Workload) -> np.ndarray:
    """Only the input X of workload ``w`` (the same values make_inputs draws)."""
    kids = np.random.SeedSequence(w.seed).spawn(len(TENSORS[w.kind]))
    return round_to_dtype(draw(kids[0], shapes(w)["X"], w.sigma_x), w.dtype)


def sample_rows(T: int, count: int, seed: int, must=()) -> np.ndarray:
    """Sorted, distinct token rows: ``must`` plus seeded uniform picks."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x5A3]))
    rows = set(int(r) for r in must if 0 <= r < T)
    count = min(count, T)
    while len(rows) < count:
        rows.update(int(r) for r in rng.integers(0, T, size=count - len(rows)))
    return np.array(sorted(rows), dtype=np.int64)


# Sequence-parallel entry side (RMSNorm before the column linear).  The pages
# give neither eps nor gain values: eps = 1e-6 and a gain of 1 + N(0, 0.1^2),
# rounded to the workload dtype, drawn from its own stream of the seed.
NORM_EPS = 1e-6
NORM_GAIN_RECIPE = "1 + N(0, 0.1^2) per feature, rounded to the workload dtype, SeedSequence([seed, 1])"


NORM_SHIFT_RECIPE = "N(0, 0.1^2) per feature, rounded to the workload dtype, SeedSequence([seed, 5])"


def norm_shift(w: Workload) -> np.ndarray:
    """The LayerNorm shift [H] of workload w's entry side (recipe above)."""
    return round_to_dtype(draw(np.random.SeedSequence([w.seed, 5]), (w.H,), 0.1), w.dtype)


def norm_gain(w: Workload) -> np.ndarray:
    """The RMSNorm gain [H] of workload w (recipe above)."""
    g = np.float32(1.0) + draw(np.random.SeedSequence([w.seed, 1]), (w.H,), 0.1)
    return round_to_dtype(g.astype(np.float32), w.dtype)


# Backward of the MLP pair: the upstream gradient dY [T x H] of the sublayer
# output.  The pages fix no values for it: N(0, 1) per element, rounded to the
# workload dtype, drawn from its own stream of the seed.
GRAD_RECIPE = "N(0, 1) per element of dY [T x H], rounded to the workload dtype, SeedSequence([seed, 2])"


def grad_output(w: Workload) -> np.ndarray:
    """The upstream gradient dY [T x H] of workload w (recipe above)."""
    return round_to_dtype(draw(np.random.SeedSequence([w.seed, 2]), (w.T, w.H), 1.0), w.dtype)


# Vocab-parallel cross-entropy: the target token of each row, uniform over the
# real vocab, from its own stream of the seed.
LABEL_RECIPE = "uniform integers in [0, V), SeedSequence([seed, 3])"


def labels(w: Workload) -> np.ndarray:
    """Target ids [T] (int32) of workload w (recipe above)."""
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 3]))
    return rng.integers(0, w.F, size=w.T).astype(np.int32)


# Vocab-parallel embedding: the token id of each row, uniform over the real
# vocab, from its own stream of the seed.
ID_RECIPE = "uniform integers in [0, V), SeedSequence([seed, 4])"


def token_ids(w: Workload, seed: int | None = None) -> np.ndarray:
    """Token ids [T] (int32) of workload w (recipe above)."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(np.random.SeedSequence([seed, 4]))
    return rng.integers(0, w.F, size=w.T).astype(np.int32)
