#!/usr/bin/env python3
"""Throughput of the tensor-parallel linear pair on one MI355X.

One step = one forward pass of the whole sublayer over one batch of seeded
synthetic input: the column GEMM with its fused activation for every shard,
the row partial of every shard, and the fixed-order reduction of the N
partials (the all-reduce stand-in), or, for the attention workload, QKV
projection, causal attention, output projection and reduction.  All N shards
run on the one GPU.  ``--share rank`` times one rank's share instead: shard 0
plus the reduction of a partial slab holding the other shards' partials (the
reduce-scatter slice of rank 0 for the sequence-parallel workload).

Prints ONE JSON line (rank 0): throughput in TFLOP/s (algorithmic FLOP of
the timed work / time), the roofline of the dominant kernel measured with HIP
events around its launches, and the fp64 CPU oracle timed on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s per sharded TP MLP/attn layer fwd on 1 GPU; % of bf16 MFMA peak"
METRIC_BWD = "TFLOP/s per sharded TP MLP layer bwd on 1 GPU; % of bf16 MFMA peak"
METRIC_VOCAB = "TFLOP/s of the vocab-parallel output head + cross-entropy fwd on 1 GPU; % of bf16 MFMA peak"
METRIC_EMBED = "GB/s (algorithmic bytes) of the vocab-parallel embedding lookup fwd on 1 GPU; % of HBM peak"
METRIC_NORM = "GB/s (algorithmic bytes) of the hidden-split norm (local statistics, their fold, local scaling) on 1 GPU; % of HBM peak"
PEAK_BF16 = 2.5e15     # dense MFMA, bf16
PEAK_F32 = 157.3e12    # dense MFMA, fp32
PEAK_HBM = 8.0e12      # bytes/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_work(w, name, shards_per_launch, rows_reduced, bmode=None):
    """Algorithmic (flops, bytes) of ONE launch of kernel `name` for workload w:
    every input read once and every output written once.  bmode: the
    backward variant ("stored" or "recompute") for the backward's kernels."""
    es = 2 if w.dtype == "bf16" else 4
    T, H, N = w.T, w.H, w.N
    c = shards_per_launch
    if w.kind in ("mlp_gelu", "mlp_swiglu"):
        Fs = w.F // N
        cols = 2 * Fs if w.kind == "mlp_swiglu" else Fs
        if name == "mlp_column_gemm":
            return 2.0 * T * H * cols * c, es * (T * H + c * cols * H + c * T * Fs) + (es * c * Fs if w.sigma_bias else 0)
        if name == "mlp_row_gemm":
            return 2.0 * T * Fs * H * c, es * (c * T * Fs + c * H * Fs) + 4 * c * T * H
        if name == "mlp_fused":  # column + activation + row partial; the intermediate stays on chip
            return (4.0 * T * H * Fs * c,
                    es * (T * H + 2 * c * Fs * H) + (es * c * Fs if w.sigma_bias else 0) + 4 * c * T * H)
    else:
        hl = w.heads // N
        hd = hl * w.head_dim
        if name == "attn_qk_gemm":
            return 2.0 * T * H * 2 * hd * c, es * (T * H + c * 2 * hd * H + c * T * 2 * hd)
        if name == "attn_vt_gemm":
            return 2.0 * T * H * hd * c, es * (T * H + c * hd * H + c * T * hd)
        if name == "attn_core":
            return (w.batch * hl * c * 4.0 * w.head_dim * w.seq * (w.seq + 1) / 2, es * 4 * c * T * hd)
        if name == "attn_out_gemm":
            return 2.0 * T * hd * H * c, es * (c * T * hd + c * H * hd) + 4 * c * T * H
    if name.startswith("bwd_"):
        return backward_kernel_work(w, name, shards_per_launch, bmode)
    if w.kind == "vocab_ce":
        c = shards_per_launch
        Vs = -(-w.F // N)
        Vs = -(-Vs // 8) * 8
        cps = -(-Vs // 64)
        if name == "vocab_logits_gemm":  # padded rows are computed too; the FLOP count is the real vocab's.
            # The epilogue writes 3 statistics per (token, 64-column chunk) instead of the logits.
            return 2.0 * T * H * w.F * c / N, es * (T * H + c * Vs * H) + 4 * T + 12 * c * cps * T
        if name == "vocab_ce_fold":  # the chunk statistics read once, 3 per-shard statistics out
            return 0.0, 12 * c * cps * T + 12 * c * T
        if name == "vocab_ce_combine":
            return 0.0, 12 * N * T + 4 * T
        if name == "vocab_ce_mean":
            return 0.0, 4 * T + 4
    if w.kind == "vocab_embed" and name == "vocab_embed_partial":
        # ids read by every shard, each token's own row read once (by its
        # owner; c/N of the tokens on average), one partial per shard out, in
        # the table's type
        return 0.0, 4 * c * T + es * T * H * c / N + es * c * T * H
    if w.kind == "vocab_embed" and name == "vocab_embed_fold":  # N partials in, the rows out
        return 0.0, es * N * T * H + es * T * H
    if w.kind.startswith("norm_split"):
        Hs = H // N
        if name == "norm_split_stats":  # each shard's slices read once, one statistic pair per (shard, row) out
            return 0.0, es * c * T * Hs + 8 * c * T
        if name == "norm_split_apply":  # the slices again, the outputs, N statistic pairs per (shard, row), g (b)
            nb = 2 if w.kind == "norm_split_layer" else 1
            return 0.0, 2 * es * c * T * Hs + 8 * N * c * T + nb * es * c * Hs
    if name == "reduce_partials":
        return 0.0, 4 * N * rows_reduced * H + es * rows_reduced * H + (es * H if w.sigma_bias else 0)
    if name == "rmsnorm_gather":  # square, add, two scalings per element; X read once, Y written once
        return 4.0 * T * H, es * (2 * T * H + H)
    if name == "layernorm_gather":  # sum, deviation, square, add, scale, gain, shift; X once, Y once
        return 7.0 * T * H, es * (2 * T * H + 2 * H)
    raise KeyError(name)


def backward_direct(w):
    """Whether tp_mlp_backward reads every operand as stored (K-outer GEMM
    operands, column sums for the bias gradients): bf16 with T, H and the
    shard's Z width multiples of 64 (the 32-bit buffer-range condition holds
    at every workload here).  Otherwise the operands are transposed first."""
    zs = 2 * (w.F // w.N) if w.kind == "mlp_swiglu" else w.F // w.N
    return w.dtype == "bf16" and w.T % 64 == 0 and w.H % 64 == 0 and zs % 64 == 0


def backward_splits(T, Fc, H, direct=False):
    """Split-K factor of the backward's token-axis GEMMs (the rule of
    tp_mlp_backward: fill the chip with 256x256 tiles when up to 16 splits
    get there, else with 128x128 tiles at ~2 per CU; K per split >= 512 and a
    multiple of 8, of 64 on the direct path)."""
    big = ((Fc + 255) // 256) * ((H + 255) // 256)
    if big >= 256:
        return 1
    s = 1
    while s < 16 and big * s < 256 and T // (2 * s) >= 512:
        s *= 2
    if big * s < 256:
        small = ((Fc + 127) // 128) * ((H + 127) // 128)
        s = 1
        while s < 16 and small * s < 512 and T // (2 * s) >= 512:
            s *= 2
    while s > 1 and T % (8 * s):
        s //= 2
    while direct and s > 1 and (T // s) % 64:
        s //= 2
    return s


def backward_flops(w, c):
    """Algorithmic FLOP of the MLP pair's backward over c shards: GELU: dH,
    dX, dA and dB, each 2*T*H*(c*Fs); SwiGLU: dH 2*T*H*Fc, dX and the fused
    dA 2*T*H*(2 Fc) each, dB 2*T*H*Fc.  The recomputed column product is work
    this implementation adds and is not counted."""
    Fc = w.Fs * c
    if w.kind == "mlp_swiglu":
        return 12.0 * w.T * w.H * Fc
    return 8.0 * w.T * w.H * Fc


def colsum_chunks(R, C):
    """Row chunks of the library's two-launch column sum over [R x C] (its
    chunking rule: about 1024 workgroups of one 128-column strip and one chunk,
    at most 128 chunks of at least 128 rows, a multiple of 16 rows each)."""
    strips = (C + 127) // 128
    chunks = min((1024 + strips - 1) // strips, 128, (R + 127) // 128)
    chunks = max(chunks, 1)
    rpc = ((R + chunks - 1) // chunks + 15) // 16 * 16
    return (R + rpc - 1) // rpc


def backward_kernel_work(w, name, c, bmode=None):
    """Algorithmic (flops, bytes) of one launch of a backward kernel over c
    shards (bf16 operands, fp32 weight gradients).  Fz = the columns of Z:
    Fc, or 2*Fc ([gate | up]) for SwiGLU.  bmode "stored": the forward's Z
    (and, GELU, its activation) are read instead of recomputed."""
    T, H = w.T, w.H
    Fc = w.Fs * c
    swi = w.kind == "mlp_swiglu"
    Fz = 2 * Fc if swi else Fc
    direct = backward_direct(w)
    S = backward_splits(T, Fz, H, direct)
    bias = w.sigma_bias is not None
    if name == "bwd_fused_gemm":  # both passes: the recomputed pre-activation and dH; writes dZ and H
        return 4.0 * T * H * Fc, 2 * (2 * T * H + 2 * Fc * H + 2 * T * Fc) + (2 * Fc if bias else 0)
    if name == "bwd_recompute_gemm":
        return 2.0 * T * H * Fz, 2 * (T * H + Fz * H + T * Fz) + (2 * Fc if bias else 0)
    if name == "bwd_dz_gemm":  # reads the pre-activation beside the accumulators; writes act(Z) too (SwiGLU,
        # and GELU on the direct path unless the forward's activation is read instead)
        writes_act = swi or (direct and w.kind == "mlp_gelu" and not (bmode == "stored" and stored_activation(w)))
        return 2.0 * T * H * Fc, 2 * (T * H + Fc * H + 2 * T * Fz + (T * Fc if writes_act else 0))
    if name == "bwd_dx_gemm":
        return 2.0 * T * Fz * H, 2 * (T * Fz + H * Fz) + 4 * c * T * H
    if name == "bwd_da_gemm":
        return 2.0 * T * Fz * H, 2 * (T * Fz + T * H) + 4 * S * Fz * H
    if name == "bwd_db_gemm":
        return 2.0 * T * Fc * H, 2 * (T * Fc + T * H) + 4 * S * Fc * H
    if name == "bwd_transpose":
        if direct:  # B's range columns, for the two-pass kernel's second operand
            return 0.0, 2 * 2 * Fc * H
        # X, dY, A, B, act(Z), dZ: each read once and written once
        return 0.0, 2 * 2 * (2 * T * H + Fz * H + Fc * H + T * Fc + T * Fz) / 6
    # da (when the workload has a column bias) and db (row bias), each a sum
    # over the T rows of a [T x C] bf16 matrix into C fp32 values
    sums = ([Fc] if bias and not swi else []) + ([H] if bias else [])
    if name == "bwd_bias_rowsum":  # one launch per sum: the matrix once, C floats out
        return 0.0, sum(2 * T * cols + 4 * cols for cols in sums) / max(1, len(sums))
    if name == "bwd_bias_colsum":  # both sums' chunk sums in one launch: each matrix once, the partials out
        return 0.0, sum(2 * T * cols + 4 * colsum_chunks(T, cols) * cols for cols in sums)
    if name == "bwd_bias_colsum_fold":  # both folds in one launch: the partials in, C floats out per sum
        return 0.0, sum(4 * colsum_chunks(T, cols) * cols + 4 * cols for cols in sums)
    if name == "bwd_splitk_reduce":  # dA and dB
        return 0.0, (4 * S * Fz * H + 4 * Fz * H + 4 * S * Fc * H + 4 * Fc * H) / 2
    raise KeyError(name)


def roofline(w, name, flops, nbytes, avg_s):
    peak_f = PEAK_BF16 if w.dtype == "bf16" else PEAK_F32
    t_f = flops / peak_f
    t_b = nbytes / PEAK_HBM
    if t_f >= t_b:
        ach = flops / avg_s
        return {"bound": "mfma", "achieved": round(ach / 1e12, 2), "peak": round(peak_f / 1e12, 1),
                "unit": "TFLOP/s", "frac": round(ach / peak_f, 4)}
    ach = nbytes / avg_s
    return {"bound": "hbm", "achieved": round(ach / 1e9, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM, 4)}


# source files each kernel's code and launch shape come from (besides the
# shared device headers and the dispatch code in tp_api.cpp)
KERNEL_SOURCES = {
    "mlp_column_gemm": "gemm.hip", "mlp_row_gemm": "gemm.hip", "mlp_fused": "mlp_fused.hip", "attn_qk_gemm": "gemm.hip",
    "attn_vt_gemm": "gemm.hip", "attn_out_gemm": "gemm.hip", "attn_core": "attention.hip",
    "reduce_partials": "reduce.hip", "rmsnorm_gather": "norm.hip",
    "bwd_transpose": "bwd.hip", "bwd_bias_rowsum": "bwd.hip", "bwd_bias_colsum": "bwd.hip",
    "bwd_bias_colsum_fold": "bwd.hip",
    "bwd_recompute_gemm": "gemm.hip",
    "bwd_dz_gemm": "gemm.hip", "bwd_dx_gemm": "gemm.hip", "bwd_da_gemm": "gemm.hip", "bwd_db_gemm": "gemm.hip",
    "bwd_splitk_reduce": "reduce.hip", "bwd_fused_gemm": "gemm.hip",
    "vocab_logits_gemm": "gemm.hip", "vocab_ce_fold": "vocab.hip", "vocab_ce_combine": "vocab.hip",
    "vocab_ce_mean": "vocab.hip", "vocab_embed_partial": "vocab.hip", "vocab_embed_fold": "vocab.hip",
    "layernorm_gather": "norm.hip", "norm_split_stats": "norm.hip", "norm_split_apply": "norm.hip",
}


def kernel_source_hash(kernel=None):
    """Hash of the sources behind one kernel (or of every kernel source)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tensor_transformer_layers_amd", "csrc")
    if kernel is None:
        files = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp", ".cpp")))
    else:
        files = [KERNEL_SOURCES[kernel], "tp_device.hpp", "tp_dma.hpp", "tp_kernels.hpp", "tp_api.cpp"]
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


# launch order of the library's kernels within one step, and a piece of the
# device function name each one has in a profiler's kernel list
KERNEL_SYMBOL = {
    "mlp_column_gemm": "gemm_", "mlp_row_gemm": "gemm_", "mlp_fused": "mlp_fused_kernel",
    "attn_qk_gemm": "gemm_", "attn_vt_gemm": "gemm_", "attn_out_gemm": "gemm_",
    "attn_core": "attn_fwd_kernel", "reduce_partials": "reduce_kernel", "rmsnorm_gather": "rmsnorm_gather_kernel",
    "bwd_transpose": "transpose_kernel", "bwd_bias_rowsum": "rowsum_kernel", "bwd_bias_colsum": "colsum_kernel",
    "bwd_bias_colsum_fold": "colsum_kernel",
    "bwd_recompute_gemm": "gemm_",
    "bwd_dz_gemm": "gemm_", "bwd_dx_gemm": "gemm_", "bwd_da_gemm": "gemm_", "bwd_db_gemm": "gemm_",
    "bwd_splitk_reduce": "reduce_kernel", "bwd_fused_gemm": "gemm_",
    "vocab_logits_gemm": "gemm_", "vocab_ce_fold": "ce_fold_kernel", "vocab_ce_combine": "ce_combine_kernel",
    "vocab_ce_mean": "ce_mean_kernel", "vocab_embed_partial": "embed_partial_kernel",
    "vocab_embed_fold": "embed_fold_kernel",
    "layernorm_gather": "rmsnorm_gather_kernel", "norm_split_stats": "norm_split_stats_kernel",
    "norm_split_apply": "norm_split_apply_kernel",
}


def stored_preactivation(w):
    """Whether the backward of workload w can take the forward's stored
    pre-activation (tp_mlp_desc.Z): the bf16 GELU and SwiGLU MLPs."""
    return w.kind in ("mlp_gelu", "mlp_swiglu") and w.dtype == "bf16"


def stored_activation(w):
    """Whether the stored-pre-activation backward of workload w also takes
    the forward's activation (tp_mlp_desc.Hact) for dB: the bf16 GELU MLP."""
    return w.kind == "mlp_gelu" and w.dtype == "bf16"


def backward_mode(w, recompute):
    """The backward variant bench.py times: "stored" (the forward's
    pre-activation) unless asked to recompute it or w cannot store it."""
    return "recompute" if recompute or not stored_preactivation(w) else "stored"


def backward_launch_order(w, mode="recompute"):
    """Kernels one backward step (all shards) launches, in order (the
    sequence of tp_mlp_backward): with the stored pre-activation, dZ reads it;
    recomputing, GELU with H <= 2048 runs the recomputation and dZ as one
    two-pass kernel, every other case a recomputing GEMM first.  On the
    direct path the GEMMs read the operands as stored (only the two-pass
    kernel needs B transposed) and each bias gradient is a column sum (two
    launches); otherwise six transposes come first and the bias gradients
    are row sums."""
    direct = backward_direct(w)
    split = backward_splits(w.T, 2 * w.F if w.kind == "mlp_swiglu" else w.F, w.H, direct) > 1
    fused = w.kind == "mlp_gelu" and w.H <= 2048 and w.dtype == "bf16"
    if mode == "stored":
        mid = ["bwd_dz_gemm"]
    else:
        mid = ["bwd_fused_gemm"] if fused else ["bwd_recompute_gemm", "bwd_dz_gemm"]
    if direct:
        order = (["bwd_transpose"] if mid == ["bwd_fused_gemm"] else []) + mid
    else:
        order = ["bwd_transpose"] * 4 + mid + ["bwd_transpose"] * 2
    order += ["bwd_dx_gemm", "bwd_da_gemm"] + (["bwd_splitk_reduce"] if split else [])
    order += ["bwd_db_gemm"] + (["bwd_splitk_reduce"] if split else [])
    bias = w.sigma_bias is not None
    n_bias = (1 if bias and w.kind == "mlp_gelu" else 0) + (1 if bias else 0)
    if direct:  # both column sums share their two launches
        order += ["bwd_bias_colsum", "bwd_bias_colsum_fold"] if n_bias else []
    else:
        order += ["bwd_bias_rowsum"] * n_bias
    return order + ["reduce_partials"]


def setup_launches(w, backward=False):
    """Library kernels bench.py launches once before its steps: for the
    stored-pre-activation backward, the training forward that writes Z (it
    always takes the GEMM path: column GEMM with Z, row GEMM, reduction)."""
    return ["mlp_column_gemm", "mlp_row_gemm", "reduce_partials"] if backward == "stored" else []


def strip_setup(w, backward, ours, name_of):
    """The library dispatches of a profiled run after the set-up launches,
    which are checked by name and dropped."""
    pre = setup_launches(w, backward)
    for k, r in zip(pre, ours):
        if KERNEL_SYMBOL[k] not in name_of(r):
            raise RuntimeError(f"set-up dispatch: expected {k} ({KERNEL_SYMBOL[k]}), profiler has {name_of(r)[:120]}")
    return ours[len(pre):]


def launch_order(w, sp_entry=False, backward=False):
    """Kernels one step of workload w launches, in order.  A bf16 GELU MLP
    with hidden 256 or 512 and a shard width that is a multiple of 32 (at
    most 4096) runs the fused kernel; every other MLP the column and row
    GEMMs (the dispatch rule of tp_mlp_forward).  With the sequence-parallel
    entry side, the norm-and-gather kernel comes first."""
    if backward:
        return backward_launch_order(w, backward)
    if w.kind == "vocab_ce":
        return ["vocab_logits_gemm", "vocab_ce_fold", "vocab_ce_combine", "vocab_ce_mean"]
    if w.kind == "vocab_embed":
        return ["vocab_embed_partial", "vocab_embed_fold"]
    if w.kind.startswith("norm_split"):
        return ["norm_split_stats", "norm_split_apply"]
    # sp_entry: False, or the entry norm ("rms" / True: RMSNorm; "layer": LayerNorm)
    head = ([("layernorm_gather" if sp_entry == "layer" else "rmsnorm_gather")] if sp_entry else [])
    if w.kind == "attn":
        return head + ["attn_qk_gemm", "attn_vt_gemm", "attn_core", "attn_out_gemm", "reduce_partials"]
    Fs = w.F // w.N
    if w.kind == "mlp_gelu" and w.dtype == "bf16" and w.H in (256, 512) and Fs % 32 == 0 and Fs <= 4096:
        return head + ["mlp_fused", "reduce_partials"]
    return head + ["mlp_column_gemm", "mlp_row_gemm", "reduce_partials"]


def traffic_path(workload_name, out_dir=None):
    return os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"traffic_{workload_name}.txt")


def measured_traffic(kernel, workload_name):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC
    summary of this workload, if it was taken on the kernel's current
    sources; otherwise None."""
    p = traffic_path(workload_name)
    if not os.path.exists(p):
        return None
    for line in open(p):
        f = line.split()
        if len(f) == 4 and f[0] == "traffic_bytes" and f[1] == kernel:
            return float(f[2]) if f[3] == kernel_source_hash(kernel) else None
    return None


def workload_tag(w, sp_entry=False, backward=False):
    return (w.name + ("_sp_entry" if sp_entry else "") + ("_layernorm" if sp_entry == "layer" else "")
            + ("_backward" if backward else "") + ("_recompute" if backward == "recompute" else ""))


def write_traffic(w, share, pmc_dir, argv_line, sp_entry=False, backward=False, out_dir=None):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, each with --calib-copy) into profiles/traffic_<workload>.txt.

    Each counter is scaled by what it reads for the 1 GiB device copy
    (2^30 bytes read, 2^30 written).  Library kernels are matched to names by
    their launch order within a step."""
    import csv
    import collections

    order = launch_order(w, sp_entry, backward)
    name = workload_tag(w, sp_entry, backward)
    per = {}
    factor = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = list(csv.DictReader(open(os.path.join(pmc_dir, counter, "run_counter_collection.csv"))))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        # the calibration copies are the run's last device copies (set-up may
        # copy too, before the timed region)
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        big = copies[-1]
        factor[counter] = float(2 ** 30) / (float(big["Counter_Value"]) * 1024.0)
        ours = [r for r in rows if "tp::" in r["Kernel_Name"] or "_ZN2tp" in r["Kernel_Name"]]
        ours = strip_setup(w, backward, ours, lambda r: r["Kernel_Name"])
        vals = collections.defaultdict(list)
        for i, r in enumerate(ours):
            k = order[i % len(order)]
            if KERNEL_SYMBOL[k] not in r["Kernel_Name"]:
                raise RuntimeError(f"dispatch {r['Dispatch_Id']}: expected {k} ({KERNEL_SYMBOL[k]}), "
                                   f"profiler has {r['Kernel_Name'][:120]}")
            vals[k].append(float(r["Counter_Value"]))
        per[counter] = {k: sum(v) / len(v) for k, v in vals.items()}
    lines = [
        f"# HBM traffic per launch: {name} ({share})",
        "#",
        "# Commands (from /tmp on the GPU host, REPO = repository root):",
        f"#   rocprofv3 --pmc FETCH_SIZE -f csv -d DIR/FETCH_SIZE -o run -- python3 $REPO/bench.py {argv_line}",
        f"#   rocprofv3 --pmc WRITE_SIZE -f csv -d DIR/WRITE_SIZE -o run -- python3 $REPO/bench.py {argv_line}",
        f"#   python3 $REPO/bench.py --config {w.key} --share {share}"
        f"{(' --sp-entry' + (' --norm layer' if sp_entry == 'layer' else '')) if sp_entry else ''}"
        f"{' --backward' if backward else ''} --traffic-from DIR",
        "#",
        f"# Calibration (1 GiB device copy): FETCH_SIZE x {factor['FETCH_SIZE']:.4f}, WRITE_SIZE x {factor['WRITE_SIZE']:.4f}",
        "#",
        "# kernel                 FETCH_KiB      WRITE_KiB      read_bytes      write_bytes     total_bytes",
    ]
    out = {}
    for k in dict.fromkeys(order):
        if k not in per["FETCH_SIZE"]:
            continue
        rb = per["FETCH_SIZE"][k] * 1024.0 * factor["FETCH_SIZE"]
        wb = per["WRITE_SIZE"].get(k, 0.0) * 1024.0 * factor["WRITE_SIZE"]
        out[k] = rb + wb
        lines.append(f"# {k:22s} {per['FETCH_SIZE'][k]:13.1f} {per['WRITE_SIZE'].get(k, 0.0):13.1f} "
                     f"{rb:15.0f} {wb:15.0f} {rb + wb:15.0f}")
    lines.append("# traffic_bytes <kernel> <bytes per launch> <hash of that kernel's sources>")
    for k, v in out.items():
        lines.append(f"traffic_bytes {k} {v:.0f} {kernel_source_hash(k)}")
    path = traffic_path(name, out_dir)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def mfma_path(tag, out_dir=None):
    return os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"mfma_{tag}.txt")


def write_mfma(w, share, pmc_dir, argv_line, sp_entry=False, backward=False, out_dir=None):
    """Turn one rocprofv3 --pmc run of this script with the derived counters
    MfmaFlopsBF16 (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) and MfmaUtil (MFMA-busy
    SIMD cycles / (active GPU cycles x SIMDs)) into profiles/mfma_<workload>.txt:
    per kernel, the matrix-core FLOP executed per launch against the
    algorithmic FLOP, and the share of time the matrix cores were busy."""
    import csv
    import collections

    order = launch_order(w, sp_entry, backward)
    tag = workload_tag(w, sp_entry, backward)
    rows = list(csv.DictReader(open(os.path.join(pmc_dir, "run_counter_collection.csv"))))
    per = collections.defaultdict(dict)  # dispatch -> counter -> value
    names = {}
    for r in rows:
        per[int(r["Dispatch_Id"])][r["Counter_Name"]] = float(r["Counter_Value"])
        names[int(r["Dispatch_Id"])] = r["Kernel_Name"]
    ours = [d for d in sorted(per) if "tp::" in names[d] or "_ZN2tp" in names[d]]
    ours = strip_setup(w, backward, ours, lambda d: names[d])
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for i, dsp in enumerate(ours):
        k = order[i % len(order)]
        if KERNEL_SYMBOL[k] not in names[dsp]:
            raise RuntimeError(f"dispatch {dsp}: expected {k} ({KERNEL_SYMBOL[k]}), profiler has {names[dsp][:120]}")
        for c, v in per[dsp].items():
            vals[k][c].append(v)
    shards = w.N if share == "layer" else 1
    lines = [
        f"# Matrix-core work and busy share per launch: {tag} ({share})",
        "#",
        "# Command (from /tmp on the GPU host, REPO = repository root):",
        f"#   rocprofv3 --pmc MfmaFlopsBF16 MfmaUtil -f csv -d DIR -o run -- python3 $REPO/bench.py {argv_line}",
        f"#   python3 $REPO/bench.py --config {w.key} --share {share}"
        f"{(' --sp-entry' + (' --norm layer' if sp_entry == 'layer' else '')) if sp_entry else ''}"
        f"{' --backward' if backward else ''} --mfma-from DIR",
        "#",
        "# MfmaFlopsBF16 = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 (executed matrix FLOP, padding and recomputation",
        "# included); MfmaUtil = 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) / (GRBM_GUI_ACTIVE * SIMDs), the share of",
        "# the kernel's active cycles the matrix cores were busy, at whatever clock the chip ran.",
        "#",
        "# kernel                 mfma_flop_per_launch   algorithmic_flop   executed/algorithmic   mfma_busy_%",
    ]
    for k in dict.fromkeys(order):
        if k not in vals:
            continue
        fl = sum(vals[k].get("MfmaFlopsBF16", [0.0])) / max(1, len(vals[k].get("MfmaFlopsBF16", [0.0])))
        ut = vals[k].get("MfmaUtil", [])
        ut = sum(ut) / len(ut) if ut else float("nan")
        alg = kernel_work(w, k, shards, w.T if share == "layer" or w.n_slices == 1 else w.T // w.n_slices)[0]
        ratio = fl / alg if alg else float("nan")
        lines.append(f"# {k:22s} {fl:20.4e} {alg:18.4e} {ratio:22.4f} {ut:13.2f}")
    path = mfma_path(tag, out_dir)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def trace_path(tag, out_dir=None):
    return os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"kernels_{tag}.md")


def write_trace(w, share, trace_dir, argv_line, steps, sp_entry=False, backward=False, out_dir=None):
    """Turn one rocprofv3 --kernel-trace --stats csv run of this script into
    profiles/kernels_<workload>.md: per library kernel (matched by launch
    order within a step), the dispatch count and the average, min and max
    duration over every dispatch, and the average over the last ``steps``
    steps (the timed region in which bench.py attaches HIP events to each
    launch, whose averages the JSON line reports)."""
    import csv
    import collections

    order = launch_order(w, sp_entry, backward)
    tag = workload_tag(w, sp_entry, backward) + ("_rank0" if share == "rank" else "")
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    ours = [r for r in rows if "tp::" in r["Kernel_Name"] or "_ZN2tp" in r["Kernel_Name"]]
    ours = strip_setup(w, backward, ours, lambda r: r["Kernel_Name"])
    if len(ours) % len(order):
        raise RuntimeError(f"{len(ours)} library dispatches is not a whole number of {len(order)}-kernel steps")
    durs = collections.defaultdict(list)
    names = {}
    for i, r in enumerate(ours):
        k = order[i % len(order)]
        if KERNEL_SYMBOL[k] not in r["Kernel_Name"]:
            raise RuntimeError(f"dispatch {r['Dispatch_Id']}: expected {k} ({KERNEL_SYMBOL[k]}), "
                               f"profiler has {r['Kernel_Name'][:120]}")
        durs[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        names[k] = r["Kernel_Name"]
    nsteps = len(ours) // len(order)
    per_step = collections.Counter(order)
    agent = ""
    ap = os.path.join(trace_dir, "run_agent_info.csv")
    if os.path.exists(ap):
        for a in csv.DictReader(open(ap)):
            if a.get("Agent_Type", a.get("Type", "")).upper().endswith("GPU") or a.get("Name", "").startswith("gfx"):
                agent = (f"{a.get('Name', '')}, {a.get('Cu_Count', a.get('Compute_Unit_Count', '?'))} CUs, "
                         f"max engine clock {a.get('Max_Engine_Clk_Fcompute', a.get('Max_Clock_Freq', '?'))} MHz")
                break

    def short(n):
        import re
        n = n.replace("void ", "").replace("tp::(anonymous namespace)::", "")
        return re.sub(r"\(tp::[A-Za-z]+Params[^)]*\)", "", n).replace("(tp::GemmParams, int, int)", "")

    shards = w.N if share == "layer" else 1
    rows_red = w.T if (share == "layer" or w.n_slices == 1) else w.T // w.n_slices
    lines = [
        f"# Kernel trace: {tag} ({'all shards + reduction' if share == 'layer' else 'rank 0 shard + reduction'})",
        "",
        "Commands (from /tmp on the GPU host, REPO = repository root):",
        "",
        f"    rocprofv3 --kernel-trace --stats -f csv -d DIR -o run -- python3 $REPO/bench.py {argv_line}",
        f"    python3 $REPO/bench.py {argv_line.split(' --steps')[0]} --trace-from DIR",
        "",
        f"{len(ours)} library dispatches = {nsteps} steps of {len(order)} kernels (set-up pass, warm-up, and "
        f"the three timed passes of {steps} steps each).  'Timed avg' is the mean over the last {steps} steps, "
        "the pass in which bench.py times each launch with HIP events.",
        "",
        "| Kernel | Role | Calls | Avg all (us) | Timed avg (us) | Min (us) | Max (us) | Achieved | Roofline frac |",
        "|---|---|---|---|---|---|---|---|---|",
    ]
    for k in dict.fromkeys(order):
        d = durs[k]
        last = d[-steps * per_step[k]:]
        avg_t = sum(last) / len(last)
        f, b = kernel_work(w, k, shards, rows_red, bmode=backward or None)
        rf = roofline(w, k, f, b, avg_t / 1e6)
        lines.append(f"| `{short(names[k])}` | {k} | {len(d)} | {sum(d) / len(d):.2f} | {avg_t:.2f} | "
                     f"{min(d):.2f} | {max(d):.2f} | {rf['achieved']} {rf['unit']} | {rf['frac']:.4f} |")
    lines += ["", f"Algorithmic work per launch and peaks as in bench.py (bf16 MFMA {PEAK_BF16 / 1e12:.0f} TFLOP/s, "
              f"HBM {PEAK_HBM / 1e9:.0f} GB/s).  Kernel sources hash: "
              + ", ".join(f"{k} {kernel_source_hash(k)}" for k in dict.fromkeys(order)) + "."]
    if agent:
        lines.append(f"Agent: {agent}.")
    path = trace_path(tag, out_dir)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def cpu_baseline(w, host, seconds):
    """fp64 oracle on a bounded, seeded sample of token rows of the same
    workload; TFLOP/s counted with the same algorithmic FLOP per row."""
    import numpy as np

    from oracle import reference as R

    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    if w.kind == "vocab_embed":
        return cpu_baseline_embed(w, host, seconds, cores)
    if w.kind.startswith("norm_split"):
        return cpu_baseline_norm(w, host, seconds, cores)
    chunk = 256 if w.kind != "attn" else 8
    order = np.random.default_rng(w.seed + 98).permutation(w.T)  # seeded order of all token rows
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    # cycle through the seeded row order (a small workload is passed over
    # several times) until the time budget is spent
    while time.perf_counter() - t0 < seconds:
        start = done % w.T
        rows = np.sort(order[start:start + chunk])
        R.workload(w.kind, host, w.batch, w.seq, w.heads, rows=rows)
        if w.kind == "attn":
            hl_all = w.heads
            pos = rows % w.seq
            flops += len(rows) * 8.0 * w.H * w.H + float(np.sum(hl_all * 4.0 * w.head_dim * (pos + 1)))
        else:
            flops += len(rows) * w.flops_layer() / w.T
        done += len(rows)
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} token rows in seeded order over the workload's {w.T} "
                      f"({done / w.T:.2f} passes), fp64 numpy/scipy, {el:.1f} s"}


def cpu_baseline_embed(w, host, seconds, cores):
    """fp64 oracle lookup (every shard's masked lookup, then the fold) on
    seeded blocks of 2048 token rows; GB/s counted with the same algorithmic
    bytes per token as the GPU figure."""
    import numpy as np

    from oracle import reference as R

    order = np.random.default_rng(w.seed + 98).permutation(w.T)
    per_token = sum(kernel_work(w, k, w.N, w.T)[1] for k in launch_order(w)) / w.T
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        start = done % w.T
        rows = np.sort(order[start:start + 2048])
        R.workload(w.kind, host, rows=rows, N=w.N)
        done += len(rows)
    el = time.perf_counter() - t0
    return {"value": round(done * per_token / el / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} token rows in seeded blocks of 2048 over the workload's {w.T}, fp64 numpy "
                      f"(each call converts the table to fp64), {el:.1f} s"}


def cpu_baseline_norm(w, host, seconds, cores):
    """fp64 oracle hidden-split norm on seeded blocks of 1024 token rows;
    GB/s counted with the same algorithmic bytes per token as the GPU figure."""
    import numpy as np

    from oracle import reference as R

    order = np.random.default_rng(w.seed + 98).permutation(w.T)
    per_token = sum(kernel_work(w, k, w.N, w.T)[1] for k in launch_order(w)) / w.T
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        start = done % w.T
        rows = np.sort(order[start:start + 1024])
        R.workload(w.kind, host, rows=rows, N=w.N, eps=1e-6)
        done += len(rows)
    el = time.perf_counter() - t0
    return {"value": round(done * per_token / el / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} token rows in seeded blocks of 1024 over the workload's {w.T}, fp64 numpy, {el:.1f} s"}


def cpu_baseline_backward(w, host, dY, seconds):
    """fp64 oracle backward on seeded blocks of token rows of the same
    workload (the weight gradients over those rows only); TFLOP/s counted
    with the same algorithmic FLOP per row as the GPU figure."""
    import numpy as np

    from oracle import reference as R

    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    chunk = 256
    order = np.random.default_rng(w.seed + 97).permutation(w.T)
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        start = done % w.T
        rows = np.sort(order[start:start + chunk])
        if w.kind == "mlp_swiglu":
            R.mlp_swiglu_backward(host["X"][rows], host["Wg"], host["Wu"], host["Wd"], dY[rows])
        else:
            R.mlp_gelu_backward(host["X"][rows], host["A"], host["a"], host["B"], dY[rows])
        flops += len(rows) * backward_flops(w, w.N) / w.T
        done += len(rows)
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"backward over {done} token rows in blocks of {chunk}, seeded order over the workload's "
                      f"{w.T} ({done / w.T:.2f} passes), fp64 numpy/scipy, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: as many as fill about 0.5 s, at least 20)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps, a minimum: warm-up always runs for at least --warmup-seconds "
                         "of wall time as well, since the shader clock takes tens of ms to settle after idle")
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="minimum wall time of the warm-up (default 0.5 s)")
    ap.add_argument("--config", type=int, default=5,
                    help="workload 1..5 (default 5: the 175B-shaped GELU MLP bf16, T=16384, H=12288, F=49152, "
                         "N=8, partial sums reduce-scattered into 8 sequence slices), 6: the "
                         "vocab-parallel output head + cross-entropy (T=16384, H=4096, V=150000, N=8), or 7: the "
                         "vocab-parallel embedding lookup (same sizes)")
    ap.add_argument("--share", choices=["layer", "rank"], default="layer")
    ap.add_argument("--sp-entry", action="store_true",
                    help="MLP workloads with a reduce-scatter: start each step with the sequence-parallel entry "
                         "side (RMSNorm of every sequence slice into the gathered input, the all-gather stand-in)")
    ap.add_argument("--norm", choices=["rms", "layer"], default="rms",
                    help="with --sp-entry: the entry norm, RMSNorm (default) or LayerNorm")
    ap.add_argument("--backward", action="store_true",
                    help="GELU MLP workloads (2, 5): time the backward of the pair instead (input, weight and "
                         "bias gradients of every shard, then the input-gradient reduction)")
    ap.add_argument("--recompute", action="store_true",
                    help="with --backward: recompute the pre-activation X A^T + a in the backward instead of taking "
                         "the one the forward stored (the bf16 GELU and SwiGLU workloads store it; the others always recompute)")
    ap.add_argument("--overlap", type=int, default=0, metavar="K",
                    help="MLP workloads, --share layer: cut the tokens into K row blocks and overlap the reduction "
                         "of block k (on a second stream) with the products of block k+1")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (PMC traffic calibration)")
    ap.add_argument("--mfma-from", metavar="DIR",
                    help="write profiles/mfma_<workload>.txt from a rocprofv3 --pmc MfmaFlopsBF16 MfmaUtil csv run "
                         "under DIR and exit; runs on the host, no GPU")
    ap.add_argument("--trace-from", metavar="DIR",
                    help="write profiles/kernels_<workload>.md from a rocprofv3 --kernel-trace --stats csv run of "
                         "this script (same --config/--share/--steps flags) under DIR and exit; runs on the host")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="write profiles/traffic_<workload>.txt from rocprofv3 --pmc csv runs under DIR "
                         "(DIR/FETCH_SIZE, DIR/WRITE_SIZE) and exit; runs on the host, no GPU")
    args = ap.parse_args()
    if args.sp_entry:
        args.sp_entry = args.norm  # the entry norm's kind travels with the flag
    sp_flags = (" --sp-entry" + (" --norm layer" if args.sp_entry == "layer" else "")) if args.sp_entry else ""
    bwd_flags = (" --backward" + (" --recompute" if args.recompute else "")) if args.backward else ""

    if args.mfma_from:
        from tensor_transformer_layers_amd import configs

        w = configs.workload(args.config)
        argv = (f"--config {args.config} --share {args.share}{sp_flags}"
                f"{bwd_flags} --steps 3 --warmup 1 --no-cpu-baseline")
        print(write_mfma(w, args.share, args.mfma_from, argv, args.sp_entry,
                         args.backward and backward_mode(w, args.recompute)))
        return

    if args.trace_from:
        from tensor_transformer_layers_amd import configs

        w = configs.workload(args.config)
        if args.steps is None or args.overlap:
            print("bench.py --trace-from needs the --steps of the profiled run (and no --overlap)", file=sys.stderr)
            sys.exit(2)
        argv = (f"--config {args.config} --share {args.share}{sp_flags}"
                f"{bwd_flags} --steps {args.steps} --no-cpu-baseline")
        print(write_trace(w, args.share, args.trace_from, argv, args.steps, args.sp_entry,
                          args.backward and backward_mode(w, args.recompute)))
        return

    if args.traffic_from:
        from tensor_transformer_layers_amd import configs

        w = configs.workload(args.config)
        argv = (f"--config {args.config} --share {args.share}{sp_flags}"
                f"{bwd_flags} --steps 3 --warmup 1 --no-cpu-baseline --calib-copy")
        print(write_traffic(w, args.share, args.traffic_from, argv, args.sp_entry,
                            args.backward and backward_mode(w, args.recompute)))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs on ONE GPU (all N tensor-parallel shards on one device, "
              "an on-device reduction standing in for the all-reduce); --gpus above 1 is not supported.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    from tensor_transformer_layers_amd import configs, inputs, tp, workloads

    tp.lib()  # fails loudly if libtp.so is missing
    w = configs.workload(args.config)
    if w.kind in ("vocab_ce", "vocab_embed") and (args.share != "layer" or args.sp_entry or args.backward):
        print("bench.py: the vocab workloads (--config 6, 7) run with --share layer only",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if w.kind.startswith("norm_split") and (args.share != "layer" or args.sp_entry or args.backward or args.overlap):
        print("bench.py: the hidden-split norm workloads (--config 8, 9) run with --share layer only",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.overlap and (w.kind not in ("mlp_gelu", "mlp_swiglu") or args.share != "layer" or args.backward
                         or w.T % args.overlap):
        print("bench.py: --overlap K needs an MLP workload, --share layer and K dividing the token count",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.sp_entry and (w.kind == "attn" or w.n_slices < 2 or args.share != "layer"):
        print("bench.py: --sp-entry needs an MLP workload with a reduce-scatter (--config 5) and --share layer",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.backward and (w.kind not in ("mlp_gelu", "mlp_swiglu") or args.share != "layer" or args.sp_entry):
        print("bench.py: --backward needs an MLP workload (--config 1, 2, 3 or 5) and --share layer",
              file=sys.stderr, flush=True)
        sys.exit(2)
    log(f"workload {w.name}: generating seeded inputs")
    host = inputs.make_inputs(w)
    d = workloads.device_inputs(w, host)
    bmode = None
    Zst = Hst = None
    if args.backward:
        dY_host = inputs.grad_output(w)
        dY = workloads.to_device(dY_host, d["X"].dtype)
        bmode = backward_mode(w, args.recompute)
        if bmode == "stored":  # one training forward before the timed region writes Z (and, GELU, H)
            zw = 2 * w.F if w.kind == "mlp_swiglu" else w.F  # SwiGLU: [gate | up] per shard
            Zst = torch.empty((w.T, zw), dtype=d["X"].dtype, device=d["X"].device)
            if stored_activation(w):
                Hst = torch.empty((w.T, w.F), dtype=d["X"].dtype, device=d["X"].device)
            tp.mlp_forward(d["X"], d["A"], d["a"], d["B"], d["b"], w.N, act=workloads.act_of(w), Z=Zst, Hact=Hst)
    if args.sp_entry:
        # X holds the n_slices sequence slices of the sublayer input; each step
        # normalizes them into Xn, the gathered input of the column GEMM
        gain = workloads.to_device(inputs.norm_gain(w), d["X"].dtype)
        shift = workloads.to_device(inputs.norm_shift(w), d["X"].dtype) if args.sp_entry == "layer" else None
        x_slices = d["X"]
        d = dict(d, X=torch.empty_like(x_slices))

        def entry_norm(stream=None):
            if args.sp_entry == "layer":
                tp.layernorm_gather(x_slices, gain, shift, inputs.NORM_EPS, w.n_slices, out=d["X"], stream=stream)
            else:
                tp.rmsnorm_gather(x_slices, gain, inputs.NORM_EPS, w.n_slices, out=d["X"], stream=stream)

        entry_norm()
    if args.backward:
        grads, ws = workloads.backward(w, d, dY, Z=Zst, Hact=Hst)  # allocates the gradients and the workspace once
        Y = grads["dX"]
    else:
        Y, ws = workloads.forward(w, d)  # allocates Y and the workspace once
    torch.cuda.synchronize()
    rank_slice = 0 if w.n_slices > 1 else -1
    Yr = None
    if args.share == "rank":
        rows = w.T // w.n_slices if w.n_slices > 1 else w.T
        Yr = torch.empty((rows, w.H), dtype=Y.dtype, device=Y.device)
    stream = torch.cuda.current_stream()
    stream2 = torch.cuda.Stream() if args.overlap else None  # default priority

    def step():
        if args.overlap:
            if args.sp_entry:
                entry_norm(stream)
            workloads.forward_overlap(w, d, args.overlap, stream2, Y=Y, ws=ws, stream=stream)
            return
        if args.backward:
            workloads.backward(w, d, dY, grads=grads, ws=ws, Z=Zst, Hact=Hst, stream=stream)
            return
        if args.sp_entry:
            entry_norm(stream)
        if args.share == "layer":
            workloads.forward(w, d, Y=Y, ws=ws, stream=stream)
        else:
            workloads.forward(w, d, ws=ws, shard_begin=0, shard_count=1, stream=stream)
            workloads.reduce_slab(w, d, ws, Y=Yr, slice=rank_slice, stream=stream)

    # Warm-up by time as well as by count: after idle the shader clock ramps
    # for tens of ms (measured 1.3 -> 1.9 GHz over ~30 ms on the large GEMMs,
    # 2.05 -> 2.3 GHz over ~40 ms on the hidden-512 workload), so a small step
    # count alone would time the ramp instead of the steady state.  --warmup
    # is a minimum number of steps; the warm-up goes on until it has also
    # filled --warmup-seconds of wall time.
    warm_min = 5 if args.warmup is None else max(0, args.warmup)
    log(f"warmup: at least {warm_min} steps and {args.warmup_seconds:.2f} s")
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    warm_done = 0
    est = None
    while warm_done < warm_min or time.perf_counter() - tw0 < args.warmup_seconds:
        step()
        warm_done += 1
        if warm_done == 3 or (warm_done >= warm_min and warm_done % 4 == 0):
            torch.cuda.synchronize()  # keep the queue short so that wall time tracks GPU time
            if est is None and warm_done == 3:
                est = (time.perf_counter() - tw0) / 3
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - tw0
    if est is None:
        est = warm_s / max(1, warm_done)
    if args.steps is None:
        args.steps = max(20, int(0.5 / max(est, 1e-6)))
    log(f"warmup done: {warm_done} steps in {warm_s:.3f} s")

    # timed region 1: the steps alone
    log(f"timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / args.steps

    # timed region 1b: the same steps with an event between steps, for the
    # spread of single-step times (median, min, max)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    step_stats = {"median": round(per_step[len(per_step) // 2], 5), "min": round(per_step[0], 5),
                  "max": round(per_step[-1], 5)}

    # timed region 2: the same steps with a HIP event pair around every kernel
    tp.tp_timing_reset()
    tp.tp_timing_enable(1)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    tp.tp_timing_enable(0)
    kern = tp.tp_timing_read()

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=Y.device)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    shards = w.N if args.share == "layer" else 1
    rows_red = w.T if (args.share == "layer" or w.n_slices == 1) else w.T // w.n_slices
    flops = w.flops_layer() if args.share == "layer" else w.flops_shard()
    if args.sp_entry:
        flops += kernel_work(w, "layernorm_gather" if args.sp_entry == "layer" else "rmsnorm_gather", 1, 0)[0]
    if args.backward:
        flops = backward_flops(w, w.N)
    value = flops / (ms_step / 1e3) / 1e12
    bytes_metric = w.kind == "vocab_embed" or w.kind.startswith("norm_split")
    if bytes_metric:  # no arithmetic to speak of: algorithmic bytes of the step (every kernel) per second
        step_bytes = sum(kernel_work(w, k, shards, rows_red)[1] for k in launch_order(w))
        value = step_bytes / (ms_step / 1e3) / 1e9

    # with --overlap each launch covers one row block of T/K tokens
    wk = configs.scaled(w, batch=1, seq=w.T // args.overlap) if args.overlap else w
    if args.overlap:
        rows_red = wk.T
    kernels = {}
    for name, (ms, n) in kern.items():
        f, b = kernel_work(wk, name, shards, rows_red, bmode=bmode)
        avg = ms / n / 1e3
        kernels[name] = {"avg_us": round(avg * 1e6, 2), "launches": n,
                         "share": round(ms / sum(v[0] for v in kern.values()), 4),
                         **roofline(w, name, f, b, avg)}
    dom = max(kern, key=lambda k: kern[k][0])
    f, b = kernel_work(wk, dom, shards, rows_red, bmode=bmode)
    avg = kern[dom][0] / kern[dom][1] / 1e3
    roof = roofline(w, dom, f, b, avg)
    src_hash = kernel_source_hash()
    roof["kernel"] = dom
    roof["avg_us"] = round(avg * 1e6, 2)
    roof["algorithmic"] = {"flop": f, "bytes": b}
    roof["traffic"] = measured_traffic(dom, workload_tag(w, args.sp_entry, bmode or False))

    out = {
        "metric": (METRIC_BWD if args.backward else METRIC_VOCAB if w.kind == "vocab_ce" else
                   METRIC_EMBED if w.kind == "vocab_embed" else
                   METRIC_NORM if w.kind.startswith("norm_split") else METRIC),
        "value": round(value, 3),
        "unit": "GB/s" if bytes_metric else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm_done,
        "warmup_requested": args.warmup,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_step, 5),
        "step_ms": step_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "kind": w.kind, "tokens": w.T, "batch": w.batch, "seq": w.seq, "hidden": w.H,
            "ffn": w.F if w.kind in ("mlp_gelu", "mlp_swiglu") else None, "heads": w.heads or None, "shards": w.N,
            **({"vocab": w.F, "vocab_padded": tp.tp_vocab_padded(w.F, w.N),
                "labels": inputs.LABEL_RECIPE} if w.kind == "vocab_ce" else {}),
            **({"vocab": w.F, "vocab_padded": tp.tp_vocab_padded(w.F, w.N), "ids": inputs.ID_RECIPE,
                "bytes_counted": "ids per shard, each token's row once, N partials in the table's type "
                                 "written and read, the rows written"} if w.kind == "vocab_embed" else {}),
            **({"norm": "layernorm" if w.kind == "norm_split_layer" else "rmsnorm", "eps": inputs.NORM_EPS,
                "features_per_shard": w.H // w.N,
                "bytes_counted": "each kernel's inputs read once and outputs written once: the slices twice "
                                 "(statistics, then scaling), the outputs once, the statistics slab written "
                                 "once and read N times per (shard, row), gain (and shift)"}
               if w.kind.startswith("norm_split") else {}),
            "share": "all shards + reduction" if args.share == "layer" else "rank 0 shard + reduction",
            "reduce_scatter_slices": w.n_slices, "seed": w.seed,
            **({"sp_entry": {"norm": "layernorm" if args.sp_entry == "layer" else "rmsnorm", "eps": inputs.NORM_EPS,
                             "gain": inputs.NORM_GAIN_RECIPE,
                             **({"shift": inputs.NORM_SHIFT_RECIPE} if args.sp_entry == "layer" else {})}}
               if args.sp_entry else {}),
            **({"overlap_chunks": args.overlap} if args.overlap else {}),
            **({"pass": "backward", "upstream_gradient": inputs.GRAD_RECIPE,
                "flop_counted": ("12*T*H*I (dH, dX, fused dA, dB)" if w.kind == "mlp_swiglu" else
                                 "8*T*H*F (dH, dX, dA, dB)")
                                + ("; the recomputed column product is extra and not counted"
                                   if bmode == "recompute" else ""),
                "preactivation": ("stored by a training forward before the timed region (bf16 Z, read by the dZ "
                                  "epilogue)" if bmode == "stored" else "recomputed in every step (X A^T + a)"),
                **({"activation": "stored by the same forward (bf16 GELU(Z), the B operand of dB)"}
                   if bmode == "stored" and stored_activation(w) else {}),
                "operands": ("read as stored (K-outer GEMM operands, column sums for the bias gradients)"
                             if backward_direct(w) else "transposed first"),
                "split_k": backward_splits(w.T, 2 * w.F if w.kind == "mlp_swiglu" else w.F, w.H,
                                           backward_direct(w))}
               if args.backward else {}),
        },
        "pct_of_bf16_mfma_peak": (round(100 * value * 1e12 / PEAK_BF16, 2)
                                  if w.dtype == "bf16" and not bytes_metric else None),
        **({"pct_of_hbm_peak": round(100 * value * 1e9 / PEAK_HBM, 2)} if bytes_metric else {}),
        "roofline": roof,
        "kernels": kernels,
        "kernel_source_hash": src_hash,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        del d, Y, ws
        if args.backward:
            del grads, dY
        torch.cuda.empty_cache()
        log(f"cpu baseline: fp64 oracle for ~{args.cpu_seconds:.0f} s")
        if args.backward:
            out["cpu_baseline"] = cpu_baseline_backward(w, host, dY_host, args.cpu_seconds)
        else:
            out["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
