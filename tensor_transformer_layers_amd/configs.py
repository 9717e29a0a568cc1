"""The five workloads of the tensor-parallel linear pair, as plain data.

Shapes follow the pages' model sizes: the 12-layer hidden-512 / MLP-2048
model of the measured table on "大模型分布式训练篇——从零实现 Tensor Para..."
(its results section), the 7B / batch 8 / seq 4096 case of "张量并行"
(its all-reduce volume paragraph), and the 175B (GPT-3) layer of the same page
(its per-layer memory paragraph).

Token order:
  * MLP workloads use sequence-major rows (row = s * batch + b), the layout of
    the sequence-parallel region, so reduce-scatter slice r (contiguous rows)
    holds sequence positions [r*seq/n, (r+1)*seq/n) of every sequence.  The MLP
    is token-wise, so the order changes where a token sits, not its value.
  * The attention workload uses batch-major rows (row = b * seq + s).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    kind: str               # "mlp_gelu" | "mlp_swiglu" | "attn" | "vocab_ce" | "vocab_embed" |
                            # "norm_split_layer" | "norm_split_rms"
    dtype: str              # "f32" | "bf16"  (inputs; accumulation is fp32)
    batch: int
    seq: int
    H: int                  # hidden
    F: int                  # FFN / intermediate (attention: unused, = H; vocab_*: the vocab size)
    N: int                  # tensor-parallel shards
    sigma_x: float = 1.0
    sigma_w: float = 0.02
    sigma_bias: float | None = None   # None: no biases
    heads: int = 0
    head_dim: int = 0
    n_slices: int = 1       # >1: reduce-scatter along the sequence
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def T(self) -> int:
        return self.batch * self.seq

    @property
    def Fs(self) -> int:
        return self.F // self.N

    # algorithmic work -------------------------------------------------------
    def flops_shard(self) -> float:
        """FLOP of one shard's column GEMM + attention + row GEMM (multiply
        and add counted as 2).  Causal attention counts the lower triangle
        with the diagonal: 4 * d * S(S+1)/2 per (batch, head)."""
        T, H = self.T, self.H
        if self.kind == "vocab_embed":  # a lookup: no arithmetic
            return 0.0
        if self.kind.startswith("norm_split"):  # HBM-bound: measured in bytes, not FLOP
            return 0.0
        if self.kind == "vocab_ce":  # the head's product over the real vocab, one shard's share
            return 2.0 * T * H * self.F / self.N
        if self.kind == "mlp_gelu":
            return 2.0 * T * H * self.Fs * 2
        if self.kind == "mlp_swiglu":
            return 2.0 * T * H * (2 * self.Fs) + 2.0 * T * self.Fs * H
        hl = self.heads // self.N
        wqkv = 2.0 * T * H * (3 * hl * self.head_dim)
        attn = self.batch * hl * 4.0 * self.head_dim * self.seq * (self.seq + 1) / 2
        wo = 2.0 * T * (hl * self.head_dim) * H
        return wqkv + attn + wo

    def flops_layer(self) -> float:
        return self.flops_shard() * self.N


CONFIGS: dict[int, Workload] = {
    1: Workload(1, "gelu_mlp_f32_T128_H512_F2048_N2", "mlp_gelu", "f32",
                batch=1, seq=128, H=512, F=2048, N=2,
                sigma_w=0.02, sigma_bias=0.02, seed=20260001),
    2: Workload(2, "gelu_mlp_bf16_T16384_H512_F2048_N4", "mlp_gelu", "bf16",
                batch=8, seq=2048, H=512, F=2048, N=4,
                sigma_w=0.02, sigma_bias=0.02, seed=20260002),
    3: Workload(3, "swiglu_mlp_bf16_T32768_H4096_I11008_N8", "mlp_swiglu", "bf16",
                batch=8, seq=4096, H=4096, F=11008, N=8,
                sigma_w=0.02, sigma_bias=None, seed=20260003),
    4: Workload(4, "attn_bf16_B2_S4096_H4096_h32x128_N8", "attn", "bf16",
                batch=2, seq=4096, H=4096, F=4096, N=8, heads=32, head_dim=128,
                sigma_w=0.02, sigma_bias=None, seed=20260004),
    5: Workload(5, "gelu_mlp_bf16_T16384_H12288_F49152_N8_rs8", "mlp_gelu", "bf16",
                batch=8, seq=2048, H=12288, F=49152, N=8, n_slices=8,
                sigma_w=0.01, sigma_bias=0.01, seed=20260005),
}

# Beyond the five: the vocab-parallel output head and cross-entropy of the
# blog post at 2kiu.com (section 6.2) at the 7B hidden size, with the
# ~150k-entry vocab "张量并行" names in its vocab-parallel paragraph (not a
# multiple of 8 shards x 8, so it is padded), 8 x 2048 tokens.
EXTRA: dict[int, Workload] = {
    6: Workload(6, "vocab_ce_bf16_T16384_H4096_V150000_N8", "vocab_ce", "bf16",
                batch=8, seq=2048, H=4096, F=150000, N=8,
                sigma_w=0.02, sigma_bias=None, seed=20260006),
    # the input side of the same split: the vocab-parallel embedding lookup
    # of those 8 x 2048 tokens in the same padded 150k x 4096 table
    7: Workload(7, "vocab_embed_bf16_T16384_H4096_V150000_N8", "vocab_embed", "bf16",
                batch=8, seq=2048, H=4096, F=150000, N=8,
                sigma_w=0.02, sigma_bias=None, seed=20260007),
}


# The norm at a sublayer boundary when its input stays split along hidden
# (the blog post at 2kiu.com, section 3.3): the 175B-shaped layer's hidden
# size, 12288, over 8 shards (1536 features each), 8 x 2048 tokens.  Gain
# 1 + N(0, 0.1^2); LayerNorm shift N(0, 0.1^2).
EXTRA[8] = Workload(8, "layernorm_split_bf16_T16384_H12288_N8", "norm_split_layer", "bf16",
                    batch=8, seq=2048, H=12288, F=12288, N=8, sigma_bias=0.1, seed=20260008)
EXTRA[9] = Workload(9, "rmsnorm_split_bf16_T16384_H12288_N8", "norm_split_rms", "bf16",
                    batch=8, seq=2048, H=12288, F=12288, N=8, sigma_bias=None, seed=20260009)


def workload(key: int) -> Workload:
    """Workload ``key``: one of the five of the path, or an extra one."""
    if key in CONFIGS:
        return CONFIGS[key]
    return EXTRA[key]


def scaled(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some fields replaced (small parity cases)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(kw)
    return Workload(**d)
