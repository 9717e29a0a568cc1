"""The overlapped forward (reduction of row block k on a second stream while
block k+1 computes; "大模型分布式训练篇——从零实现 Tensor Para...", section 三:
overlap the communication with computation) against the fp64 CPU oracle,
and bit for bit against the plain forward, through the C ABI (gfx950 GPU
required).

Tolerances as for the plain forward: bf16 max|Y - O| / max|O| <= 2e-2,
fp32 <= 1e-4."""
import sys

import numpy as np
import pytest

from oracle import reference as R
from tensor_transformer_layers_amd import configs, inputs, tp, workloads

BF16_TOL = 2e-2
F32_TOL = 1e-4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


CASES = {
    "fused_gelu": configs.scaled(configs.CONFIGS[2], batch=1, seq=1024, H=512, F=4 * 128, seed=31),
    "gemm_gelu": configs.scaled(configs.CONFIGS[5], batch=2, seq=264, H=264, F=8 * 64, n_slices=1, seed=32),
    "swiglu": configs.scaled(configs.CONFIGS[3], batch=1, seq=600, H=512, F=8 * 40, seed=33),
    "f32": configs.scaled(configs.CONFIGS[1], batch=1, seq=96, H=64, F=2 * 96, seed=34),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("chunks", [1, 2, 4, 8])
def test_overlap_is_bit_identical(name, chunks):
    w = CASES[name]
    if w.T % chunks:
        pytest.skip("T not divisible")
    say(f"overlap {name} T={w.T} chunks={chunks}")
    host = inputs.make_inputs(w)
    d = workloads.device_inputs(w, host)
    Y, ws = workloads.forward(w, d)
    s2 = torch.cuda.Stream()
    Yo, _ = workloads.forward_overlap(w, d, chunks, s2)
    Yo2, _ = workloads.forward_overlap(w, d, chunks, s2, ws=ws)
    torch.cuda.synchronize()
    view = torch.int16 if Y.dtype == torch.bfloat16 else torch.int32
    # against the oracle (the unsharded layer in fp64), on every case and
    # block count, before the comparison with the plain forward: a mistake
    # shared by both paths, or in how the blocks are put together, shows here
    ref = R.workload(w.kind, host, w.batch, w.seq, w.heads)
    e = err(Yo.float().cpu().numpy(), ref)
    say(f"  err vs oracle {e:.3e}")
    assert e <= (F32_TOL if w.dtype == "f32" else BF16_TOL)
    assert torch.equal(Yo.view(view), Y.view(view))
    assert torch.equal(Yo2.view(view), Y.view(view))


def test_overlap_full_size_workload_2():
    """The hidden-512 workload at full size (16384 tokens, 4 shards): every
    row against the fp64 oracle, and bit for bit against the plain forward."""
    w = configs.CONFIGS[2]
    say(f"overlap full size {w.name}")
    host = inputs.make_inputs(w)
    d = workloads.device_inputs(w, host)
    Y, ws = workloads.forward(w, d)
    s2 = torch.cuda.Stream()
    ref = R.workload(w.kind, host, w.batch, w.seq, w.heads)
    for chunks in (2, 4):
        Yo, _ = workloads.forward_overlap(w, d, chunks, s2, ws=ws)
        torch.cuda.synchronize()
        e = err(Yo.float().cpu().numpy(), ref)
        say(f"  chunks={chunks} err vs oracle {e:.3e}")
        assert e <= BF16_TOL, chunks
        assert torch.equal(Yo.view(torch.int16), Y.view(torch.int16)), chunks
