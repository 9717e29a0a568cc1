"""The overlapped forward (reduction of row block k on a second stream while
block k+1 computes) gives the same bits as the plain forward, through the C
ABI (gfx950 GPU required)."""
import sys

import numpy as np
import pytest

from tensor_transformer_layers_amd import configs, inputs, tp, workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


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
    assert torch.equal(Yo.view(view), Y.view(view))
    assert torch.equal(Yo2.view(view), Y.view(view))


def test_overlap_full_size_workload_2():
    w = configs.CONFIGS[2]
    host = inputs.make_inputs(w)
    d = workloads.device_inputs(w, host)
    Y, ws = workloads.forward(w, d)
    s2 = torch.cuda.Stream()
    for chunks in (2, 4):
        Yo, _ = workloads.forward_overlap(w, d, chunks, s2, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(Yo.view(torch.int16), Y.view(torch.int16)), chunks
