"""The allocation-free MLP forward (tp_mlp_forward_noalloc: the workspace is
the library's static per-GPU scratch) against the workspace entry point
tp_mlp_forward, through the C ABI (gfx950 GPU required).

Both run the same kernels on the same inputs, so their outputs must agree
bit for bit; each call is also held to the oracle's bf16 / fp32 tolerance.
Two calls in a row, the second smaller than the first: the scratch keeps the
first call's contents, and the second must not depend on them."""
import sys

import numpy as np
import pytest

from oracle import reference as R
from tensor_transformer_layers_amd import configs, inputs, tp, workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

BF16_TOL = 2e-2
F32_TOL = 1e-4


def say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    return float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def _bits(Y):
    return Y.view(torch.int16) if Y.dtype == torch.bfloat16 else Y.view(torch.int32)


# (first call, second smaller call): the GEMM path, the fused narrow-hidden
# kernel, SwiGLU, fp32, and a reduce-scatter slice
PAIRS = [
    ("gemm_gelu", configs.scaled(configs.CONFIGS[5], batch=4, seq=256, H=1024, F=8 * 256, n_slices=4, seed=41),
     configs.scaled(configs.CONFIGS[5], batch=2, seq=136, H=264, F=8 * 64, n_slices=2, seed=42)),
    ("fused_gelu", configs.scaled(configs.CONFIGS[2], batch=2, seq=1024, H=512, F=4 * 256, seed=43),
     configs.scaled(configs.CONFIGS[2], batch=1, seq=300, H=256, F=4 * 64, seed=44)),
    ("swiglu", configs.scaled(configs.CONFIGS[3], batch=1, seq=1024, H=512, F=8 * 64, seed=45),
     configs.scaled(configs.CONFIGS[3], batch=1, seq=200, H=256, F=8 * 40, seed=46)),
    ("f32", configs.scaled(configs.CONFIGS[1], batch=1, seq=256, H=512, F=2 * 512, seed=47),
     configs.scaled(configs.CONFIGS[1], batch=1, seq=64, H=128, F=2 * 96, seed=48)),
]


def _noalloc(w, d, slice=-1):
    return tp.mlp_forward_noalloc(d["X"], d["A"], d["a"], d["B"], d["b"], w.N, act=workloads.act_of(w),
                                  n_slices=w.n_slices, slice=slice)


@pytest.mark.parametrize("name,big,small", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_matches_workspace_entry_point(name, big, small):
    for w in (big, small):
        say(f"noalloc {name}: T={w.T} H={w.H} F={w.F} N={w.N} slices={w.n_slices}")
        host = inputs.make_inputs(w)
        d = workloads.device_inputs(w, host)
        Yb = torch.empty((w.T, w.H), dtype=d["X"].dtype, device=d["X"].device)
        d_ws = tp.mlp_desc(d["X"], d["A"], d["a"], d["B"], d["b"], w.N, workloads.act_of(w), Yb)
        assert 0 < tp.tp_mlp_workspace_size(d_ws) <= tp.NOALLOC_SCRATCH_BYTES
        Y_ref, _ = workloads.forward(w, d)  # the workspace entry point
        Y = _noalloc(w, d)
        torch.cuda.synchronize()
        assert torch.equal(_bits(Y), _bits(Y_ref)), "differs from tp_mlp_forward"
        ref = R.workload(w.kind, host, w.batch, w.seq, w.heads)
        e = err(Y.float().cpu().numpy(), ref)
        say(f"  err vs oracle {e:.3e}")
        assert e <= (F32_TOL if w.dtype == "f32" else BF16_TOL)
        if w.n_slices > 1:  # one reduce-scatter slice into a slice-sized Y
            r = w.n_slices - 1
            Ys = _noalloc(w, d, slice=r)
            torch.cuda.synchronize()
            s = w.T // w.n_slices
            assert torch.equal(_bits(Ys), _bits(Y_ref[r * s:(r + 1) * s]))


def test_noalloc_rejects_a_workspace_beyond_its_scratch():
    """A problem whose workspace exceeds the static scratch fails with a
    clear error before any launch, and the next call still works."""
    w = configs.scaled(configs.CONFIGS[2], batch=1, seq=4096, H=1024, F=4 * 512, seed=49)
    host = inputs.make_inputs(w)
    d = workloads.device_inputs(w, host)
    Yb = torch.empty((w.T, w.H), dtype=d["X"].dtype, device=d["X"].device)
    desc = tp.mlp_desc(d["X"], d["A"], d["a"], d["B"], d["b"], w.N, tp.TP_ACT_GELU, Yb)
    assert tp.tp_mlp_workspace_size(desc) > tp.NOALLOC_SCRATCH_BYTES
    with pytest.raises(tp.TPError, match="static scratch"):
        _noalloc(w, d)
    small = configs.scaled(w, seq=256, seed=50)
    host = inputs.make_inputs(small)
    d = workloads.device_inputs(small, host)
    Y_ref, _ = workloads.forward(small, d)
    Y = _noalloc(small, d)
    torch.cuda.synchronize()
    assert torch.equal(_bits(Y), _bits(Y_ref))
