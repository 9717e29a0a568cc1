"""The checklist test of the pages: the same layer, same seed, with TP=1 and
with TP=N gives the same result up to the order of the float sums (the blog
post at 2kiu.com, section 6.4; "张量并行", practice section: a small, stable
difference from the single-GPU result; a large one means a sharding bug).

Through the C ABI (gfx950 GPU required).  bf16 outputs may differ by one
rounding step where the fp32 sums of the two orders straddle a bf16 boundary,
so the bound is 2^-7 of max|Y| (two bf16 steps), far below any sharding bug
(a wrong block or a doubled bias moves the result by O(1) of max|Y|).
"""
import numpy as np
import pytest

from tensor_transformer_layers_amd import configs, inputs, tp, workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

BOUND = 2.0 ** -7


def _rel(a, b):
    a, b = a.float(), b.float()
    return float((a - b).abs().max() / b.abs().max())


@pytest.mark.parametrize("base,kw", [
    (2, dict(batch=1, seq=1024, H=512, F=2048)),   # fused narrow-hidden kernel
    (5, dict(batch=2, seq=256, H=768, F=3072, n_slices=1)),
    (3, dict(batch=1, seq=512, H=512, F=8 * 64)),
])
def test_mlp_tp1_equals_tpn(base, kw):
    w8 = configs.scaled(configs.CONFIGS[base], seed=41, **kw)
    w1 = configs.scaled(w8, N=1)
    host = inputs.make_inputs(w8)
    Y8, _ = workloads.forward(w8, workloads.device_inputs(w8, host))
    Y1, _ = workloads.forward(w1, workloads.device_inputs(w1, host))
    torch.cuda.synchronize()
    r = _rel(Y8, Y1)
    assert r <= BOUND, r


def test_attention_tp1_equals_tpn():
    w4 = configs.scaled(configs.CONFIGS[4], batch=1, seq=512, H=1024, F=1024, heads=8, N=4, seed=42)
    w1 = configs.scaled(w4, N=1)
    host = inputs.make_inputs(w4)
    Y4, _ = workloads.forward(w4, workloads.device_inputs(w4, host))
    Y1, _ = workloads.forward(w1, workloads.device_inputs(w1, host))
    torch.cuda.synchronize()
    assert _rel(Y4, Y1) <= BOUND


def test_backward_tp1_equals_tpn():
    w4 = configs.scaled(configs.CONFIGS[2], batch=1, seq=1024, H=256, F=1024, seed=43)
    w1 = configs.scaled(w4, N=1)
    host = inputs.make_inputs(w4)
    dY = torch.from_numpy(inputs.grad_output(w4)).to("cuda", torch.bfloat16)
    g4, _ = workloads.backward(w4, workloads.device_inputs(w4, host), dY)
    g1, _ = workloads.backward(w1, workloads.device_inputs(w1, host), dY)
    torch.cuda.synchronize()
    for k in ("dX", "dA", "da", "dB", "db"):
        assert _rel(g4[k], g1[k]) <= BOUND, k


def test_vocab_ce_tp1_equals_tpn():
    rng = np.random.default_rng(44)
    T, H, V = 512, 256, 10007
    X = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to("cuda", torch.bfloat16)
    E = (rng.standard_normal((V, H)) * 0.05).astype(np.float32)
    labels = torch.from_numpy(rng.integers(0, V, T).astype(np.int32)).to("cuda")
    out = {}
    for N in (1, 8):
        Ep = np.zeros((tp.tp_vocab_padded(V, N), H), dtype=np.float32)
        Ep[:V] = E
        loss, _, _ = tp.vocab_ce_forward(X, torch.from_numpy(Ep).to("cuda", torch.bfloat16), labels, V, N)
        out[N] = loss
    torch.cuda.synchronize()
    # fp32 loss: only the summation order differs
    assert _rel(out[8], out[1]) <= 1e-5
