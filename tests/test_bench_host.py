"""Host logic of bench.py (no GPU): the per-kernel algorithmic work adds up to
the workload's FLOP count, the launch-order tables match the library's
dispatch rules, and the rocprofv3 summaries are parsed and scaled right
(synthetic counter files)."""
import csv
import os

import pytest

import bench
from tensor_transformer_layers_amd import configs


@pytest.mark.parametrize("k", [2, 3, 4, 5, 6])
def test_kernel_flops_add_up_to_the_workload(k):
    w = configs.workload(k)
    order = bench.launch_order(w)
    total = sum(bench.kernel_work(w, name, w.N, w.T)[0] for name in dict.fromkeys(order))
    assert abs(total - w.flops_layer()) <= 1e-9 * w.flops_layer()


def test_embedding_bytes_and_cpu_baseline():
    """The embedding step's algorithmic bytes: ids once per shard, each row
    read once, N partials (bf16, the table's type) written, then read by
    the fold, and the rows written.  The CPU baseline runs the oracle on a small copy of the
    workload and reports GB/s with those bytes per token."""
    w = configs.workload(7)
    assert bench.launch_order(w) == ["vocab_embed_partial", "vocab_embed_fold"]
    T, H, N = w.T, w.H, w.N
    total = sum(bench.kernel_work(w, n, N, T)[1] for n in bench.launch_order(w))
    assert total == 4 * N * T + 2 * T * H + 2 * N * T * H + 2 * N * T * H + 2 * T * H
    assert w.flops_layer() == 0.0
    from tensor_transformer_layers_amd import inputs
    small = configs.scaled(w, batch=1, seq=4096, H=64, F=1000)
    host = inputs.make_inputs(small)
    assert host["ids"].dtype.name == "int32" and host["ids"].max() < 1000
    cb = bench.cpu_baseline(small, host, 0.2)
    assert cb["unit"] == "GB/s" and cb["value"] > 0 and cb["kind"] == "oracle"


@pytest.mark.parametrize("k", [2, 3, 5])
def test_backward_kernel_flops_cover_the_counted_work(k):
    """The FLOP of the launched GEMMs minus the recomputed column product
    equals the counted backward FLOP (fused two-pass kernel or not); with the
    stored pre-activation the launched GEMMs are exactly the counted work."""
    w = configs.workload(k)
    order = bench.backward_launch_order(w, "recompute")
    assert ("bwd_fused_gemm" in order) == (k == 2)
    total = sum(bench.kernel_work(w, n, w.N, w.T)[0] * order.count(n) for n in dict.fromkeys(order))
    fz = 2 * w.F if w.kind == "mlp_swiglu" else w.F
    recompute = 2.0 * w.T * w.H * fz
    assert abs(total - recompute - bench.backward_flops(w, w.N)) <= 1e-9 * total
    assert bench.backward_mode(w, False) == "stored"
    if bench.backward_mode(w, False) == "stored":
        order = bench.backward_launch_order(w, "stored")
        assert "bwd_recompute_gemm" not in order and "bwd_fused_gemm" not in order
        total = sum(bench.kernel_work(w, n, w.N, w.T)[0] * order.count(n) for n in dict.fromkeys(order))
        assert abs(total - bench.backward_flops(w, w.N)) <= 1e-9 * total
        assert bench.workload_tag(w, backward="stored").endswith("_backward")
        assert bench.workload_tag(w, backward="recompute").endswith("_backward_recompute")


def test_fused_path_rule():
    assert bench.launch_order(configs.workload(2)) == ["mlp_fused", "reduce_partials"]
    assert bench.launch_order(configs.workload(5), sp_entry=True)[0] == "rmsnorm_gather"
    assert bench.launch_order(configs.workload(3))[:2] == ["mlp_column_gemm", "mlp_row_gemm"]


def _write_counters(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                           "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(r)


def test_traffic_summary_scales_by_the_copy(tmp_path):
    """Two steps of workload 2 (fused kernel, then the fold) plus the set-up
    copy and the 1 GiB calibration copy, whose counters read 2x (FETCH) and
    1x (WRITE) its size."""
    w = configs.workload(2)
    for counter, per_kib, copy_kib in (("FETCH_SIZE", {"fused": 1000.0, "fold": 500.0}, 2 * 2 ** 20),
                                       ("WRITE_SIZE", {"fused": 300.0, "fold": 100.0}, 2 ** 20)):
        rows = [{"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 99999999,
                 "Counter_Name": counter, "Counter_Value": 5.0}]
        d = 2
        for _ in range(2):
            rows.append({"Dispatch_Id": d, "Kernel_Name": "void tp::(anonymous namespace)::mlp_fused_kernel<x>",
                         "Grid_Size": 1, "Counter_Name": counter, "Counter_Value": per_kib["fused"]})
            rows.append({"Dispatch_Id": d + 1, "Kernel_Name": "void tp::(anonymous namespace)::reduce_kernel<y>",
                         "Grid_Size": 1, "Counter_Name": counter, "Counter_Value": per_kib["fold"]})
            d += 2
        rows.append({"Dispatch_Id": d, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 1024,
                     "Counter_Name": counter, "Counter_Value": copy_kib})
        _write_counters(str(tmp_path / "pmc" / counter / "run_counter_collection.csv"), rows)
    path = bench.write_traffic(w, "layer", str(tmp_path / "pmc"), "ARGS", out_dir=str(tmp_path))
    vals = {l.split()[1]: float(l.split()[2]) for l in open(path) if l.startswith("traffic_bytes")}
    # FETCH scaled by 1/2, WRITE by 1: fused 500 + 300 KiB, fold 250 + 100 KiB
    assert vals["mlp_fused"] == pytest.approx(800 * 1024)
    assert vals["reduce_partials"] == pytest.approx(350 * 1024)


def test_traffic_summary_rejects_a_wrong_launch_order(tmp_path):
    w = configs.workload(2)
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = [{"Dispatch_Id": 1, "Kernel_Name": "void tp::(anonymous namespace)::reduce_kernel<y>",
                 "Grid_Size": 1, "Counter_Name": counter, "Counter_Value": 1.0},
                {"Dispatch_Id": 2, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 1,
                 "Counter_Name": counter, "Counter_Value": 1.0}]
        _write_counters(str(tmp_path / "pmc" / counter / "run_counter_collection.csv"), rows)
    with pytest.raises(RuntimeError, match="expected mlp_fused"):
        bench.write_traffic(w, "layer", str(tmp_path / "pmc"), "ARGS", out_dir=str(tmp_path))


def test_mfma_summary(tmp_path):
    w = configs.workload(5)
    rows = []
    d = 1
    alg_col = bench.kernel_work(w, "mlp_column_gemm", w.N, w.T)[0]
    for name, flop, util in (("gemm_bf16_kernel<G<256>>", alg_col, 60.0), ("gemm_bf16_kernel<G<256>>", alg_col, 70.0),
                             ("reduce_kernel<z>", 0.0, 0.0)):
        for cn, v in (("MfmaFlopsBF16", flop), ("MfmaUtil", util)):
            rows.append({"Dispatch_Id": d, "Kernel_Name": f"void tp::(anonymous namespace)::{name}", "Grid_Size": 1,
                         "Counter_Name": cn, "Counter_Value": v})
        d += 1
    _write_counters(str(tmp_path / "m" / "run_counter_collection.csv"), rows)
    path = bench.write_mfma(w, "layer", str(tmp_path / "m"), "ARGS", out_dir=str(tmp_path))
    lines = {l.split()[1]: l.split() for l in open(path) if l.startswith("# mlp_") or l.startswith("# reduce")}
    assert float(lines["mlp_column_gemm"][4]) == pytest.approx(1.0)
    assert float(lines["mlp_column_gemm"][5]) == pytest.approx(60.0)
    assert float(lines["mlp_row_gemm"][5]) == pytest.approx(70.0)


def test_stored_backward_summaries_skip_the_set_up_forward(tmp_path):
    """The stored-pre-activation backward starts with one training forward
    (column GEMM writing Z, row GEMM, reduction): the converters check and
    drop those dispatches before matching steps, so a summary sees whole
    backward steps only; a run without them is rejected."""
    w = configs.workload(2)
    order = bench.backward_launch_order(w, "stored")
    assert bench.setup_launches(w, "stored") == ["mlp_column_gemm", "mlp_row_gemm", "reduce_partials"]
    assert bench.setup_launches(w, "recompute") == []
    sym = {"mlp_column_gemm": "gemm_bf16_kernel<G0>", "mlp_row_gemm": "gemm_bf16_kernel<G0>",
           "reduce_partials": "reduce_kernel<r>"}
    names = [sym[k] for k in bench.setup_launches(w, "stored")]
    for _ in range(2):
        names += [bench.KERNEL_SYMBOL[k] + "<x>" for k in order]
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = [{"Dispatch_Id": i + 1, "Kernel_Name": f"void tp::(anonymous namespace)::{n}", "Grid_Size": 1,
                 "Counter_Name": counter, "Counter_Value": 7.0 if i < 3 else 1.0} for i, n in enumerate(names)]
        rows.append({"Dispatch_Id": len(names) + 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 1,
                     "Counter_Name": counter, "Counter_Value": 2 ** 20})
        _write_counters(str(tmp_path / "pmc" / counter / "run_counter_collection.csv"), rows)
    path = bench.write_traffic(w, "layer", str(tmp_path / "pmc"), "ARGS", backward="stored", out_dir=str(tmp_path))
    vals = {l.split()[1]: float(l.split()[2]) for l in open(path) if l.startswith("traffic_bytes")}
    assert set(vals) == set(order)
    # every backward dispatch read 1 KiB x (2^30 / 2^30) and wrote 1 KiB; the set-up's 7 KiB never enter
    assert all(v == pytest.approx(2 * 1024) for v in vals.values())
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = [{"Dispatch_Id": i + 1, "Kernel_Name": f"void tp::(anonymous namespace)::{n}", "Grid_Size": 1,
                 "Counter_Name": counter, "Counter_Value": 1.0} for i, n in enumerate(names[3:])]
        rows.append({"Dispatch_Id": len(names) + 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": 1,
                     "Counter_Name": counter, "Counter_Value": 2 ** 20})
        _write_counters(str(tmp_path / "pmc2" / counter / "run_counter_collection.csv"), rows)
    with pytest.raises(RuntimeError, match="set-up dispatch"):
        bench.write_traffic(w, "layer", str(tmp_path / "pmc2"), "ARGS", backward="stored", out_dir=str(tmp_path))
