"""Host logic of the benchmark, on the CPU: which kernel a profiled
dispatch counts for, the algorithmic bytes of the quantize launches, the
HBM bytes per launch from rocprofv3 counter CSVs scaled by the copy
calibration, and the order in which a step issues its calls.  No GPU and
no kernel call."""

import csv

import pytest

import bench
from scaled_quantize_fp8_amd import workloads as WL

GEMM3 = "void fp8l::gemm3_kernel<128, 128, 2, 2, {}>(fp8l::GemmArgs)"
GEMM4 = "void fp8l::gemm4_kernel<{}, 0, 0>(fp8l::GemmArgs)"
GEMM5 = "void fp8l::gemm5_kernel<{}>(fp8l::GemmArgs)"


@pytest.mark.parametrize("ops,kind", [("0, 0, 0, 0", "fwd"), ("0, 1, 1, 0", "dx"),
                                      ("1, 1, 1, 0", "dw"), ("1, 0, 0, 1", None)])
def test_gemm_kind_of_operand_args(ops, kind):
    assert bench.gemm_kind_of(GEMM4.format(ops)) == kind
    assert bench.gemm_kind_of(GEMM5.format(ops)) == kind
    # gemm3: the operand arguments follow BM, BN, WGM, WGN; with and without
    # the trailing epilogue mode and output format (bf16 epilogue = 0)
    assert bench.gemm_kind_of(GEMM3.format(ops)) == kind
    assert bench.gemm_kind_of(GEMM3.format(ops + ", 0, 0")) == kind


def test_gemm_kind_of_excludes_other_kernels():
    # an FP8-output epilogue (mode 1..3) is not one of the three linear GEMMs
    for epi in (1, 2, 3):
        assert bench.gemm_kind_of(GEMM3.format(f"0, 0, 0, 0, {epi}, 0")) is None
    for name in ("void fp8l::quantize_flat_kernel<2, 0, 0>(fp8l::QArgs)",
                 "void fp8l::amax_ring_kernel<2>(void const*, long, int, fp8l::RingHdr*)",
                 "__amd_rocclr_copyBuffer", "void fp8l::gemm6_kernel<0, 0, 0, 0>(x)"):
        assert bench.gemm_kind_of(name) is None


# (K, N) of the dim1536 layer's five linears: qkv, out, up, gate, down
_DIM1536 = [(1536, 4608), (1536, 1536), (1536, 6912), (1536, 6912), (6912, 1536)]


def test_quant_launch_bytes_counts_whole_steps():
    M = 2048
    xw = sum(3 * (M * K + N * K) for K, N in _DIM1536)   # bf16 in, one fp8 byte out
    g = sum(3 * M * N for K, N in _DIM1536)
    # 3 steps of 15 launches after the seeding step's 10 (its G is quantized
    # by the column-sum kernel, which is not a flat-quantize dispatch)
    assert bench.quant_launch_bytes("dim1536_m2048", 55) == pytest.approx(
        (3 * (xw + g) + xw) / 55, rel=1e-12)
    for bad in (54, 10, 9):
        with pytest.raises(SystemExit):
            bench.quant_launch_bytes("dim1536_m2048", bad)


_FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Kernel_Name", "Counter_Name",
           "Counter_Value"]


def _pmc_csv(path, counter, dispatches):
    """A rocprofv3 --pmc CSV: one row per (dispatch, per-XCD part) of the
    counter, plus a row of another counter that must be ignored."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=_FIELDS)
        w.writeheader()
        for d, (name, parts) in enumerate(dispatches, start=1):
            for v in parts:
                w.writerow({"Correlation_Id": d, "Dispatch_Id": d, "Agent_Id": "Agent 1",
                            "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})
            w.writerow({"Correlation_Id": d, "Dispatch_Id": d, "Agent_Id": "Agent 1",
                        "Kernel_Name": name, "Counter_Name": "GRBM_COUNT", "Counter_Value": 1e9})
    return str(path)


def test_traffic_record_scales_by_copy_calibration(tmp_path):
    fwd = GEMM4.format("0, 0, 0, 0")
    dx = GEMM5.format("0, 1, 1, 0")
    copy = "__amd_rocclr_copyBuffer"
    fill = "void at::native::vectorized_elementwise_kernel<4>(int)"
    # the forward kernel: two dispatches, values split over rows and summed
    fetch = _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE",
                     [(fwd, [1000.0, 2000.0]), (dx, [9e9]), (fwd, [5000.0]), (fill, [1.0])])
    write = _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE",
                     [(fwd, [300.0]), (dx, [9e9]), (fwd, [100.0, 100.0])])
    cb = bench.COPY_BYTES
    # the copy reads 2x what it moves by this counter and writes it 1x; the
    # largest dispatch is the calibration copy
    cfetch = _pmc_csv(tmp_path / "cf.csv", "FETCH_SIZE",
                      [(fill, [4.0]), (copy, [2 * cb / 1024 / 2] * 2), (copy, [7.0])])
    cwrite = _pmc_csv(tmp_path / "cw.csv", "WRITE_SIZE", [(copy, [cb / 1024]), (fill, [3.0])])
    rec = bench.traffic_record("fwd", fetch, write, cfetch, cwrite, "dim1536_m2048")
    assert rec["dispatches"] == [2, 2]
    assert rec["fetch_kib_raw"] == 4000.0 and rec["write_kib_raw"] == 250.0
    assert rec["fetch_scale"] == pytest.approx(0.5) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_read_bytes_per_launch"] == pytest.approx(4000.0 * 1024 * 0.5)
    assert rec["hbm_write_bytes_per_launch"] == pytest.approx(250.0 * 1024)
    assert rec["hbm_bytes_per_launch"] == pytest.approx((2000.0 + 250.0) * 1024)
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()
    assert "algorithmic_bytes_per_launch" not in rec
    assert all("rocprofv3 --pmc" in c for c in rec["commands"][1:5])


def test_traffic_record_quant_and_missing_kernel(tmp_path):
    q = "void fp8l::quantize_flat_kernel<2, 0, 1>(fp8l::QArgs)"
    pair = "void fp8l::quantize_flat2_kernel<2, 0>(fp8l::QArgs, fp8l::QArgs, unsigned int)"
    copy = "__amd_rocclr_copyBuffer"
    cb = bench.COPY_BYTES
    fetch = _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", [(q, [10.0])] * 55 + [(pair, [1e6])])
    write = _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", [(q, [5.0])] * 55)
    cf = _pmc_csv(tmp_path / "cf.csv", "FETCH_SIZE", [(copy, [cb / 1024])])
    cw = _pmc_csv(tmp_path / "cw.csv", "WRITE_SIZE", [(copy, [cb / 1024])])
    rec = bench.traffic_record("quant", fetch, write, cf, cw, "dim1536_m2048")
    assert rec["dispatches"] == [55, 55]
    assert rec["hbm_bytes_per_launch"] == pytest.approx(15.0 * 1024)
    assert rec["algorithmic_bytes_per_launch"] == pytest.approx(
        bench.quant_launch_bytes("dim1536_m2048", 55))
    # a CSV without the kernel is an error, not a zero
    with pytest.raises(SystemExit):
        bench.traffic_record("dx", fetch, write, cf, cw, "dim1536_m2048")


def test_layer_step_order_forwards_then_backwards_then_join():
    """The step issues every forward (one fp8_linear_fwd call: quantize, then
    the GEMM that folds the rings) in order, then every backward in reverse
    order, then makes the main stream wait for the dW stream; the launch hook
    sees each call with its kind."""
    log = []

    class FakeLayer:
        def __init__(self, i):
            self.fwd = lambda: log.append(("fwd", i))
            self.bwd = lambda: log.append(("bwd", i))

    class FakeStream:
        def wait_stream(self, other):
            log.append(("join", other))

    main, side = FakeStream(), "side"
    layers = [FakeLayer(i) for i in range(3)]
    step = bench.layer_step(layers, main, side)
    step()
    assert log == [("fwd", 0), ("fwd", 1), ("fwd", 2),
                   ("bwd", 2), ("bwd", 1), ("bwd", 0), ("join", "side")]
    log.clear()
    seen = []

    def hook(kind, li, fn):
        seen.append((kind, li))
        fn()
    step(hook)
    assert seen == [("fwd", 0), ("fwd", 1), ("fwd", 2), ("bwd", 2), ("bwd", 1), ("bwd", 0)]
    assert log[-1] == ("join", "side")


def test_trace_record_per_kind_averages(tmp_path):
    """The trace record averages each GEMM kind's dispatch durations from a
    kernel-trace CSV and turns the average flops per launch of the
    workload's linears over that duration into a fraction of the peak."""
    import csv
    path = tmp_path / "trace.csv"
    names = {"fwd": "void fp8l::gemm4_kernel<0, 0, 0, 0, 0, 0>(fp8l::GemmArgs)",
             "dx": "void fp8l::gemm5_kernel<0, 1, 1, 0>(fp8l::GemmArgs)",
             "dw": "void fp8l::gemm3_kernel<128, 128, 2, 2, 1, 1, 1, 0, 0, 0>(fp8l::GemmArgs)",
             "q": "void fp8l::quantize_flat_kernel<2, 0, 0>(fp8l::QArgs)",
             "f8": "void fp8l::gemm3_kernel<128, 128, 2, 2, 0, 0, 0, 0, 1, 0>(fp8l::GemmArgs)"}
    rows = [("fwd", 20000), ("fwd", 30000), ("dx", 10000), ("dw", 40000), ("q", 5000),
            ("f8", 99000)]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 1000
        for k, d in rows:
            w.writerow([names[k], t, t + d])
            t += d
    rec = bench.trace_record(str(path), "dim1536_m2048")
    assert rec["kinds"]["fwd"] == {"launches": 2, "avg_us": 25.0,
                                   "frac": pytest.approx(rec["flops_per_launch_avg"] / 25e-6 / 1e12
                                                         / bench.MI355X_FP8_DENSE_TFLOPS, abs=1e-4)}
    assert rec["kinds"]["dx"]["avg_us"] == 10.0 and rec["kinds"]["dw"]["avg_us"] == 40.0
    assert set(rec["kinds"]) == {"fwd", "dx", "dw"}  # quantize and fp8-output GEMM not counted
    from scaled_quantize_fp8_amd import workloads as WL
    wl = WL.WORKLOADS["dim1536_m2048"]
    assert rec["flops_per_launch_avg"] == sum(2.0 * wl.M * L.N * L.K for L in wl.linears) / 5


def test_mfma_record_busy_over_dispatch_cycles(tmp_path):
    """mfma_busy_pct divides the MFMA-busy cycles (summed over the SIMDs) by
    the dispatch's engine-busy cycles (summed over the engines, so divided
    by their count) times the SIMDs; MfmaUtil is kept as measured."""
    fwd = GEMM4.format("0, 0, 0, 0")
    dx = GEMM5.format("0, 1, 1, 0")
    path = tmp_path / "m.csv"
    se, simds = bench.MI355X_SHADER_ENGINES, bench.MI355X_SIMDS
    rows = [  # dispatch, kernel, counter, value
        (1, fwd, "MfmaUtil", 20.0), (1, fwd, "SQ_VALU_MFMA_BUSY_CYCLES", 0.4 * 1000 * simds),
        (1, fwd, "SQ_BUSY_CYCLES", 1000.0 * se),
        (2, fwd, "MfmaUtil", 22.0), (2, fwd, "SQ_VALU_MFMA_BUSY_CYCLES", 0.2 * 500 * simds),
        (2, fwd, "SQ_BUSY_CYCLES", 500.0 * se),
        (1, fwd, "SQ_INSTS_VALU_MFMA_MOPS_F8", 1000.0), (2, fwd, "SQ_INSTS_VALU_MFMA_MOPS_F8", 3000.0),
        (3, dx, "MfmaUtil", 30.0),  # no busy counters: only MfmaUtil for this kind
    ]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=_FIELDS)
        w.writeheader()
        for d, name, c, v in rows:
            w.writerow({"Correlation_Id": d, "Dispatch_Id": d, "Agent_Id": "Agent 1",
                        "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})
    rec = bench.mfma_record(str(path), "dim1536_m2048")
    assert rec["mfma_util_pct"] == {"dx": 30.0, "fwd": 21.0}
    assert rec["mfma_busy_pct"] == {"fwd": pytest.approx(30.0)}
    assert rec["dispatches"] == {"dx": 1, "fwd": 2}
    assert "SQ_BUSY_CYCLES" in rec["commands"][1]
    # the MOPs counter books multiply-adds / 512
    assert rec["f8_mfma_flops_per_dispatch"] == {"fwd": pytest.approx(512.0 * 2000.0)}
    wl = WL.WORKLOADS["dim1536_m2048"]
    assert rec["algorithmic_flops_per_dispatch"] == pytest.approx(
        sum(2.0 * wl.M * L.N * L.K for L in wl.linears) / len(wl.linears))
    assert set(rec["paths"]) == {"$REPO", "$OUT"}
