"""Benchmark of the FP8 linear-layer hot path on one MI355X.

One step = one transformer layer of the dim1536 / ffn6912 model at M = 2048
tokens: for each of its five linears (qkv, out, up, gate, down) the forward
(quantize X and W with delayed-scaling rings, Y = X8 W8^T / (sx sw) + bias),
the weight/bias gradient (quantize G with its ring and column partials,
dW = G8^T X8 / (sg sx), db) and the input gradient (dX = G8 W8 / (sg sw)):
15 FP8 GEMMs and 15 quantizes.  Inputs are seeded synthetic bf16 tensors,
resident in HBM before the timed region.

The step runs in a training step's order: every forward as one
fp8_linear_fwd(X, W) call (X and W quantized with their rings in one launch
that runs no ring election, then the GEMM, whose first block folds both
rings before its first operand load); then every backward in reverse order,
each one fp8_linear_bwd(G): G quantized once (with db's column partials, the
ring fold again left to the GEMM), the dX GEMM on the main stream, and the
dW GEMM with db on a second stream after the quantize, so that the weight
gradients fill the CUs the dX chain leaves idle.  The step ends with the
main stream waiting for the second.  In each timed step one linear's
forward is issued instead as fp8_quantize_pair(X, W) and fp8_linear_fwd(X8,
W8), so that its GEMM launch can be bracketed with events for the roofline
entry (rotating over the linears).

The timed steps walk enough copies of the layer (>= 1 GiB of bf16 inputs,
each copy with its own buffers and rings) that no step finds its inputs in
L2 or the MALL: the headline is this cold step.  Beside it the line carries
the warm step (one copy every step), the same step replayed from a HIP graph
(one copy), and the step of every other full-size workload: the dim1024 layer at M = 2048,
the dim1536 layer at M = 512, the generic 4096 <-> 11008 pair at M = 4096
with dynamic scaling, and the dim1536 layer with W and bias pre-quantized.

Prints one JSON line (see the fields below).  --gpus N > 1 is refused: this
benchmark measures one GPU.
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

MI355X_FP8_DENSE_TFLOPS = 5000.0   # published dense FP8 MFMA peak
MI355X_HBM_GBPS = 8000.0           # published HBM3E bandwidth
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="dim1536_m2048")
    p.add_argument("--kernel-reps", type=int, default=200,
                   help="timed launches of each isolated kernel timing (in batches of 20)")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the MFMA-only and HBM-stream probes")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-other-configs", action="store_true",
                   help="skip the other workloads' steps")
    p.add_argument("--no-widened", action="store_true",
                   help="skip the isolated timings of the entry points beyond the layer step "
                        "(for a profile of the step alone)")
    p.add_argument("--cpu-seconds", type=float, default=25.0,
                   help="budget of the oracle sample (it stops after the linear that crosses it)")
    p.add_argument("--sweep-tiles", action="store_true",
                   help="time every GEMM of the step under each tile configuration and exit")
    p.add_argument("--traffic-from", nargs=5, default=None,
                   metavar=("KIND", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                   help="no GPU: turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of "
                        "'--only KIND' and '--only copy' runs into the HBM-traffic record that "
                        "the roofline entry reads, and exit")
    p.add_argument("--trace-from", default=None, metavar="KERNEL_TRACE_CSV",
                   help="no GPU: turn the rocprofv3 --kernel-trace CSV of a profiled run of this "
                        "benchmark into the per-kind GEMM duration record under profiles/, and "
                        "exit")
    p.add_argument("--mfma-from", default=None, metavar="MFMAUTIL_CSV",
                   help="no GPU: turn a rocprofv3 --pmc MfmaUtil CSV of an '--only gemm' run "
                        "into the per-kind MFMA-utilisation record under profiles/, and exit")
    p.add_argument("--only", default=None,
                   help="profiling aid: run only this kernel class (fwd, dx, dw, gemm = all "
                        "three, quant, copy) for --steps iterations and exit")
    return p.parse_args()


class Layer:
    """Device buffers, rings and bound C calls of one linear.  Delayed
    workloads get a ring per quantized tensor, dynamic ones none; the
    pre-quantized workload takes W and the bias as e4m3 codes with their
    scales (made once here) and quantizes only X in the forward.  inputs:
    CPU tensors (X, W, b, G) to copy instead of generating them."""

    def __init__(self, F, WL, wl, li, dev, stream, side, inputs=None):
        import torch

        # every buffer is made, filled and first written on `stream`, the
        # stream the library calls run on, so that no zero fill or copy on
        # another stream can land after a library write to the same scalar
        with torch.cuda.stream(stream):
            self._build(F, WL, wl, li, dev, stream, side, inputs)
        stream.synchronize()

    def _build(self, F, WL, wl, li, dev, stream, side, inputs):
        import torch

        X, W, b, G = WL.layer_inputs(wl, li) if inputs is None else inputs
        self.delayed = wl.delayed
        self.prequant = wl.name.startswith("prequant")
        self.name = wl.linears[li].name
        self.M, self.K = X.shape
        self.N = W.shape[0]
        M, N, K = self.M, self.N, self.K
        e = lambda *s, dt=torch.uint8: torch.empty(*s, dtype=dt, device=dev)
        f = lambda: torch.zeros(1, dtype=torch.float32, device=dev)
        self.X, self.W, self.b, self.G = X.to(dev), W.to(dev), b.to(dev), G.to(dev)
        self.x8, self.w8, self.g8 = e(M, K), e(N, K), e(M, N)
        self.y = e(M, N, dt=torch.bfloat16)
        self.dx = e(M, K, dt=torch.bfloat16)
        self.dw = e(N, K, dt=torch.bfloat16)
        self.db = e(N, dt=torch.bfloat16)
        self.ws = e(max(1, F.fp8_db_workspace_bytes(M, N) // 4), dt=torch.float32)
        self.sx, self.sw, self.sg, self.ax, self.aw, self.ag = (f() for _ in range(6))
        ring = (lambda: F.ScaleRing(wl.hist_len, stream=stream)) if wl.delayed else (lambda: None)
        self.rx, self.rw, self.rg = ring(), ring(), ring()
        self.flops = 2.0 * M * N * K  # per GEMM
        x8q = F.Quantized(self.x8, F.FP8_E4M3, self.sx)
        w8q = F.Quantized(self.w8, F.FP8_E4M3, self.sw)
        g8q = F.Quantized(self.g8, F.FP8_E5M2, self.sg)
        bias = self.b
        if self.prequant:
            # W8 and b8 with their dynamic scales, made once (the pre-quantized
            # operands a caller would hand in)
            self.b8, self.sb, ab = e(N), f(), f()
            F.fp8_quantize(self.W, F.FP8_E4M3, self.w8, None, self.sw, self.aw, stream=stream)
            F.fp8_quantize(self.b, F.FP8_E4M3, self.b8, None, self.sb, ab, stream=stream)
            bias = F.Quantized(self.b8, F.FP8_E4M3, self.sb)
        # the calls of a training step: the forward as quantize pair + GEMM,
        # the backward as one fp8_linear_bwd (G quantized once; dX on stream,
        # dW and db on side after the quantize)
        self.bwd = F.bind_fp8_linear_bwd(self.G, F.FP8_E5M2, x8q, w8q, self.dx, self.dw, self.db,
                                         self.ws, self.rg, self.g8, self.sg, self.ag,
                                         stream=stream, stream_dw=side)
        # the backward on one stream: the dX and dW GEMMs as one grouped launch
        self.bwd_one = F.bind_fp8_linear_bwd(self.G, F.FP8_E5M2, x8q, w8q, self.dx, self.dw,
                                             self.db, self.ws, self.rg, self.g8, self.sg, self.ag,
                                             stream=stream, stream_dw=stream)
        # the same backward as two one-stream calls (the dW call quantizes G),
        # for a step that brackets the dX GEMM alone
        self.bwd_dw = F.bind_fp8_linear_bwd_dw(self.G, F.FP8_E5M2, x8q, self.dw, self.db, self.ws,
                                               self.rg, self.g8, self.sg, self.ag, stream=stream)
        self.bwd_dx = F.bind_fp8_linear_bwd_dx(g8q, F.FP8_E5M2, w8q, self.dx, stream=stream)
        # the forward as one call: quantize X (and W) with their rings, then
        # the GEMM, which folds the rings in its first block (the quantize
        # launch runs no election)
        w_in = w8q if self.prequant else self.W
        self.fwd = F.bind_fp8_linear_fwd(self.X, w_in, bias, F.FP8_E4M3, self.y, self.rx,
                                         None if self.prequant else self.rw, self.x8,
                                         None if self.prequant else self.w8, self.sx,
                                         None if self.prequant else self.sw, self.ax,
                                         None if self.prequant else self.aw, stream=stream)
        # single-kernel calls (pre-quantized operands) for isolated timings
        self.gemm_fwd = F.bind_fp8_linear_fwd(x8q, w8q, bias, F.FP8_E4M3, self.y, stream=stream)
        self.gemm_dw = F.bind_fp8_linear_bwd_dw(g8q, F.FP8_E5M2, x8q, self.dw, stream=stream)
        if self.prequant:  # the forward's quantize: X only
            self.quant_xw = F.bind_fp8_quantize(self.X, F.FP8_E4M3, self.x8, self.rx, self.sx,
                                                self.ax, stream=stream)
        else:
            self.quant_xw = F.bind_fp8_quantize_pair(self.X, self.x8, self.rx, self.sx, self.ax,
                                                     self.W, self.w8, self.rw, self.sw, self.aw,
                                                     F.FP8_E4M3, stream=stream)
        self.quant = {
            "X": F.bind_fp8_quantize(self.X, F.FP8_E4M3, self.x8, self.rx, self.sx, self.ax,
                                     stream=stream),
            "W": F.bind_fp8_quantize(self.W, F.FP8_E4M3, self.w8, self.rw, self.sw, self.aw,
                                     stream=stream),
            "G": F.bind_fp8_quantize(self.G, F.FP8_E5M2, self.g8, self.rg, self.sg, self.ag,
                                     stream=stream),
        }

    def quant_bytes(self, which):
        """Algorithmic bytes of one quantize of X, W or G: bf16 read + fp8
        write, plus the second read of the dynamic path's amax pass."""
        n = {"X": self.M * self.K, "W": self.N * self.K, "G": self.M * self.N}[which]
        return (3.0 if self.delayed else 5.0) * n

    def step_quant_bytes(self):
        """Quantize bytes of one training step of this linear (W is not
        quantized on the pre-quantized path)."""
        return sum(self.quant_bytes(w) for w in (("X", "G") if self.prequant else ("X", "W", "G")))


def event_time_ms(torch, fn, reps, stream):
    """Average GPU duration of fn() over reps calls: a GPU sleep is queued
    first so every call is enqueued before the GPU reaches the start event,
    and the events bracket pure device time."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(2_000_000)
        start.record(stream)
        for _ in range(reps):
            fn()
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def _pct(vals, q):
    import numpy as np
    return float(np.percentile(np.asarray(vals, dtype=np.float64), q))


def batched_stats_us(torch, fns, stream, reps=200, warm=20, batch=20):
    """Per-launch device time in µs: `warm` untimed launches, then `reps`
    launches in batches of `batch` back-to-back launches, each batch inside
    one event pair (all queued behind a GPU sleep, so the device runs them
    back to back); median, p10 and p90 of the per-launch time over the
    batches.  fns: one callable, or a list the launches cycle through."""
    fns = fns if isinstance(fns, (list, tuple)) else [fns]
    for i in range(warm):
        fns[i % len(fns)]()
    nb = max(1, reps // batch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nb)]
    k = 0
    with torch.cuda.stream(stream):
        torch.cuda._sleep(5_000_000)
        for a, b in evs:
            a.record(stream)
            for _ in range(batch):
                fns[k % len(fns)]()
                k += 1
            b.record(stream)
    evs[-1][1].synchronize()
    per = [1e3 * a.elapsed_time(b) / batch for a, b in evs]
    return {"median": round(_pct(per, 50), 3), "p10": round(_pct(per, 10), 3),
            "p90": round(_pct(per, 90), 3), "launches": nb * batch}


def bracket_overhead_us(torch, fn, reps, stream):
    """How much longer a launch measures when an event pair brackets it on
    its own (as the live roofline figures do) than its share of one pair
    around reps back-to-back launches: both taken on the same call, behind
    a GPU sleep, in microseconds."""
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(reps)]
    with torch.cuda.stream(stream):
        torch.cuda._sleep(2_000_000)
        for a, b in pairs:
            a.record(stream)
            fn()
            b.record(stream)
    pairs[-1][1].synchronize()
    single = sum(a.elapsed_time(b) for a, b in pairs) / reps
    return 1e3 * (single - event_time_ms(torch, fn, reps, stream))


def kernel_source_hash() -> str:
    """Hash of the FP8 path's kernel sources (the measurement probes'
    source excluded): records taken on other sources are not used."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scaled_quantize_fp8_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        if fn == "fp8l_probe.hip":
            continue
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


COPY_BYTES = 256 << 20            # the --only copy calibration moves this much each way
# GEMM kinds by the operand template arguments <.., LA, LB, FA, FB> of the
# pipelined kernels: the first four of gemm4_kernel<...> and gemm5_kernel<...>,
# the four after BM, BN, WGM, WGN of gemm3_kernel<...> (followed there by its
# epilogue mode and output format)
KIND_OPERANDS = {"fwd": (0, 0, 0, 0), "dx": (0, 1, 1, 0), "dw": (1, 1, 1, 0)}


def gemm_kind_of(kernel_name: str):
    """'fwd' / 'dx' / 'dw' for a pipelined GEMM kernel name, else None."""
    head = kernel_name.split("(")[0].replace("void ", "").strip()
    if not any(head.startswith(f"fp8l::gemm{v}_kernel<") for v in (3, 4, 5)):
        return None
    targs = [int(a) for a in head[head.index("<") + 1:head.rindex(">")].split(",")]
    if head.startswith("fp8l::gemm3_kernel<"):
        if len(targs) > 8 and targs[8] != 0:  # an FP8-output epilogue
            return None
        args = tuple(targs[4:8])
    else:
        args = tuple(targs[:4])
    for kind, ops in KIND_OPERANDS.items():
        if args == ops:
            return kind
    return None


def _pmc_per_dispatch(path, counter):
    """{dispatch id: (kernel name, counter value in KiB)} from a rocprofv3
    --pmc CSV (values of one dispatch summed over its rows)."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, v + float(r["Counter_Value"]))
    return out


def traffic_key(kind, workload):
    """Name of the traffic record of a GEMM kind (fwd, dx, dw) or of the
    quantize (quant) on a workload."""
    return f"quant_{workload}" if kind == "quant" else f"gemm_{kind}_{workload}"


def quant_launch_bytes(workload, dispatches):
    """Average algorithmic bytes (bf16 in, fp8 out) of the flat-quantize
    dispatches of an '--only quant --steps S' run: S steps of X, W and G of
    every linear, plus the X and W quantizes of the seeding step before
    them (whose G goes through the column-sum kernel)."""
    from scaled_quantize_fp8_amd import workloads as WL
    wl = WL.WORKLOADS[workload]
    xw = [3.0 * n for L in wl.linears for n in (wl.M * L.K, L.N * L.K)]
    g = [3.0 * wl.M * L.N for L in wl.linears]
    steps, rem = divmod(dispatches - len(xw), len(xw) + len(g))
    if rem or steps < 1:
        raise SystemExit(f"{dispatches} flat-quantize dispatches do not fit whole steps")
    return (steps * (sum(xw) + sum(g)) + sum(xw)) / dispatches


def traffic_record(kind, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload):
    """HBM bytes per launch of the KIND GEMM kernel (or of the flat quantize,
    KIND quant): FETCH_SIZE and WRITE_SIZE averaged over its dispatches,
    each scaled by the factor that makes the same counter read COPY_BYTES
    for the 256 MiB copy of the calibration run."""
    def per_kernel(path, counter, match):
        vals = [v for name, v in _pmc_per_dispatch(path, counter).values() if match(name)]
        if not vals:
            raise SystemExit(f"{path}: no dispatch of the kernel with {counter}")
        return sum(vals) / len(vals), len(vals)

    if kind == "quant":
        is_gemm = lambda n: "fp8l::quantize_flat_kernel<" in n
    else:
        is_gemm = lambda n: gemm_kind_of(n) == kind
    # the copy: the largest dispatches of the calibration run (torch's copy_)
    def copy_kib(path, counter):
        vals = sorted(v for _, v in _pmc_per_dispatch(path, counter).values())
        return vals[-1]
    fetch_kib, n_f = per_kernel(fetch_csv, "FETCH_SIZE", is_gemm)
    write_kib, n_w = per_kernel(write_csv, "WRITE_SIZE", is_gemm)
    f_scale = COPY_BYTES / (copy_kib(copy_fetch_csv, "FETCH_SIZE") * 1024)
    w_scale = COPY_BYTES / (copy_kib(copy_write_csv, "WRITE_SIZE") * 1024)
    rd = fetch_kib * 1024 * f_scale
    wr = write_kib * 1024 * w_scale
    runs = [f"rocprofv3 --pmc {c} --output-format csv -d $OUT/traffic -o t_{w}_{c} -- "
            f"python3 $REPO/bench.py --only {w} --steps 3"
            for w in (kind, "copy") for c in ("FETCH_SIZE", "WRITE_SIZE")]
    cmds = ["cd /tmp && export TMPDIR=/tmp"] + runs + [
        f"python3 bench.py --traffic-from {kind} " + " ".join(
            f"$OUT/traffic/t_{w}_{c}_counter_collection.csv"
            for w in (kind, "copy") for c in ("FETCH_SIZE", "WRITE_SIZE"))]
    return {"kernel_kind": kind, "workload": workload, "kernel_source_hash": kernel_source_hash(),
            "commands": cmds, "paths": CMD_PATHS,
            "dispatches": [n_f, n_w], "fetch_kib_raw": fetch_kib, "write_kib_raw": write_kib,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
            "hbm_bytes_per_launch": rd + wr,
            **({"algorithmic_bytes_per_launch": quant_launch_bytes(workload, n_f)}
               if kind == "quant" else {})}


# MI355X: 8 XCDs x 4 shader engines, 256 CUs x 4 SIMDs
MI355X_SHADER_ENGINES = 32
MI355X_SIMDS = 1024

# placeholders in the commands a profile record carries
CMD_PATHS = {"$REPO": "the repository root",
             "$OUT": "the directory rocprofv3 wrote its output to (outside the sources)"}


def mfma_record(csv_path, workload):
    """MFMA utilisation of each GEMM kind, averaged over its dispatches in a
    rocprofv3 --pmc run of '--only gemm' with MfmaUtil, SQ_VALU_MFMA_BUSY_CYCLES
    and SQ_BUSY_CYCLES:

      mfma_util_pct   rocprofv3's MfmaUtil: MFMA-busy cycles over
                      GRBM_GUI_ACTIVE x SIMDs.  GRBM_GUI_ACTIVE spans more
                      than the dispatch under counter collection (a 2.8 us
                      copy reads ~287k cycles), so this under-reads.
      mfma_busy_pct   MFMA-busy cycles (summed over the SIMDs) over the
                      dispatch's own shader-engine busy cycles
                      (SQ_BUSY_CYCLES summed over the engines, divided by
                      their count) x SIMDs: the share of the dispatch's
                      cycles the matrix pipes were busy, over all SIMDs."""
    util = _pmc_per_dispatch(csv_path, "MfmaUtil")
    mbusy = _pmc_per_dispatch(csv_path, "SQ_VALU_MFMA_BUSY_CYCLES")
    sbusy = _pmc_per_dispatch(csv_path, "SQ_BUSY_CYCLES")
    mops = _pmc_per_dispatch(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_F8")
    by, busy, flops = {}, {}, {}
    for d, (name, v) in util.items():
        kind = gemm_kind_of(name)
        if not kind:
            continue
        by.setdefault(kind, []).append(v)
        if d in mbusy and d in sbusy and sbusy[d][1] > 0:
            cycles = sbusy[d][1] / MI355X_SHADER_ENGINES
            busy.setdefault(kind, []).append(100.0 * mbusy[d][1] / (cycles * MI355X_SIMDS))
        if d in mops:  # the counter books fp8 multiply-adds / 512
            flops.setdefault(kind, []).append(512.0 * mops[d][1])
    if not by:
        raise SystemExit(f"{csv_path}: no GEMM dispatch with MfmaUtil")
    counters = "MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F8"
    cmds = ["cd /tmp && export TMPDIR=/tmp",
            f"rocprofv3 --pmc {counters} --output-format csv -d $OUT/traffic "
            "-o t_gemm_MfmaUtil -- python3 $REPO/bench.py --only gemm --steps 3",
            "python3 bench.py --mfma-from $OUT/traffic/t_gemm_MfmaUtil_counter_collection.csv"]
    rec = {"workload": workload, "kernel_source_hash": kernel_source_hash(), "commands": cmds,
           "mfma_util_pct": {k: round(sum(v) / len(v), 2) for k, v in sorted(by.items())},
           "dispatches": {k: len(v) for k, v in sorted(by.items())}}
    if busy:
        rec["mfma_busy_pct"] = {k: round(sum(v) / len(v), 2) for k, v in sorted(busy.items())}
    if flops:
        # every linear's GEMM of a kind is launched equally often, so the
        # algorithmic average is the layer's mean 2MNK
        from scaled_quantize_fp8_amd import workloads as WL
        wl = WL.WORKLOADS[workload]
        alg = sum(2.0 * wl.M * L.N * L.K for L in wl.linears) / len(wl.linears)
        rec["f8_mfma_flops_per_dispatch"] = {k: sum(v) / len(v) for k, v in sorted(flops.items())}
        rec["algorithmic_flops_per_dispatch"] = alg
    rec["paths"] = CMD_PATHS
    return rec


def trace_record(trace_csv, workload):
    """Per-kind GEMM durations from the rocprofv3 --kernel-trace CSV of a
    profiled run of this benchmark (--no-widened --no-other-configs, so
    every GEMM launch in it is one of this workload's linears, and every
    linear's GEMM of a kind is launched equally often): launches, average
    duration, and the frac of the FP8 peak that the average flops per
    launch over the average duration give."""
    import csv
    from scaled_quantize_fp8_amd import workloads as WL
    wl = WL.WORKLOADS[workload]
    by = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            kind = gemm_kind_of(r["Kernel_Name"])
            if kind:
                by.setdefault(kind, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if not by:
        raise SystemExit(f"{trace_csv}: no GEMM dispatch")
    flops = sum(2.0 * wl.M * L.N * L.K for L in wl.linears) / len(wl.linears)
    kinds = {}
    for k, v in sorted(by.items()):
        avg_us = sum(v) / len(v) / 1e3
        kinds[k] = {"launches": len(v), "avg_us": round(avg_us, 3),
                    "frac": round(flops / (avg_us * 1e-6) / 1e12 / MI355X_FP8_DENSE_TFLOPS, 4)}
    cmds = ["cd /tmp && export TMPDIR=/tmp",
            "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_step "
            "-o step -- python3 $REPO/bench.py --steps 20 --warmup 5 --no-widened "
            "--no-other-configs --no-cpu-baseline --no-ceilings",
            f"python3 bench.py --workload {workload} --trace-from "
            "$OUT/prof_step/step_kernel_trace.csv"]
    return {"workload": workload, "kernel_source_hash": kernel_source_hash(), "commands": cmds,
            "paths": CMD_PATHS, "flops_per_launch_avg": flops, "kinds": kinds}


def trace_record_path(workload):
    return os.path.join(PROFILE_DIR, f"gemm_trace_{workload}.txt")


def load_trace_record(kind, workload):
    """The kind's trace figures from the committed record, or None if absent
    or taken on different kernel sources."""
    path = trace_record_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec["kinds"].get(kind)


def load_mfma(workload):
    """Per-kind MFMA utilisation (percent, as rocprofv3's MfmaUtil and as
    busy cycles of the dispatch; see mfma_record) from the committed record,
    or None if absent or taken on different kernel sources."""
    path = os.path.join(PROFILE_DIR, f"mfma_util_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return {"mfma_util_pct": rec.get("mfma_util_pct"), "mfma_busy_pct": rec.get("mfma_busy_pct")}


def load_quant_traffic(workload):
    """Measured vs algorithmic HBM bytes per flat-quantize launch from the
    committed record, or None if absent or taken on different sources."""
    path = traffic_path(traffic_key("quant", workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return {"hbm_bytes_per_launch": round(rec["hbm_bytes_per_launch"]),
            "algorithmic_bytes_per_launch": round(rec["algorithmic_bytes_per_launch"])}


def traffic_path(kernel_key: str) -> str:
    return os.path.join(PROFILE_DIR, f"traffic_{kernel_key}.txt")


def load_traffic(kernel_key: str):
    """HBM bytes per launch from the committed PMC summary of this kernel, or
    None if absent or taken on different kernel sources."""
    path = traffic_path(kernel_key)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_oracle_rate(layers_cpu, budget_s, rows, threads=None, min_s=5.0):
    """The oracle (untuned) on the host: per linear, the dynamic quantizes of
    X, W, G and the three GEMMs plus db, on the first `rows` rows of X and
    G (full W), repeated over the layer's linears until min_s has passed at
    a layer boundary or budget_s at any linear.  threads: BLAS threads for
    the oracle's float64 matmuls (None = all).  Rate in TFLOP/s of the
    GEMMs' 2MNK flops."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import fp8_oracle as O

    flops = 0.0
    done = 0
    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        t0 = time.perf_counter()
        order = [layers_cpu[i % len(layers_cpu)] for i in range(64 * len(layers_cpu))]
        for (X, W, b, G) in order:
            xs = X[:rows].float().numpy()
            gs = G[:rows].float().numpy()
            ws = W.float().numpy()
            x8, sx, _ = O.quantize_step(xs, O.E4M3, None)
            w8, sw, _ = O.quantize_step(ws, O.E4M3, None)
            g8, sg, _ = O.quantize_step(gs, O.E5M2, None)
            beta = O.bias_values(b.view(__import__("torch").int16).numpy().view(np.uint16), "bf16")
            O.linear_fwd(x8, w8, O.E4M3, sx, sw, beta)
            O.linear_bwd_dx(g8, O.E5M2, w8, O.E4M3, sg, sw)
            O.linear_bwd_dw(g8, O.E5M2, x8, O.E4M3, sg, sx)
            O.bias_grad(gs.astype(np.float64))
            K, N = X.shape[1], W.shape[0]
            flops += 3 * 2.0 * rows * N * K
            done += 1
            el = time.perf_counter() - t0
            if el > budget_s or (el >= min_s and done % len(layers_cpu) == 0):
                break
        dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": used,
            "sample": f"{rows} of {layers_cpu[0][0].shape[0]} rows of X and G, full W; "
                      f"{done} linear passes over the layer's {len(layers_cpu)} linears: "
                      f"quantize X/W/G (dynamic) + fwd/dX/dW GEMMs + db, fp64 accumulation; "
                      f"{dt:.1f} s with {used} BLAS thread(s)"}


def cpu_baseline(layers_cpu, budget_s):
    """The oracle on the host's cores at all threads (value) and at one
    thread (on a smaller row sample), with the CPU model."""
    all_t = cpu_oracle_rate(layers_cpu, 0.55 * budget_s, rows=layers_cpu[0][0].shape[0])
    one_t = cpu_oracle_rate(layers_cpu, 0.45 * budget_s, rows=256, threads=1, min_s=3.0)
    return {**all_t, "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_thread": one_t}


def ceilings(torch, stream):
    """The machine's own ceilings, from the measurement kernels of
    libfp8probe.so: the MFMA-only rate (v_mfma_f32_32x32x64_f8f6f4, 8 waves
    per CU, one block per CU) on random e4m3 operands and on zeros, with all
    CUs busy and with the tile counts of the layer's GEMMs; and a plain HBM
    stream (copy, read, write) of 512 MiB at 4 and 8 blocks per CU."""
    from scaled_quantize_fp8_amd import probe as P
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {"cus": cus, "mfma_TFLOPs": {}, "hbm_GBps": {}}
    out = torch.empty(65536 * 8, dtype=torch.float32, device="cuda")
    iters = 2000
    for label, rnd in (("random", True), ("zeros", False)):
        codes = P.mfma_codes(rnd)
        for blocks in sorted({cus, 216, 192, 144, 48}):
            if blocks > cus:
                continue
            st = batched_stats_us(torch, lambda: P.mfma(blocks, iters, codes, out, stream), stream,
                                  reps=20, warm=3, batch=5)
            res["mfma_TFLOPs"][f"{label}_{blocks}cu"] = round(
                P.mfma_flops(blocks, iters) / (st["median"] * 1e-6) / 1e12, 1)
    # fixed cost of a GEMM launch: the layer's output shapes at K = 64 (one
    # K step: prologue, one stage, epilogue, launch and block-end spread)
    # beside K = 1536, through the forward entry point on zero codes
    import scaled_quantize_fp8_amd as F
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    res["gemm_fixed_us"] = {}
    for M, N in ((2048, 6912), (2048, 4608), (2048, 1536)):
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        row = {}
        for K in (64, 1536):
            a = F.Quantized(torch.zeros(M, K, dtype=torch.uint8, device="cuda"), F.FP8_E4M3, one)
            b = F.Quantized(torch.zeros(N, K, dtype=torch.uint8, device="cuda"), F.FP8_E4M3, one)
            fn = F.bind_fp8_linear_fwd(a, b, None, F.FP8_E4M3, y, stream=stream)
            row[f"K{K}"] = batched_stats_us(torch, fn, stream, reps=100, warm=10)["median"]
        res["gemm_fixed_us"][f"{M}x{N}"] = row
    # the 2048 x 6912 forward (the up projection's shape) on random finite
    # e4m3 codes at K = 512 .. 2048: a least-squares line through the
    # medians splits the launch into a fixed part and a cost per 64-byte K
    # step, to set beside the MFMA-only time of one step (16 MFMAs of
    # 32x32x64 per SIMD on 216 CUs at the random-data rate above)
    gen = torch.Generator(device="cpu").manual_seed(11)
    M, N = 2048, 6912
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ks, us = [], []
    for K in (512, 1024, 1536, 2048):
        def rnd(r):
            c = torch.randint(0, 254, (r, K), generator=gen, dtype=torch.int32)
            return torch.where(c >= 0x7F, c + 1, c).to(torch.uint8).to("cuda")  # no NaN code
        a = F.Quantized(rnd(M), F.FP8_E4M3, one)
        b = F.Quantized(rnd(N), F.FP8_E4M3, one)
        fn = F.bind_fp8_linear_fwd(a, b, None, F.FP8_E4M3, y, stream=stream)
        ks.append(K)
        us.append(batched_stats_us(torch, fn, stream, reps=100, warm=10)["median"])
    n = len(ks)
    steps = [k / 64 for k in ks]
    mx, my = sum(steps) / n, sum(us) / n
    slope = (sum((x - mx) * (v - my) for x, v in zip(steps, us)) /
             sum((x - mx) ** 2 for x in steps))
    mfma_step_us = None
    r216 = res["mfma_TFLOPs"].get("random_216cu")
    if r216:
        mfma_step_us = 216 * 4 * 16 * 2 * 32 * 32 * 64 / (r216 * 1e12) * 1e6
    res["gemm_kslope_2048x6912"] = {
        "us_by_K": {f"K{k}": round(v, 3) for k, v in zip(ks, us)},
        "us_per_64B_step": round(slope, 4), "fixed_us": round(my - slope * mx, 3),
        "mfma_only_us_per_step": None if mfma_step_us is None else round(mfma_step_us, 4),
        "loop_efficiency": None if mfma_step_us is None else round(mfma_step_us / slope, 3)}
    # fixed cost of a quantize launch: the standalone quantize (seeded ring,
    # last-block election) of bf16 tensors from one block's worth of
    # elements to the layer's largest, and a launch of the stream probe over
    # 16 bytes (the floor of any launch)
    res["quantize_us"] = {}
    for n in (4096, 1 << 20, 3 << 20, 14 << 20):
        x = torch.randn(n, device="cuda").to(torch.bfloat16)
        q = torch.empty(n, dtype=torch.uint8, device="cuda")
        su, am = (torch.zeros(1, dtype=torch.float32, device="cuda") for _ in range(2))
        ring = F.ScaleRing(16, stream=stream)
        fn = F.bind_fp8_quantize(x, F.FP8_E4M3, q, ring, su, am, stream=stream)
        fn()
        res["quantize_us"][f"n{n}"] = batched_stats_us(torch, fn, stream, reps=100, warm=10)["median"]
    tiny = torch.zeros(16, dtype=torch.uint8, device="cuda")
    sink0 = torch.zeros(4, dtype=torch.int32, device="cuda")
    res["launch_floor_us"] = batched_stats_us(
        torch, lambda: P.stream(tiny, tiny, 16, 0, 1, sink0, stream), stream, reps=100,
        warm=10)["median"]
    nbytes = 512 << 20
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for mode, name, moved in ((0, "copy", 2 * nbytes), (1, "read", nbytes), (2, "write", nbytes)):
        best = 0.0
        for bpc in (4, 8):
            st = batched_stats_us(torch, lambda: P.stream(src, dst, nbytes, mode, bpc, sink, stream),
                                  stream, reps=20, warm=3, batch=5)
            best = max(best, moved / (st["median"] * 1e-6) / 1e9)
        res["hbm_GBps"][name] = round(best, 1)
    del src, dst
    return res


def layer_step(layers, stream, side, grouped=False):
    """One training step over the linears in a training step's order: every
    forward (the quantize launch, then the GEMM), then every backward in
    reverse order, each one fp8_linear_bwd (G quantized once, with db's
    column partials; the dX GEMM on stream; the dW GEMM and db on side after
    the quantize, overlapping the dX chain).  The step ends with stream
    waiting for side, so the next step's forward meets no dW GEMM and no
    buffer is rewritten while a dW GEMM still reads it.

    launch(kind, li, fn) issues call fn of kind "fwd" or "bwd" of linear li
    (the timed region brackets one of them with events); by default it just
    calls fn.  grouped: each backward on stream alone, its dX and dW GEMMs
    in one grouped launch (no second stream, no join)."""
    def plain(kind, li, fn):
        fn()

    def step(launch=plain):
        for li, L in enumerate(layers):
            launch("fwd", li, L.fwd)
        for li in reversed(range(len(layers))):
            launch("bwd", li, layers[li].bwd_one if grouped else layers[li].bwd)
        if not grouped:
            stream.wait_stream(side)
    return step


def isolated_timings(torch, layers, reps, stream):
    """Per-linear isolated kernel times, warm (the same buffers at every
    launch), as batched medians with p10/p90 (batched_stats_us):

      fwd_gemm, dx_gemm, dw_gemm   the three GEMMs as one-kernel calls on
                                   pre-quantized operands (dW without db)
      quant_X, quant_W, quant_G    the standalone fp8_quantize of each tensor
                                   (ring election in its last block)
      quant_fwd_pair               fp8_quantize_pair(X, W): one launch
      fwd_call                     fp8_linear_fwd(X, W): the pair quantize
                                   without election, then the GEMM that folds
                                   the rings
      bwd_dw_call                  fp8_linear_bwd_dw(G): the G quantize with
                                   db's column partials, no election, then
                                   the dW GEMM (with db) that folds the ring

    The quantize inside the fused calls costs what a call takes beyond its
    GEMM: fwd_call - fwd_gemm and bwd_dw_call - dw_gemm (the latter also
    holds the db finalize)."""
    per = {}
    for L in layers:
        p = {"fwd_gemm": batched_stats_us(torch, L.gemm_fwd, stream, reps),
             "dx_gemm": batched_stats_us(torch, L.bwd_dx, stream, reps),
             "dw_gemm": batched_stats_us(torch, L.gemm_dw, stream, reps)}
        for w in ("X", "W", "G"):
            p[f"quant_{w}"] = batched_stats_us(torch, L.quant[w], stream, reps)
        p["quant_fwd_pair"] = batched_stats_us(torch, L.quant_xw, stream, reps)
        p["fwd_call"] = batched_stats_us(torch, L.fwd, stream, reps)
        p["bwd_dw_call"] = batched_stats_us(torch, L.bwd_dw, stream, reps)
        med = lambda k: p[k]["median"]
        fq_bytes = L.quant_bytes("X") + (0.0 if L.prequant else L.quant_bytes("W"))
        derived = {
            "quant_in_fwd_call_us": round(med("fwd_call") - med("fwd_gemm"), 3),
            "quant_in_bwd_dw_call_us": round(med("bwd_dw_call") - med("dw_gemm"), 3),
        }
        derived["quant_in_fwd_call_GBps"] = round(
            fq_bytes / max(derived["quant_in_fwd_call_us"], 1e-3) / 1e3, 1)
        derived["quant_in_bwd_dw_call_GBps"] = round(
            L.quant_bytes("G") / max(derived["quant_in_bwd_dw_call_us"], 1e-3) / 1e3, 1)
        for w in ("X", "W", "G"):
            derived[f"quant_{w}_GBps"] = round(L.quant_bytes(w) / (med(f"quant_{w}") * 1e3), 1)
        for g_ in ("fwd", "dx", "dw"):
            derived[f"{g_}_TFLOPs"] = round(L.flops / (med(f"{g_}_gemm") * 1e-6) / 1e12, 1)
        p["derived"] = derived
        per[L.name] = p
    tot = {g_: sum(per[L.name][f"{g_}_gemm"]["median"] for L in layers) for g_ in ("fwd", "dx", "dw")}
    # the quantizes as the step runs them, inside the fused calls
    q_us = sum(per[L.name]["derived"]["quant_in_fwd_call_us"] +
               per[L.name]["derived"]["quant_in_bwd_dw_call_us"] for L in layers)
    q_bytes = sum(L.step_quant_bytes() for L in layers)
    return per, tot, q_us, q_bytes / (q_us * 1e-6) / 1e9


def cold_quant_sweep(torch, sets, stream, reps=100):
    """The standalone quantizes of one step over the cold rotation: a batch
    is one copy's paired X/W launch and G launch for every linear, and
    consecutive batches take consecutive copies, so every input was last
    read ~1 GB of other inputs ago (past the 256 MB MALL).  Beside it the
    same batch on one copy, warm.  Aggregate GB/s of the algorithmic bytes
    (median, p10, p90 over batches)."""
    R = len(sets)
    sweeps = [[fn for L in ls for fn in (L.quant_xw, L.quant["G"])] for ls in sets]
    nbytes = sum(L.step_quant_bytes() for L in sets[0])
    out = {}
    for label, order in (("cold", list(range(R))), ("warm", [0])):
        for i in range(2 * R):  # warm-up batches
            for fn in sweeps[order[i % len(order)]]:
                fn()
        nb = max(len(order), reps // len(sweeps[0]))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(nb)]
        with torch.cuda.stream(stream):
            torch.cuda._sleep(5_000_000)
            for bi, (a, b) in enumerate(evs):
                a.record(stream)
                for fn in sweeps[order[bi % len(order)]]:
                    fn()
                b.record(stream)
        evs[-1][1].synchronize()
        us = [1e3 * a.elapsed_time(b) for a, b in evs]
        gbps = [nbytes / (u * 1e-6) / 1e9 for u in us]
        out[label] = {"us_per_step": round(_pct(us, 50), 2), "GBps": round(_pct(gbps, 50), 1),
                      "GBps_p10": round(_pct(gbps, 10), 1), "GBps_p90": round(_pct(gbps, 90), 1),
                      "batches": nb}
    out["bytes_per_step"] = nbytes
    out["launches_per_step"] = len(sweeps[0])
    return out


def timed_steps_ms(torch, step, steps, stream):
    """ms per step over `steps` eager steps (GPU events, or the host wall
    clock if that is longer)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    with torch.cuda.stream(stream):
        a.record(stream)
        for _ in range(steps):
            step()
        b.record(stream)
    torch.cuda.synchronize()
    return max(a.elapsed_time(b), (time.perf_counter() - w0) * 1e3) / steps


def workload_label(wl):
    names = "/".join(L.name for L in wl.linears)
    dims = ", ".join(f"{L.name} {L.K}->{L.N}" for L in wl.linears)
    mode = f"delayed scaling H={wl.hist_len}" if wl.delayed else "dynamic scaling"
    pre = "; W and bias pre-quantized e4m3" if wl.name.startswith("prequant") else ""
    return f"{wl.name}: {dims}; M={wl.M} tokens; {names} fwd+dW(+db)+dX; {mode}{pre}"


def other_configs(torch, F, WL, dev, stream, side, skip, steps, reps):
    """The step of every other full-size workload on its own: ms per step,
    TFLOP/s and % of the FP8 peak over its GEMMs, quantize GB/s as the step
    issues it, and the isolated GEMM totals per kind."""
    res = {}
    for name in ("dim1024_m2048", "dim1536_m512", "generic_m4096", "prequant_dim1536_m2048"):
        if name == skip:
            continue
        wl = WL.WORKLOADS[name]
        layers = [Layer(F, WL, wl, li, dev, stream, side) for li in range(len(wl.linears))]
        step = layer_step(layers, stream, side)
        for _ in range(2):  # the first step seeds the rings
            step()
        per, tot, q_us, q_gbps = isolated_timings(torch, layers, reps, stream)
        ms = timed_steps_ms(torch, step, steps, stream)
        flops = sum(3 * L.flops for L in layers)
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {
            "workload": workload_label(wl),
            "gemms_per_step": 3 * len(layers),
            "ms_per_step": round(ms, 4),
            "TFLOPs": round(tf, 2),
            "pct_fp8_peak": round(100 * tf / MI355X_FP8_DENSE_TFLOPS, 2),
            "quantize_GBps": round(q_gbps, 1),
            "quantize_pct_hbm": round(100 * q_gbps / MI355X_HBM_GBPS, 2),
            "quant_us_per_step": round(q_us, 1),
            "gemm_us_per_step": {k: round(v, 1) for k, v in tot.items()},
            "gemm_TFLOPs": {k: round(sum(L.flops for L in layers) / (v * 1e-6) / 1e12, 1)
                            for k, v in tot.items()},
        }
        del layers, step
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


def widened_rows(torch, F, WL, wl, layers, stream, reps):
    """Isolated timings of the entry points beyond the layer step (not part of
    the step or its value): the transposed and dual quantize, the weight
    gradient run k-contiguous from transposed operands next to the crosswise
    one, a batched fp8_gemm, the FP8-output forward next to the bf16 one, and
    the flat quantize of a 2^28-element tensor (its streaming rate once the
    fixed costs of a launch no longer count)."""
    dev = "cuda:0"
    up = next(L for L in layers if L.name == "up")
    M, N, K = up.M, up.N, up.K
    res = {}
    g8t = torch.empty(N, M, dtype=torch.uint8, device=dev)
    x8t = torch.empty(K, M, dtype=torch.uint8, device=dev)
    g8 = torch.empty(M, N, dtype=torch.uint8, device=dev)
    s1, a1, s2, a2 = (torch.zeros(1, dtype=torch.float32, device=dev) for _ in range(4))
    # delayed scaling through seeded rings, as in the step (the first calls
    # seed them): one pass over the input, 2 B read and 1 B per output
    rg, rx = (F.ScaleRing(wl.hist_len, stream=stream) for _ in range(2))
    dual = F.bind_fp8_quantize_2d(up.G, F.FP8_E5M2, F.FP8_QUANT_DUAL, g8, g8t, rg, s1, a1,
                                  stream=stream)
    tq = F.bind_fp8_quantize_2d(up.G, F.FP8_E5M2, F.FP8_QUANT_TRANSPOSED, None, g8t, rg, s1, a1,
                                stream=stream)
    tx = F.bind_fp8_quantize_2d(up.X, F.FP8_E4M3, F.FP8_QUANT_TRANSPOSED, None, x8t, rx, s2, a2,
                                stream=stream)
    for fn in (dual, tq, tx):
        fn()
    n = M * N
    us = 1e3 * event_time_ms(torch, dual, reps, stream)
    res["quantize_2d_dual_G_up_us"] = round(us, 2)
    res["quantize_2d_dual_G_up_GBps"] = round(4.0 * n / (us * 1e-6) / 1e9, 1)  # 2 B in, 1 + 1 out
    us = 1e3 * event_time_ms(torch, tq, reps, stream)
    res["quantize_2d_transposed_G_up_GBps"] = round(3.0 * n / (us * 1e-6) / 1e9, 1)
    dw = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
    kc = F.bind_fp8_gemm(F.Quantized(g8t, F.FP8_E5M2, s1), F.Quantized(x8t, F.FP8_E4M3, s2), dw,
                         stream=stream)
    kc()
    flops = 2.0 * M * N * K
    us_kc = 1e3 * event_time_ms(torch, kc, reps, stream)
    us_x = 1e3 * event_time_ms(torch, up.gemm_dw, reps, stream)
    res["dw_up_kcontig_us"] = round(us_kc, 2)
    res["dw_up_crosswise_us"] = round(us_x, 2)
    res["dw_up_kcontig_TFLOPs"] = round(flops / (us_kc * 1e-6) / 1e12, 1)
    # batched NT GEMM: 8 x (1024 x 2048) x 2048, distinct slices
    B, bm, bn, bk = 8, 1024, 2048, 2048
    a = torch.randint(0, 0x7e, (B, bm, bk), dtype=torch.uint8, device=dev)
    b = torch.randint(0, 0x7e, (B, bn, bk), dtype=torch.uint8, device=dev)
    c = torch.empty(B, bm, bn, dtype=torch.bfloat16, device=dev)
    one = torch.ones(1, dtype=torch.float32, device=dev)
    bmm = F.bind_fp8_gemm(F.Quantized(a, F.FP8_E4M3, one), F.Quantized(b, F.FP8_E4M3, one), c,
                          stream=stream)
    bmm()
    us = 1e3 * event_time_ms(torch, bmm, reps, stream)
    res["gemm_batched_8x1024x2048x2048_us"] = round(us, 2)
    res["gemm_batched_8x1024x2048x2048_TFLOPs"] = round(2.0 * B * bm * bn * bk / (us * 1e-6) / 1e12, 1)
    # FP8-in / FP8-out forward of up (2048 x 6912 x 1536), steady ring, next
    # to the bf16-output forward of the same operands
    c8 = torch.empty(M, N, dtype=torch.uint8, device=dev)
    ring = F.ScaleRing(wl.hist_len, stream=stream)
    su, am = (torch.zeros(1, dtype=torch.float32, device=dev) for _ in range(2))
    q8 = F.bind_fp8_gemm_fp8out(F.Quantized(up.x8, F.FP8_E4M3, up.sx),
                                F.Quantized(up.w8, F.FP8_E4M3, up.sw), c8, F.FP8_E4M3, ring, su,
                                am, bias=up.b, stream=stream)
    q8()  # seeds the ring (amax pass + converting pass)
    us_q = 1e3 * event_time_ms(torch, q8, reps, stream)
    us_b = 1e3 * event_time_ms(torch, up.gemm_fwd, reps, stream)
    res["gemm_fp8out_up_fwd_us"] = round(us_q, 2)
    res["gemm_fp8out_up_fwd_TFLOPs"] = round(flops / (us_q * 1e-6) / 1e12, 1)
    res["gemm_bf16out_up_fwd_us"] = round(us_b, 2)
    # the flat quantize where its fixed costs vanish: 2^28 seeded-normal bf16
    # elements (512 MiB in, 256 MiB of codes out) through a seeded ring
    n = 1 << 28
    gen = torch.Generator(device=dev)
    gen.manual_seed(28)
    big = torch.randn(n, device=dev, generator=gen).to(torch.bfloat16)
    qbig = torch.empty(n, dtype=torch.uint8, device=dev)
    rbig = F.ScaleRing(wl.hist_len, stream=stream)
    s3, a3 = (torch.zeros(1, dtype=torch.float32, device=dev) for _ in range(2))
    qf = F.bind_fp8_quantize(big, F.FP8_E4M3, qbig, rbig, s3, a3, stream=stream)
    qf()  # seeds the ring
    us = 1e3 * event_time_ms(torch, qf, reps, stream)
    res["quantize_flat_2p28_bf16_us"] = round(us, 2)
    res["quantize_flat_2p28_bf16_GBps"] = round(3.0 * n / (us * 1e-6) / 1e9, 1)
    # beside it, torch's device copy of the same tensor (read + write 2 B per
    # element): the streaming rate a plain copy reaches at this size
    cbig = torch.empty_like(big)
    us = 1e3 * event_time_ms(torch, lambda: cbig.copy_(big), reps, stream)
    res["copy_2p28_bf16_GBps"] = round(4.0 * n / (us * 1e-6) / 1e9, 1)
    del big, qbig, cbig
    res["e2e_train_step"] = e2e_train_step(torch, dev)
    return res


def e2e_train_step(torch, dev, steps=10, warmup=3):
    """ms per training step of the 12-layer dim-1024 transformer (B4 x T512,
    synthetic tokens, fused AdamW) with FP8 linears and with bf16 ones, each
    step replayed as one HIP graph (the eager step is bound by Python
    dispatch on this model, so its time says little about the GPU), plus the
    eager times beside them."""
    from scaled_quantize_fp8_amd import e2e as E
    out = {"model": "12L dim1024 ffn4096 heads16 vocab32000, B4xT512, fused AdamW",
           "steps": steps}
    for name, lin in (("bf16", E.bf16_linear), ("fp8", E.fp8_linear)):
        losses, ms = E.train(lin, steps, dev, graph=True, warmup=warmup)
        _, ms_eager = E.train(lin, steps, dev, graph=False, warmup=warmup)
        out[f"{name}_graph_ms_per_step"] = round(ms, 3)
        out[f"{name}_eager_ms_per_step"] = round(ms_eager, 3)
        out[f"{name}_final_loss"] = round(losses[-1], 4)
    out["fp8_speedup_graph"] = round(out["bf16_graph_ms_per_step"] / out["fp8_graph_ms_per_step"], 3)
    return out


def main():
    args = parse()
    if args.traffic_from:
        kind, *csvs = args.traffic_from
        rec = traffic_record(kind, *csvs, workload=args.workload)
        os.makedirs(PROFILE_DIR, exist_ok=True)
        with open(traffic_path(traffic_key(kind, args.workload)), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.trace_from:
        rec = trace_record(args.trace_from, args.workload)
        os.makedirs(PROFILE_DIR, exist_ok=True)
        with open(trace_record_path(args.workload), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.mfma_from:
        rec = mfma_record(args.mfma_from, args.workload)
        os.makedirs(PROFILE_DIR, exist_ok=True)
        with open(os.path.join(PROFILE_DIR, f"mfma_util_{args.workload}.txt"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.steps < 2:
        print("bench.py needs --steps >= 2 (the live GEMM timing pairs two bracketed steps)",
              file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note, not a built path)", file=sys.stderr)
        sys.exit(2)
    import torch

    import scaled_quantize_fp8_amd as F
    from scaled_quantize_fp8_amd import workloads as WL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    F.lib()  # fails loudly if the HIP library is missing
    wl = WL.WORKLOADS[args.workload]
    stream = torch.cuda.Stream()
    side = torch.cuda.Stream()  # the backward's dW GEMMs (default priority, like stream)
    layers = [Layer(F, WL, wl, li, dev, stream, side) for li in range(len(wl.linears))]
    step = layer_step(layers, stream, side)

    if args.sweep_tiles:
        step()  # seed the rings and fill the quantized operands
        torch.cuda.synchronize()
        res = {}
        for tile in ("256x256w8", "128x128w8", "256x256", "256x128", "128x128", "v1"):
            os.environ["FP8L_TILE"] = tile
            for L in layers:
                for gname, fn in (("fwd", L.gemm_fwd), ("dx", L.bwd_dx), ("dw", L.gemm_dw)):
                    fn()
                    us = 1e3 * event_time_ms(torch, fn, args.kernel_reps, stream)
                    res.setdefault(f"{L.name}.{gname}", {})[tile] = round(us, 2)
        os.environ.pop("FP8L_TILE", None)
        for L in layers:
            for gname, fn in (("fwd", L.gemm_fwd), ("dx", L.bwd_dx), ("dw", L.gemm_dw)):
                us = 1e3 * event_time_ms(torch, fn, args.kernel_reps, stream)
                res[f"{L.name}.{gname}"]["auto"] = round(us, 2)
        print(json.dumps({"sweep_us": res}))
        return

    if args.only:
        # profiling aid: one kernel class only, args.steps times
        step()  # seed the rings
        torch.cuda.synchronize()
        src = dst = None
        if args.only == "copy":
            src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(args.steps):
                if args.only == "copy":
                    dst.copy_(src)
                    continue
                for L in layers:
                    calls = {"fwd": [L.gemm_fwd], "dx": [L.bwd_dx], "dw": [L.gemm_dw],
                             "gemm": [L.gemm_fwd, L.bwd_dx, L.gemm_dw],
                             "quant": [L.quant[w] for w in ("X", "W", "G")]}[args.only]
                    for fn in calls:
                        fn()
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "steps": args.steps}))
        return

    for _ in range(max(1, args.warmup)):  # the first step seeds the rings
        step()
    torch.cuda.synchronize()

    # ---- the rotation the timed region walks: R copies of the layer (set 0 is
    # `layers`, the others made from the same host inputs, each with its own
    # buffers and rings), >= 1 GiB of bf16 inputs in all, past the 256 MB MALL
    # and the 4 MB L2s, so that a timed step finds none of its inputs in a
    # cache (the headline is this cold step; the warm one is reported beside)
    cpu_in = [WL.layer_inputs(wl, li) for li in range(len(wl.linears))]
    per_set = sum(t.numel() * t.element_size() for inp in cpu_in for t in inp)
    R = max(2, -(-(1 << 30) // per_set))
    sets = [layers] + [[Layer(F, WL, wl, li, dev, stream, side, inputs=cpu_in[li])
                        for li in range(len(cpu_in))] for _ in range(R - 1)]
    steps_of = [step] + [layer_step(ls, stream, side) for ls in sets[1:]]
    for st_ in steps_of[1:]:
        for _ in range(max(1, args.warmup)):
            st_()
    torch.cuda.synchronize()

    # ---- isolated per-kernel timings (batched medians with p10/p90, warm),
    # before the timed region: they decide which GEMM kind the live events
    # follow; then the step's standalone quantizes over the cold rotation
    per, tot, q_us, quant_gbps = isolated_timings(torch, layers, args.kernel_reps, stream)
    qsweep = cold_quant_sweep(torch, sets, stream)

    # ---- timed region: exactly args.steps eager steps, step s on copy s mod R
    # of the layer.  Every other step (s even) carries one event pair on
    # stream, around the forward of linear (i / 2) mod n for the i-th such
    # step, issued as its two calls: the paired X/W quantize
    # (fp8_quantize_pair) and the GEMM (fp8_linear_fwd on X8, W8).  For
    # even i the pair brackets quantize and GEMM, for odd i the quantize
    # alone (the GEMM follows outside the bracket), so per linear
    #   GEMM time = [quantize + GEMM] - [quantize],
    # the GEMM's launch-to-launch time in a busy stream, with the events'
    # own cost (a marker after a kernel adds a dispatch round trip to what
    # it brackets) and the quantize cancelling out.  A bracket around the
    # GEMM alone is reported beside it (raw, and less an overhead measured
    # on isolated launches).  The event pairs are created up front, outside
    # the timed region.  (Where the dX GEMM dominates the isolated timings,
    # the same scheme brackets fp8_linear_bwd_dw + the dX GEMM against
    # fp8_linear_bwd_dw alone.)
    # Every step from the second carries a bracket: the timed region starts
    # on an idle stream, and a bracket in its first step would time the GPU
    # catching up with the host's first submissions as well as the kernels.
    # (Measured, a bracket in every step against one in every other step
    # moves the step time by less than its run-to-run spread.)
    dom = "fwd" if tot["fwd"] >= tot["dx"] else "dx"
    brack = list(range(1, args.steps))
    if len(brack) < 2 * len(layers):
        brack = list(range(args.steps))
    ev = {si: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for si in brack}
    ev_what = {}  # step -> (linear, with_gemm)

    def bracketing(step_i):
        ls = sets[step_i % R]
        if step_i in ev:
            i = brack.index(step_i)
            target, with_gemm = (i // 2) % len(ls), i % 2 == 0
        else:
            target, with_gemm = -1, False

        def launch(kind, li, fn):
            if li != target or kind != ("fwd" if dom == "fwd" else "bwd"):
                fn()
                return
            a, b_ = ev[step_i]
            ev_what[step_i] = (li, with_gemm)
            first, gemm = ((ls[li].quant_xw, ls[li].gemm_fwd) if dom == "fwd"
                           else (ls[li].bwd_dw, ls[li].bwd_dx))
            a.record(stream)
            first()
            if with_gemm:
                gemm()
                b_.record(stream)
            else:
                b_.record(stream)
                gemm()
        return launch

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    with torch.cuda.stream(stream):
        t_start.record(stream)
        for si in range(args.steps):
            steps_of[si % R](bracketing(si))
        t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = t_start.elapsed_time(t_end)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    step_flops = sum(3 * L.flops for L in layers)
    tflops = step_flops / (ms_per_step * 1e-3) / 1e12

    # per linear: mean bracketed [first call + GEMM] and [first call] times;
    # the GEMM's live time is their difference
    sums = {}
    for si in brack:
        li, with_gemm = ev_what[si]
        ms = ev[si][0].elapsed_time(ev[si][1])
        sums.setdefault(li, {True: [], False: []})[with_gemm].append(ms)
    covered = sorted(li for li, d in sums.items() if d[True] and d[False])
    mean = lambda v: sum(v) / len(v)
    gemm_us = {li: 1e3 * (mean(sums[li][True]) - mean(sums[li][False])) for li in covered}
    live = {"avg_us": mean(list(gemm_us.values())),
            "flops": mean([layers[li].flops for li in covered]),
            "per_linear_us": {layers[li].name: round(v, 2) for li, v in gemm_us.items()},
            "bracketed_with_gemm_us": {layers[li].name: round(1e3 * mean(sums[li][True]), 2)
                                       for li in covered},
            "launches": sum(len(sums[li][True]) for li in covered),
            "total_us": sum(gemm_us.values()) if len(covered) == len(layers) else None}

    # ---- the same step captured as one HIP graph and replayed (one copy),
    # with the two-stream backward and with the grouped one-stream backward
    def graph_ms(fn):
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                fn()
            torch.cuda.synchronize()
            gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                g.replay()
                gs.record(stream)
                for _ in range(args.steps):
                    g.replay()
                ge.record(stream)
            torch.cuda.synchronize()
            return gs.elapsed_time(ge) / args.steps
        except Exception as exc:  # graph capture is an extra measurement only
            print(f"graph capture skipped: {exc}", file=sys.stderr)
            return None
    step_grouped = layer_step(layers, stream, side, grouped=True)
    graph_ms_per_step = graph_ms(step)
    graph_grouped_ms = graph_ms(step_grouped)

    # ---- the warm step beside it: copy 0 of the layer every step, so its
    # inputs stay in the MALL from one step to the next; and the same with
    # the grouped one-stream backward
    warm_ms = timed_steps_ms(torch, step, args.steps, stream)
    warm_grouped_ms = timed_steps_ms(torch, step_grouped, args.steps, stream)
    rotation = {"copies": R, "input_MB": round(R * per_set / 1e6, 1)}
    del steps_of, sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # the roofline entry: the dominant GEMM kind of the forward and dX (the
    # two issued as one-kernel calls), timed live; all three isolated totals
    # are reported beside it.  An event pair around a single launch adds a
    # fixed overhead (measured here on the same launches); `achieved` takes
    # it out, `achieved_raw` keeps it, and the kernel trace of a profiled
    # run of this benchmark gives the third figure (`trace`).
    dominant_isolated = max(tot, key=tot.get)
    kernel_names = {
        "fwd": "gemm4/gemm5/gemm3_kernel <.., kKContig, kKContig, E4M3, E4M3> "
               "(Y = X8 W8^T, both operands k-contiguous; tile chosen per shape)",
        "dx": "gemm4/gemm5/gemm3_kernel <.., kKContig, kCross, E5M2, E4M3> "
              "(dX = G8 W8, W8 read crosswise; tile chosen per shape)",
    }
    overhead_us = sum(bracket_overhead_us(torch, getattr(L, {"fwd": "gemm_fwd", "dx": "bwd_dx"}[dom]),
                                          20, stream) for L in layers) / len(layers)
    achieved = live["flops"] / (live["avg_us"] * 1e-6) / 1e12
    # beside it: a bracket around the GEMM alone (its first call outside the
    # bracket), taken after the timed region on copy 0, raw and less the
    # isolated bracket overhead
    alone = []
    for L in layers:
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            (L.quant_xw if dom == "fwd" else L.bwd_dw)()
            a.record(stream)
            (L.gemm_fwd if dom == "fwd" else L.bwd_dx)()
            b_.record(stream)
        b_.synchronize()
        alone.append(1e3 * a.elapsed_time(b_))
    alone_us = sum(alone) / len(alone)
    traffic = load_traffic(traffic_key(dom, args.workload))
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MI355X_FP8_DENSE_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MI355X_FP8_DENSE_TFLOPS, 4),
                "traffic": traffic,
                "kernel": kernel_names[dom],
                "launch_avg_us": round(live["avg_us"], 2),
                "live_method": "per linear, bracketed [first call + GEMM] minus bracketed [first "
                               "call], in the timed steps (events on the kernel's stream)",
                "live_per_linear_us": live["per_linear_us"],
                "live_bracketed_with_gemm_us": live["bracketed_with_gemm_us"],
                "gemm_alone_bracket_us_raw": round(alone_us, 2),
                "gemm_alone_bracket_us_less_overhead": round(alone_us - overhead_us, 2),
                "isolated_bracket_overhead_us": round(overhead_us, 2),
                "trace": load_trace_record(dom, args.workload),
                "flops_per_launch": live["flops"],
                "live_launches": live["launches"],
                "live_us_per_step": (None if live["total_us"] is None
                                     else round(live["total_us"], 1)),
                "isolated_gemm_us_per_step": {k: round(v, 1) for k, v in tot.items()},
                "mfma_util_pct_by_kind": load_mfma(args.workload),
                "dominant_gemm_by_isolated_totals": dominant_isolated}

    out = {
        "metric": "FP8 linear fwd+dX+dW TFLOP/s and % FP8 MFMA peak; quantize GB/s vs HBM peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": workload_label(wl), "global_batch": wl.M,
                   "gemms_per_step": 3 * len(layers)},
        "step_schedule": "every forward in order as fp8_linear_fwd(X, W) (quantize without "
                         "election; the GEMM folds the rings), in every step after the first one of "
                         "them split into fp8_quantize_pair + fp8_linear_fwd(X8, W8) inside an "
                         "event pair; then every backward in reverse order as fp8_linear_bwd (dX on "
                         "the main stream, dW and db on a second stream after the G quantize); "
                         "one join of the two streams per step",
        "pct_fp8_peak": round(100 * tflops / MI355X_FP8_DENSE_TFLOPS, 2),
        "quantize_GBps": qsweep["cold"]["GBps"],
        "quantize_pct_hbm": round(100 * qsweep["cold"]["GBps"] / MI355X_HBM_GBPS, 2),
        "quantize": {
            "standalone_cold": qsweep["cold"], "standalone_warm": qsweep["warm"],
            "standalone_note": "fp8_quantize_pair(X, W) and fp8_quantize(G) of every linear, "
                               "ring election in each launch's last block",
            "in_fused_calls_warm_GBps": round(quant_gbps, 1),
            "in_fused_calls_warm_us_per_step": round(q_us, 1),
            "in_fused_calls_note": "the step's quantizes as it runs them (no election; the GEMM "
                                   "folds the ring): fused call minus its GEMM, warm medians",
            "bytes_per_step": qsweep["bytes_per_step"]},
        "quantize_traffic": load_quant_traffic(args.workload),
        "wall_s_timed": round(wall, 4),
        "cold_rotation": rotation,
        "warm": {"ms_per_step": round(warm_ms, 4),
                 "TFLOPs": round(step_flops / (warm_ms * 1e-3) / 1e12, 2)},
        "graph_ms_per_step": None if graph_ms_per_step is None else round(graph_ms_per_step, 4),
        "graph_TFLOPs": None if graph_ms_per_step is None else
        round(step_flops / (graph_ms_per_step * 1e-3) / 1e12, 2),
        "grouped_backward": {
            "note": "each backward as fp8_linear_bwd on one stream: G quantize, then dX and dW "
                    "GEMMs in one grouped launch",
            "warm_ms_per_step": round(warm_grouped_ms, 4),
            "graph_ms_per_step": None if graph_grouped_ms is None else round(graph_grouped_ms, 4)},
        "gemm_us_per_step": {g: round(v, 1) for g, v in tot.items()},
        "per_linear": per,
        "timing_method": "isolated kernels: 20 warm-up launches, then 200 launches in batches of "
                         "20 back-to-back launches, one event pair per batch; median, p10, p90 "
                         "of the per-launch time over the batches (warm: the same buffers)",
        "roofline": roofline,
    }
    if not args.no_ceilings:
        out["ceilings"] = c = ceilings(torch, stream)
        # the same figures against this chip's own ceilings, measured in this
        # run: the MFMA-only rate on random e4m3 codes with every CU busy,
        # and a plain HBM copy
        mfma = c["mfma_TFLOPs"].get(f"random_{c['cus']}cu")
        if mfma:
            roofline["frac_of_measured_mfma_ceiling"] = round(achieved / mfma, 4)
        if c["hbm_GBps"].get("copy"):
            out["quantize_pct_measured_copy"] = round(
                100 * qsweep["cold"]["GBps"] / c["hbm_GBps"]["copy"], 2)
    if not args.no_widened:
        out["widened"] = widened_rows(torch, F, WL, wl, layers, stream, args.kernel_reps)
    if not args.no_other_configs:
        out["other_configs"] = other_configs(torch, F, WL, dev, stream, side, wl.name, args.steps,
                                             args.kernel_reps)
    if not args.no_cpu_baseline:
        layers_cpu = [WL.layer_inputs(wl, li) for li in range(len(wl.linears))]
        out["cpu_baseline"] = cpu_baseline(layers_cpu, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
