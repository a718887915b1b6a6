#!/usr/bin/env python3
"""Throughput of the FP8 W8A8 hot path on one MI355X.

One step = one pass of every step of the hot path:
  1. re-quantize all 144 bf16 weights of a 36-layer Qwen3-8B-shaped policy
     (qkv 4096->6144, o 4096->4096, gate_up 4096->24576, down 12288->4096) into
     E4M3 128x128 blocks with fp32 scales (one batched library call), and the
     two stacked expert weights of a Qwen3-30B-A3B-shaped MoE layer (a second);
  2. for every layer and linear of the dense policy, quantize that layer's bf16
     activations in 1x128 groups and run the block-scaled W8A8 GEMM, bf16 out,
     at M = 8192 (prefill) and at M = 256 (decode);
  3. the per-token path: fused RMSNorm + per-token quantization of h [4096,
     5120], per-row quantization of a [12288, 5120] weight, row-scaled GEMM;
  4. the MoE path: 1x128 quantization of the 32768 routed rows and the grouped
     block-scaled GEMMs gate_up (N=1536, K=2048) and down (N=2048, K=768) over
     128 experts with top-8 routing;
  5. the E8M0 variant: the 144 policy weights re-quantized again with E8M0
     scales, and one layer's four linears at M = 8192 through 1x128 E8M0
     activation quantization and the MX-scaled GEMM.
Every (layer, linear) has its own weight and activation tensors, so weights
and activations stream from HBM as they would in a real forward pass.  Inputs
are seeded synthetic tensors generated on the device before timing.

Prints one JSON line.  ``value`` = all GEMM flops of a step / wall time of a
step (the quantization work in the step is not counted as flops but its time
is).  ``roofline`` is for the dominant kernel, the block-scaled GEMM at
M = 8192, timed with HIP events on the launch stream inside the timed steps;
its ``traffic`` comes from the HBM counter summary committed under profiles/
and is reported only while the GEMM sources still hash to the value recorded
there.  ``cpu_baseline`` times the CPU oracle on a bounded sample of the work.

``--calibrate-copy`` instead runs a plain device copy of 1 GiB a few times,
the reference kernel whose counter reading scales FETCH_SIZE / WRITE_SIZE.
``--one-gemm M N K`` instead runs one block-scaled GEMM shape (seeded dense
inputs, quantized by the library) ``--reps`` times over ``--copies`` distinct
operand sets, for counter runs.  ``--vendor-compare`` times the four M = 8192
shapes on this library's row- and block-scaled GEMMs and on torch._scaled_mm
(row-wise and per-tensor FP8 scales) on the same box.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E
METRIC = "block-scaled FP8 GEMM TFLOPS (% FP8 MFMA peak); quantize/requant GB/s (% HBM)"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_gemm_pp_m8192.md")
GEMM_SOURCES = ["fp8_w8a8_quantized_amd/csrc/gemm.hip", "fp8_w8a8_quantized_amd/csrc/device.hpp",
                "fp8_w8a8_quantized_amd/csrc/launch.hpp"]


def gemm_source_hash() -> str:
    """SHA-256 of the GEMM sources' code: line comments, trailing blanks and
    empty lines are dropped, so a comment edit keeps recorded counters valid."""
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per M=8192 GEMM launch from the committed counter summary, or
    None when the summary is missing or was taken on other GEMM sources."""
    try:
        fields = {}
        with open(TRAFFIC_SUMMARY) as f:
            for line in f:
                if line.startswith("- `") and "`: " in line:
                    k, v = line[3:].split("`: ", 1)
                    fields[k] = v.strip().strip("`")
        if fields.get("source_sha256") != gemm_source_hash():
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def calibrate_copy():
    """A plain 1 GiB device-to-device copy, three times (for the counter runs)."""
    import torch

    dev = torch.device("cuda:0")
    n = 1 << 30
    src = torch.full((n,), 3, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def one_gemm(M: int, N: int, K: int, reps: int, copies: int = 1):
    """One block-scaled GEMM shape, reps launches (for counter runs).  With
    copies > 1 the launches rotate over that many distinct operand sets, so
    weights stream from HBM as in a model's layers."""
    import torch

    import fp8_w8a8_quantized_amd as fp8
    import synth

    dev = torch.device("cuda:0")
    ops = []
    for c in range(copies):
        X = synth.act_col_outliers(M, K, seed=1 + 2 * c, device=dev)
        W = synth.weight(N, K, seed=2 + 2 * c, device=dev)
        a = fp8.quantize_block(X)
        (w,) = fp8.requantize_weights([W], fp8.SCALE_F32)
        ops.append((a, w))
        del X, W
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((max(fp8.gemm_workspace_size(M, N, K), 16),), dtype=torch.uint8, device=dev)
    for a, w in ops:  # warm-up: one launch per operand set
        fp8.gemm_a8w8_scaled(a, w, fp8.GRAN_BLOCK, out=y, workspace=ws)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        a, w = ops[r % copies]
        fp8.gemm_a8w8_scaled(a, w, fp8.GRAN_BLOCK, out=y, workspace=ws)
    e1.record()
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) * 1e3 / reps
    print(json.dumps({"gemm": [M, N, K], "reps": reps, "copies": copies, "avg_us": round(us, 2),
                      "tflops": round(2.0 * M * N * K / us / 1e6, 1)}))


def vendor_compare(reps: int):
    """The M=8192 dense shapes on this library's row- and block-scaled GEMMs
    and on torch._scaled_mm (the vendor library; row-wise and per-tensor FP8
    scales), same box, same codes for the row-wise pair (one JSON line per
    shape and GEMM).  Two operand sets alternate, as layers would."""
    import torch

    import fp8_w8a8_quantized_amd as fp8
    import synth

    dev = torch.device("cuda:0")

    def timed(fn, n):
        for i in range(2):
            fn(i)
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) * 1e3 / n

    for name, (N, K) in synth.DENSE_SHAPES.items():
        M = 8192
        row, blk = [], []
        for c in range(2):
            X = synth.act_col_outliers(M, K, seed=1 + 2 * c, device=dev)
            W = synth.weight(N, K, seed=2 + 2 * c, device=dev)
            row.append((fp8.quantize_token(X), fp8.quantize_token(W)))
            blk.append((fp8.quantize_block(X), fp8.requantize_weights([W], fp8.SCALE_F32)[0]))
            del X, W
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty((16,), dtype=torch.uint8, device=dev)
        one = torch.ones((), dtype=torch.float32, device=dev)

        def vend(i, per_tensor=False):
            (qa, sa), (qw, sw) = row[i % 2]
            a8 = qa.view(torch.float8_e4m3fn)
            w8 = qw.view(torch.float8_e4m3fn)
            if per_tensor:
                return torch._scaled_mm(a8, w8.t(), scale_a=one, scale_b=one,
                                        out_dtype=torch.bfloat16)
            return torch._scaled_mm(a8, w8.t(), scale_a=sa.view(M, 1), scale_b=sw.view(1, N),
                                    out_dtype=torch.bfloat16)

        calls = {
            "library_row": lambda i: fp8.gemm_a8w8_scaled(*row[i % 2], fp8.GRAN_ROW, out=y,
                                                          workspace=ws),
            "library_block": lambda i: fp8.gemm_a8w8_scaled(*blk[i % 2], fp8.GRAN_BLOCK, out=y,
                                                            workspace=ws),
            "vendor_row": lambda i: vend(i),
            "vendor_tensor": lambda i: vend(i, True),
        }
        # two rounds over the four, keeping each one's faster round
        res = {}
        for _ in range(2):
            for kind, fn in calls.items():
                us = timed(fn, reps)
                res[kind] = min(us, res.get(kind, us))
        # the row-wise pair computes the same products: their outputs agree to bf16 rounding
        fp8.gemm_a8w8_scaled(*row[0], fp8.GRAN_ROW, out=y, workspace=ws)
        ref = vend(0).float()
        rel = float(((y.float() - ref).abs().amax(dim=1) /
                     ref.abs().amax(dim=1).clamp_min(1e-30)).max())
        for kind, us in res.items():
            print(json.dumps({"shape": name, "M": M, "N": N, "K": K, "gemm": kind,
                              "avg_us": round(us, 2),
                              "tflops": round(2.0 * M * N * K / us / 1e6, 1),
                              "row_pair_max_rel_diff": round(rel, 6)}), flush=True)


def environment(torch, dev) -> dict:
    """What the numbers were measured on: versions, device, clocks, host CPU."""
    props = torch.cuda.get_device_properties(dev)
    env = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
           "device": torch.cuda.get_device_name(dev),
           "arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count,
           "hbm_gib": round(props.total_memory / 2**30, 1), "host_cpu": host_cpu_model()}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    env["sclk"] = gpu_clock()
    return env


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gpu_clock():
    """Current and maximum shader clock as rocm-smi reports them (None if it
    cannot be read)."""
    import subprocess

    # under rocprofv3 the child would inherit the profiler's preloaded
    # library and start on the GPU before rocm-smi's interpreter replaces it
    if any(k.startswith("ROCPROF") for k in os.environ):
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                           timeout=20)
        lines = [ln.strip() for ln in r.stdout.splitlines() if "sclk" in ln.lower()]
        return lines[0] if lines else None
    except Exception:
        return None


def measured_peaks(torch, L, dev, stream) -> dict:
    """Peaks measured on this GPU: the matrix-core rate of the library's
    register-operand MFMA probe, and a plain 1 GiB device copy (2 GiB moved)."""
    import ctypes

    out = torch.empty((4096,), dtype=torch.float32, device=dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    iters = 20000
    L.fp8_mfma_rate_probe(1000, ctypes.c_void_p(out.data_ptr()), sptr)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    rc = L.fp8_mfma_rate_probe(iters, ctypes.c_void_p(out.data_ptr()), sptr)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    assert rc == 0, rc
    flops = 4096.0 * iters * 8 * 2 * 16 * 16 * 128
    mfma = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    n = 1 << 30
    src = torch.full((n,), 3, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    copy = 5 * 2.0 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return {"mfma_fp8_tflops": round(mfma, 1), "copy_gbs": round(copy, 1),
            "mfma_probe": "4096 waves x 8 independent 16x16x128 E4M3 MFMA chains, register operands",
            "copy_probe": "torch copy_ of 1 GiB device to device, bytes read + written"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=8192)
    ap.add_argument("--cpu-sample-layers", type=int, default=3)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--one-gemm", type=int, nargs=3, metavar=("M", "N", "K"))
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--copies", type=int, default=1)
    ap.add_argument("--vendor-compare", action="store_true")
    return ap.parse_args()


def cpu_baseline(rows: int, layers: int):
    """The oracle (as it stands) on a bounded sample of a step: for `layers`
    layers, re-quantize the four bf16 weights, quantize `rows` rows of each
    M = 8192 activation and run the fp64 GEMM of those rows.  Reported in GEMM
    TFLOP/s."""
    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info

        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = 1
    omp = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    flops = 0.0
    elapsed = 0.0
    for li in range(layers):
        inputs = []
        for j, name in enumerate(synth.DENSE_SHAPES):
            N, K = synth.DENSE_SHAPES[name]
            X = synth.act_col_outliers(rows, K, seed=500 + 8 * li + j)
            W = synth.weight(N, K, seed=600 + 8 * li + j)
            inputs.append((X, W))
        t0 = time.perf_counter()
        for X, W in inputs:
            qw, sw = oracle.quantize_weight_block(W, 0)
            qa, sa = oracle.quantize_block(X)
            y = oracle.gemm(qa, qw, sa, sw, oracle.GRAN_BLOCK)
            flops += 2.0 * y.shape[0] * y.shape[1] * qa.shape[1]
        elapsed += time.perf_counter() - t0
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": max(omp, blas),
        "omp_threads": omp, "blas_threads": blas, "host_cpus": os.cpu_count(),
        "cpu_model": host_cpu_model(),
        "kind": "oracle",
        "sample": (f"{layers} layers of the step: requantize each layer's 4 bf16 weights "
                   f"(128x128, fp32 scales), 1x128-quantize {rows} rows of each M=8192 "
                   f"activation, fp64 dequantize-then-matmul of those rows; "
                   f"{flops / 1e9:.1f} GFLOP in {elapsed:.1f} s (input generation not timed)"),
    }


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.one_gemm:
        one_gemm(*args.one_gemm, args.reps, args.copies)
        return
    if args.vendor_compare:
        vendor_compare(args.reps if args.reps > 3 else 10)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1 "
                          "(the sharded path is not built)"}))
        sys.exit(2)

    import torch

    import fp8_w8a8_quantized_amd as fp8
    import synth

    L = fp8.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    vp = ctypes.c_void_p

    shapes = list(synth.DENSE_SHAPES.items())
    Ms = synth.DENSE_M
    layers = args.layers

    # ---- inputs (device-generated, seeded) and preallocated outputs ----
    W, Wq, Ws = [], [], []
    X, Xq, Xs = {}, {}, {}
    Y = {}
    for li in range(layers):
        for j, (name, (N, K)) in enumerate(shapes):
            W.append(synth.weight(N, K, seed=10_000 + 4 * li + j, device=dev))
            Wq.append(torch.empty((N, K), dtype=torch.uint8, device=dev))
            Ws.append(torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev))
            for M in Ms:
                X[(li, j, M)] = synth.act_col_outliers(M, K, seed=20_000 + 8 * li + 2 * j + M,
                                                       device=dev)
                Xq[(li, j, M)] = torch.empty((M, K), dtype=torch.uint8, device=dev)
                Xs[(li, j, M)] = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    for j, (name, (N, K)) in enumerate(shapes):
        for M in Ms:
            Y[(j, M)] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    descs = (fp8._WeightDesc * len(W))()
    for i in range(len(W)):
        descs[i] = fp8._WeightDesc(W[i].data_ptr(), Wq[i].data_ptr(), Ws[i].data_ptr(),
                                   W[i].shape[0], W[i].shape[1])

    # per-token path: RMSNorm + per-token quant -> row-scaled GEMM
    RM, RK, RN = synth.RMS_M, synth.RMS_K, synth.RMS_N
    h, gamma = synth.rms_inputs(seed=1, device=dev)
    # 8 distinct h buffers (63 MB each), one per step in turn, so the fused
    # RMSNorm + quant never reads an h the cache still holds
    NROT = 8
    hrot = [h] + [synth.rms_inputs(seed=1 + j, device=dev)[0] for j in range(1, NROT)]
    Wr = synth.weight(RN, RK, seed=31, device=dev)
    hx = synth.normal_bf16((RM, RK), seed=2, std=3.0, device=dev)  # residual stream
    hq = torch.empty((RM, RK), dtype=torch.uint8, device=dev)
    hs = torch.empty((RM,), dtype=torch.float32, device=dev)
    Wrq = torch.empty((RN, RK), dtype=torch.uint8, device=dev)
    Wrs = torch.empty((RN,), dtype=torch.float32, device=dev)
    Yr = torch.empty((RM, RN), dtype=torch.bfloat16, device=dev)

    # MoE path: token rows + routing, stacked expert weights, grouped GEMMs
    token_of_row, _ = synth.moe_routing()
    moe_tok = torch.as_tensor(token_of_row, dtype=torch.int32, device=dev)
    moe_x = synth.normal_bf16((synth.MOE_TOKENS, synth.MOE_HIDDEN), seed=11, device=dev)
    moe = {}
    for which in ("gate_up", "down"):
        A, Wm, offsets = synth.moe_inputs(which, seed=0, device=dev)
        E, N, K = Wm.shape
        T = A.shape[0]
        moe[which] = dict(
            A=A, W=Wm.reshape(E * N, K), E=E, N=N, K=K, T=T,
            off=torch.as_tensor(offsets, dtype=torch.int32, device=dev),
            Aq=torch.empty((T, K), dtype=torch.uint8, device=dev),
            As=torch.empty((T, K // 128), dtype=torch.float32, device=dev),
            Wq=torch.empty((E * N, K), dtype=torch.uint8, device=dev),
            Ws=torch.empty((E * N // 128, K // 128), dtype=torch.float32, device=dev),
            Y=torch.empty((T, N), dtype=torch.bfloat16, device=dev))
    # E8M0 variant: all policy weights again with E8M0 scales; layer 0 at M=8192
    Wq8 = [torch.empty_like(w, dtype=torch.uint8) for w in W]
    Ws8 = [torch.empty((w.shape[0] // 128, w.shape[1] // 128), dtype=torch.uint8, device=dev)
           for w in W]
    descs8 = (fp8._WeightDesc * len(W))()
    for i in range(len(W)):
        descs8[i] = fp8._WeightDesc(W[i].data_ptr(), Wq8[i].data_ptr(), Ws8[i].data_ptr(),
                                    W[i].shape[0], W[i].shape[1])
    MXM = 8192
    Xq8 = {j: torch.empty((MXM, K), dtype=torch.uint8, device=dev)
           for j, (name, (N, K)) in enumerate(shapes)}
    Xs8 = {j: torch.empty((MXM, K // 128), dtype=torch.uint8, device=dev)
           for j, (name, (N, K)) in enumerate(shapes)}

    # K/V cache recalibration: per-tensor quant of every layer's K and V
    kv_x, kv_q, kv_s = [], [], []
    for li in range(layers):
        for t in synth.kv_cache(li, seed=3, device=dev):
            kv_x.append(t)
            kv_q.append(torch.empty_like(t, dtype=torch.uint8))
            kv_s.append(torch.empty((), dtype=torch.float32, device=dev))
    kvdescs = (fp8._TensorDesc * len(kv_x))()
    for i, t in enumerate(kv_x):
        kvdescs[i] = fp8._TensorDesc(t.data_ptr(), kv_q[i].data_ptr(), kv_s[i].data_ptr(),
                                     t.numel())

    # output projection of the DeepSeek-V4-style attention: inverse RoPE + E8M0
    # group quant of o, batched MX GEMM over 8 head groups
    OT, OG, ON = synth.ROPE_TOKENS, synth.ROPE_GROUPS, synth.ROPE_OUT
    OKG = synth.ROPE_HEADS * synth.ROPE_HEAD_DIM // OG
    ro, rpos = synth.rope_inputs(OT, seed=7, device=dev)
    rpos = torch.as_tensor(rpos, device=dev)
    rcos, rsin = (torch.as_tensor(a, device=dev) for a in synth.rope_cache())
    rW = synth.normal_bf16((OG * ON, OKG), seed=8, std=0.02, device=dev)
    rWq = torch.empty_like(rW, dtype=torch.uint8)
    rWs = torch.empty((OG * ON // 128, OKG // 128), dtype=torch.uint8, device=dev)
    rdesc = (fp8._WeightDesc * 1)()
    rdesc[0] = fp8._WeightDesc(rW.data_ptr(), rWq.data_ptr(), rWs.data_ptr(), OG * ON, OKG)
    rq = torch.empty((OT, OG * OKG), dtype=torch.uint8, device=dev)
    rs = torch.empty((OT, OG * OKG // 128), dtype=torch.uint8, device=dev)
    rY = torch.empty((OT, OG, ON), dtype=torch.bfloat16, device=dev)

    mdescs = (fp8._WeightDesc * 2)()
    for i, which in enumerate(("gate_up", "down")):
        m = moe[which]
        mdescs[i] = fp8._WeightDesc(m["W"].data_ptr(), m["Wq"].data_ptr(), m["Ws"].data_ptr(),
                                    m["E"] * m["N"], m["K"])
    # the small-M GEMMs' partial-tile workspace: one buffer of the largest size
    # any shape queries, shared by the calls of the one stream
    ws_bytes = max(int(L.fp8_gemm_workspace_size(M, N, K, fp8.GRAN_BLOCK))
                   for (name, (N, K)) in shapes for M in Ms)
    ws_bytes = max(ws_bytes, int(L.fp8_gemm_workspace_size(RM, RN, RK, fp8.GRAN_ROW)))
    gws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)
    gwsa = (vp(gws.data_ptr()), gws.numel())
    torch.cuda.synchronize(dev)

    # ---- pre-marshalled calls of one step, grouped by kernel category ----
    calls = [("requant", L.fp8_requantize_weights, (descs, len(W), fp8.SCALE_F32, None, 0, sptr))]
    for li in range(layers):
        for j, (name, (N, K)) in enumerate(shapes):
            wi = 4 * li + j
            for M in Ms:
                key = (li, j, M)
                calls.append((f"quant_m{M}", L.fp8_quantize_block,
                              (vp(X[key].data_ptr()), M, K, vp(Xq[key].data_ptr()),
                               vp(Xs[key].data_ptr()), sptr), name))
                calls.append((f"gemm_m{M}", L.fp8_gemm_a8w8_scaled,
                              (vp(Xq[key].data_ptr()), vp(Wq[wi].data_ptr()),
                               vp(Xs[key].data_ptr()), vp(Ws[wi].data_ptr()), None,
                               vp(Y[(j, M)].data_ptr()), M, N, K, fp8.GRAN_BLOCK, *gwsa,
                               sptr), name))
    rms_at = len(calls)  # these two calls take h from the rotation, per step
    calls.append(("rmsnorm_quant", L.fp8_rmsnorm_quant,
                  (vp(hq.data_ptr()), vp(h.data_ptr()), vp(hs.data_ptr()), vp(gamma.data_ptr()),
                   synth.RMS_EPS, RM, RK, 0, sptr)))
    calls.append(("add_rmsnorm_quant", L.fp8_add_rmsnorm_quant,
                  (vp(hq.data_ptr()), vp(h.data_ptr()), vp(hx.data_ptr()), vp(hs.data_ptr()),
                   vp(gamma.data_ptr()), synth.RMS_EPS, RM, RK, 0, sptr)))
    rms_args = [[(vp(hq.data_ptr()), vp(hb.data_ptr()), vp(hs.data_ptr()), vp(gamma.data_ptr()),
                  synth.RMS_EPS, RM, RK, 0, sptr),
                 (vp(hq.data_ptr()), vp(hb.data_ptr()), vp(hx.data_ptr()), vp(hs.data_ptr()),
                  vp(gamma.data_ptr()), synth.RMS_EPS, RM, RK, 0, sptr)] for hb in hrot]
    calls.append(("quant_token_w", L.fp8_quantize_token,
                  (vp(Wr.data_ptr()), RN, RK, vp(Wrq.data_ptr()), vp(Wrs.data_ptr()), sptr)))
    calls.append(("gemm_row", L.fp8_gemm_a8w8_scaled,
                  (vp(hq.data_ptr()), vp(Wrq.data_ptr()), vp(hs.data_ptr()), vp(Wrs.data_ptr()),
                   None, vp(Yr.data_ptr()), RM, RN, RK, fp8.GRAN_ROW, *gwsa, sptr)))
    calls.append(("requant_e8m0", L.fp8_requantize_weights,
                  (descs8, len(W), fp8.SCALE_E8M0, None, 0, sptr)))
    for j, (name, (N, K)) in enumerate(shapes):
        key = (0, j, MXM)
        calls.append(("quant_e8m0_m8192", L.fp8_quantize_block_e8m0,
                      (vp(X[key].data_ptr()), MXM, K, vp(Xq8[j].data_ptr()),
                       vp(Xs8[j].data_ptr()), sptr)))
        calls.append(("gemm_mx_m8192", L.fp8_batched_gemm_a8w8_mxscale,
                      (vp(Xq8[j].data_ptr()), vp(Wq8[j].data_ptr()), vp(Xs8[j].data_ptr()),
                       vp(Ws8[j].data_ptr()), vp(Y[(j, MXM)].data_ptr()), 1, MXM, N, K, *gwsa,
                       sptr)))
    calls.append(("quant_kv_tensor", L.fp8_quantize_tensors, (kvdescs, len(kv_x), sptr)))
    calls.append(("requant_e8m0_wo", L.fp8_requantize_weights, (rdesc, 1, fp8.SCALE_E8M0, None, 0, sptr)))
    calls.append(("rope_quant_m8192", L.fp8_inverse_rope_group_quant,
                  (vp(ro.data_ptr()), vp(rpos.data_ptr()), vp(rcos.data_ptr()),
                   vp(rsin.data_ptr()), OT, synth.ROPE_HEADS, synth.ROPE_HEAD_DIM,
                   synth.ROPE_DIM, rcos.shape[0], OG, vp(rq.data_ptr()), vp(rs.data_ptr()),
                   sptr)))
    calls.append(("gemm_mx_wo_m8192", L.fp8_batched_gemm_a8w8_mxscale,
                  (vp(rq.data_ptr()), vp(rWq.data_ptr()), vp(rs.data_ptr()), vp(rWs.data_ptr()),
                   vp(rY.data_ptr()), OG, OT, ON, OKG, *gwsa, sptr)))
    calls.append(("requant_moe", L.fp8_requantize_weights, (mdescs, 2, fp8.SCALE_F32, None, 0, sptr)))
    # the expert chain: 1x128 quant of the routed rows, gate_up GEMM, SwiGLU +
    # 1x128 quant of its output, down GEMM
    mg, md = moe["gate_up"], moe["down"]
    assert mg["N"] == 2 * md["K"] and mg["T"] == md["T"]
    for which in ("gate_up", "down"):
        m = moe[which]
        if which == "gate_up":  # dispatch: gather each routed row's token, quantize 1x128
            calls.append(("quant_gather_moe", L.fp8_quantize_block_gather,
                          (vp(moe_x.data_ptr()), moe_x.shape[0], m["K"], vp(moe_tok.data_ptr()),
                           m["T"], vp(m["Aq"].data_ptr()), vp(m["As"].data_ptr()), sptr)))
        else:
            calls.append(("swiglu_quant_moe", L.fp8_swiglu_quant,
                          (vp(mg["Y"].data_ptr()), m["T"], m["K"], vp(m["Aq"].data_ptr()),
                           vp(m["As"].data_ptr()), sptr)))
        calls.append(("gemm_moe", L.fp8_grouped_gemm_a8w8_scaled,
                      (vp(m["Aq"].data_ptr()), vp(m["Wq"].data_ptr()), vp(m["As"].data_ptr()),
                       vp(m["Ws"].data_ptr()), vp(m["off"].data_ptr()), vp(m["Y"].data_ptr()),
                       m["T"], m["E"], m["N"], m["K"], sptr)))

    # algorithmic work per step, per category
    work = {"requant": {"bytes": 0.0}, "gemm_m8192": {"flops": 0.0, "bytes": 0.0},
            "gemm_m256": {"flops": 0.0, "bytes": 0.0}, "quant_m8192": {"bytes": 0.0},
            "quant_m256": {"bytes": 0.0}}
    for li in range(layers):
        for (name, (N, K)) in shapes:
            work["requant"]["bytes"] += 2 * N * K + N * K + 4 * (N // 128) * (K // 128)
            for M in Ms:
                work[f"quant_m{M}"]["bytes"] += 2 * M * K + M * K + 4 * M * (K // 128)
                g = work[f"gemm_m{M}"]
                g["flops"] += 2.0 * M * N * K
                g["bytes"] += M * K + N * K + 4 * (M * (K // 128) + (N // 128) * (K // 128)) \
                    + 2 * M * N
    work["rmsnorm_quant"] = {"bytes": 2 * RM * RK + RM * RK + 4 * RM + 2 * RK}
    work["add_rmsnorm_quant"] = {"bytes": 3 * 2 * RM * RK + RM * RK + 4 * RM + 2 * RK}
    work["quant_token_w"] = {"bytes": 2 * RN * RK + RN * RK + 4 * RN}
    work["gemm_row"] = {"flops": 2.0 * RM * RN * RK,
                        "bytes": RM * RK + RN * RK + 4 * (RM + RN) + 2 * RM * RN}
    work["requant_e8m0"] = {"bytes": 0.0}
    work["quant_e8m0_m8192"] = {"bytes": 0.0}
    work["gemm_mx_m8192"] = {"flops": 0.0, "bytes": 0.0}
    for li in range(layers):
        for (name, (N, K)) in shapes:
            work["requant_e8m0"]["bytes"] += 3 * N * K + (N // 128) * (K // 128)
    for (name, (N, K)) in shapes:
        work["quant_e8m0_m8192"]["bytes"] += 3 * MXM * K + MXM * (K // 128)
        work["gemm_mx_m8192"]["flops"] += 2.0 * MXM * N * K
        work["gemm_mx_m8192"]["bytes"] += (MXM * K + N * K + MXM * (K // 128)
                                           + (N // 128) * (K // 128) + 2 * MXM * N)
    work["quant_kv_tensor"] = {"bytes": float(sum(3 * t.numel() + 4 for t in kv_x))}
    work["requant_e8m0_wo"] = {"bytes": float(3 * OG * ON * OKG
                                              + (OG * ON // 128) * (OKG // 128))}
    rope_elems = OT * OG * OKG
    work["rope_quant_m8192"] = {"bytes": float(3 * rope_elems + rope_elems // 128 + 8 * OT
                                               + OT * synth.ROPE_DIM * 4)}
    work["gemm_mx_wo_m8192"] = {"flops": 2.0 * OT * OG * ON * OKG,
                                "bytes": float(rope_elems + OG * ON * OKG + rope_elems // 128
                                               + (OG * ON // 128) * (OKG // 128)
                                               + 2 * OT * OG * ON)}
    work["requant_moe"] = {"bytes": 0.0}
    work["quant_gather_moe"] = {"bytes": 0.0}
    work["swiglu_quant_moe"] = {"bytes": 0.0}
    work["gemm_moe"] = {"flops": 0.0, "bytes": 0.0}
    for m in moe.values():
        E, N, K, T = m["E"], m["N"], m["K"], m["T"]
        work["requant_moe"]["bytes"] += 3 * E * N * K + 4 * (E * N // 128) * (K // 128)
        if m is moe["gate_up"]:  # token rows read once, routed codes written
            work["quant_gather_moe"]["bytes"] += (2 * moe_x.numel() + 4 * T + T * K
                                                  + 4 * T * (K // 128))
        else:  # SwiGLU: reads gate and up (2 x 2 B), writes 1 B per output element
            work["swiglu_quant_moe"]["bytes"] += 5 * T * K + 4 * T * (K // 128)
        work["gemm_moe"]["flops"] += 2.0 * T * N * K
        work["gemm_moe"]["bytes"] += T * K + E * N * K + 4 * (T * (K // 128) + (E * N // 128)
                                                             * (K // 128)) + 2 * T * N
    launches = {"requant": 1, "rmsnorm_quant": 1, "add_rmsnorm_quant": 1, "quant_token_w": 1,
                "gemm_row": 1,
                "requant_moe": 1, "quant_gather_moe": 1, "swiglu_quant_moe": 1, "gemm_moe": 2,
                "requant_e8m0": 1,
                "quant_e8m0_m8192": len(shapes), "gemm_mx_m8192": len(shapes),
                "quant_kv_tensor": 1, "requant_e8m0_wo": 1, "rope_quant_m8192": 1,
                "gemm_mx_wo_m8192": 1}
    for M in Ms:
        launches[f"quant_m{M}"] = launches[f"gemm_m{M}"] = layers * len(shapes)

    def run_step(step, events=None):
        for ci, call in enumerate(calls):
            cat, fn, a = call[:3]
            if rms_at <= ci < rms_at + 2:
                a = rms_args[step % NROT][ci - rms_at]
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            rc = fn(*a)
            if rc != 0:
                raise fp8.Fp8Error(cat, rc, fp8.status_string(rc))
            if events is not None:
                e1.record(stream)
                events.append((cat, call[3] if len(call) > 3 else None, e0, e1))

    peaks = measured_peaks(torch, L, dev, stream)
    for w in range(args.warmup):
        run_step(w)
    torch.cuda.synchronize(dev)

    # ---- timed region: exactly `steps` steps, wall clock, synchronized; no
    # per-op events inside it (they would add their own commands to the step)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for k in range(args.steps):
        run_step(args.warmup + k)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0

    # ---- the same steps again with a HIP event pair around every launch, for
    # the per-op breakdown (each pair spans its launch on the library's stream)
    events = []
    for k in range(args.steps):
        run_step(args.warmup + args.steps + k, events)
    torch.cuda.synchronize(dev)

    per_cat_ms, per_shape_ms = {}, {}
    for cat, shape, e0, e1 in events:
        ms = e0.elapsed_time(e1)
        per_cat_ms[cat] = per_cat_ms.get(cat, 0.0) + ms
        if shape is not None:
            per_shape_ms[(cat, shape)] = per_shape_ms.get((cat, shape), 0.0) + ms
    ms_per_step = elapsed * 1e3 / args.steps
    total_flops = sum(w.get("flops", 0.0) for w in work.values())
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    breakdown = {}
    for cat, w in work.items():
        ms = per_cat_ms.get(cat, 0.0) / args.steps  # per step, summed over launches
        d = {"ms_per_step": round(ms, 4), "launches_per_step": launches[cat],
             "avg_launch_us": round(ms * 1e3 / launches[cat], 3)}
        if "flops" in w:
            d["tflops"] = round(w["flops"] / (ms * 1e-3) / 1e12, 2)
            d["frac_fp8_peak"] = round(d["tflops"] / PEAK_FP8_TFLOPS, 4)
            d["frac_measured_mfma"] = round(d["tflops"] / peaks["mfma_fp8_tflops"], 4)
        d["gbs"] = round(w["bytes"] / (ms * 1e-3) / 1e9, 1)
        d["frac_hbm"] = round(d["gbs"] / PEAK_HBM_GBS, 4)
        d["frac_measured_copy"] = round(d["gbs"] / peaks["copy_gbs"], 4)
        breakdown[cat] = d

    # the four linears of each M: one launch per layer and step
    per_shape = {}
    for (cat, shape), ms_total in per_shape_ms.items():
        N, K = synth.DENSE_SHAPES[shape]
        M = int(cat.split("_m")[1])
        us = ms_total * 1e3 / (args.steps * layers)
        d = {"M": M, "N": N, "K": K, "avg_launch_us": round(us, 3)}
        if cat.startswith("gemm"):
            flops = 2.0 * M * N * K
            nbytes = M * K + N * K + 4 * (M * (K // 128) + (N // 128) * (K // 128)) + 2 * M * N
            d["tflops"] = round(flops / us / 1e6, 2)
            d["frac_fp8_peak"] = round(d["tflops"] / PEAK_FP8_TFLOPS, 4)
            d["frac_hbm_roofline"] = round(max(flops / (PEAK_FP8_TFLOPS * 1e12),
                                               nbytes / (PEAK_HBM_GBS * 1e9)) / (us * 1e-6), 4)
        else:
            nbytes = 3 * M * K + 4 * M * (K // 128)
            d["gbs"] = round(nbytes / us / 1e3, 1)
            d["frac_hbm"] = round(d["gbs"] / PEAK_HBM_GBS, 4)
        per_shape.setdefault(cat, {})[shape] = d

    # the fused RMSNorm (+ residual) over the 8 rotated h buffers, alone
    def rms_rotated(which):
        fn = L.fp8_rmsnorm_quant if which == 0 else L.fp8_add_rmsnorm_quant
        for j in range(NROT):
            fn(*rms_args[j][which])
        torch.cuda.synchronize(dev)
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 4 * NROT
        ea.record(stream)
        for j in range(reps):
            fn(*rms_args[j % NROT][which])
        eb.record(stream)
        torch.cuda.synchronize(dev)
        us = ea.elapsed_time(eb) * 1e3 / reps
        nbytes = work["rmsnorm_quant" if which == 0 else "add_rmsnorm_quant"]["bytes"]
        return {"avg_launch_us": round(us, 3), "gbs": round(nbytes / us / 1e3, 1),
                "frac_hbm": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4),
                "buffers": NROT, "launches": reps}

    rotated = {"rmsnorm_quant": rms_rotated(0), "add_rmsnorm_quant": rms_rotated(1)}

    dom = breakdown["gemm_m8192"]
    flops_per_launch = work["gemm_m8192"]["flops"] / launches["gemm_m8192"]
    achieved = flops_per_launch / (dom["avg_launch_us"] * 1e-6) / 1e12
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
        "traffic": recorded_traffic(),
        "frac_of_measured_mfma": round(achieved / peaks["mfma_fp8_tflops"], 4),
        "kernel": "block-scaled FP8 GEMM k_gemm_pp<0, false>, the 144 M=8192 launches of a "
                  "step",
    }

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {
            "workload": ("qwen3-8b-shaped dense linears, block-scaled W8A8: per step, "
                         "128x128 re-quantization of the 36-layer bf16 policy, then for "
                         "every layer and linear 1x128 activation quant + GEMM at M=8192 "
                         "and M=256; plus once per step the per-token path (RMSNorm + "
                         "per-token quant of [4096,5120], its residual-add form, per-row weight quant of "
                         "[12288,5120], row-scaled GEMM) and the qwen3-30b-a3b-shaped MoE "
                         "path (expert re-quant, token gather + 1x128 quant of 32768 routed rows, grouped "
                         "GEMM gate_up 2048->1536, SwiGLU + 1x128 quant, grouped GEMM down "
                         "768->2048, over 128 experts), "
                         "and the E8M0 variant (the policy re-quantized with E8M0 scales, one "
                         "layer's four linears at M=8192 through E8M0 activation quant and "
                         "the MX-scaled GEMM), the K/V cache recalibration (per-tensor "
                         "quant of every layer's K and V, [8192, 1024] each), and an "
                         "attention output projection (inverse RoPE + E8M0 group quant of "
                         "o [8192, 64 heads, 128], batched MX GEMM over 8 head groups "
                         "1024->1024, its weight re-quantized with E8M0 scales)"),
            "layers": layers, "M": list(Ms),
            "linears": {name: {"N": N, "K": K} for name, (N, K) in shapes},
            "per_token": {"M": RM, "K": RK, "N": RN},
            "kv_cache": {"tensors": len(kv_x), "shape": list(kv_x[0].shape)},
            "out_proj_rope": {"tokens": OT, "heads": synth.ROPE_HEADS,
                              "head_dim": synth.ROPE_HEAD_DIM, "rope_dim": synth.ROPE_DIM,
                              "groups": OG, "N_per_group": ON, "K_per_group": OKG},
            "moe": {"experts": moe["gate_up"]["E"], "rows": moe["gate_up"]["T"],
                    "gate_up": {"N": moe["gate_up"]["N"], "K": moe["gate_up"]["K"]},
                    "down": {"N": moe["down"]["N"], "K": moe["down"]["K"]}},
            "parallelism": "single-gpu",
        },
        "roofline": roofline,
        "measured_peaks": peaks,
        "breakdown": breakdown,
        "per_shape": per_shape,
        "rotated_inputs": rotated,
        "env": environment(torch, dev),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_sample_rows, args.cpu_sample_layers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
