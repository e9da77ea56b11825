#!/usr/bin/env python3
"""Throughput of the 4-bit codec and dequantize-and-multiply on one MI355X.

Workload (LLM MLP up-projection): bf16 weight [14336, 4096], N(0, 0.02^2) with
0.1 % entries scaled x20, NF4, block 64, double-quantized scales (8-bit, groups
of 256, fp32 group scale, mean offset); x bf16 [1, 4096]; A bf16 [512, 4096].

A step is one pass of the whole path on that weight: quantize_4bit ->
double_quant -> dequantize_4bit (to bf16) -> gemv_4bit (M = 1) ->
gemm_4bit (M = 512).  The headline value is gemv_4bit's achieved HBM
bandwidth: algorithmic bytes per launch / average launch duration, timed with
HIP events on the launch stream while rotating over distinct weight copies
(> 512 MB, twice the 256 MB Infinity Cache) so the bytes come from HBM.
Each kernel is also timed alone, including gemm_4bit_backward (dX = dY @
W_hat with a bf16 dY [512, 14336]) and the 8-bit blockwise codec on the same
bf16 weight (blocksize 4096; linear and dynamic-tree tables) and an
embedding gather (8192 random rows of a 128256 x 4096 NF4 table to bf16),
which are not part of the step.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
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
sys.path.insert(0, ROOT)

METRIC = "gemv_4bit achieved HBM GB/s (NF4, 14336x4096, M=1) + codec GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores
N, K, BS, BS2, M_GEMV, M_GEMM = 14336, 4096, 64, 256, 1, 512
BS8 = 4096                     # 8-bit blockwise codec block size
EMB_V, EMB_T = 128256, 8192    # embedding table rows (x K columns) and gathered tokens
ROTATE_BYTES = 640 << 20       # > 2 x 256 MB Infinity Cache


def algorithmic_bytes():
    """Bytes each op must move at this workload (intermediates excluded)."""
    numel = N * K
    nb = numel // BS
    dq_state = nb + 4 * (-(-nb // BS2)) + 4 + 4 * 256     # codes, group scales, offset, table
    packed = numel // 2
    return {
        "quantize_4bit+double_quant": 2 * numel + packed + dq_state,
        "dequantize_4bit": packed + dq_state + 2 * numel,
        "gemv_4bit": packed + dq_state + 2 * K * M_GEMV + 2 * N * M_GEMV,
        "gemm_4bit": packed + dq_state + 2 * K * M_GEMM + 2 * N * M_GEMM,
        # 8-bit blockwise codec: bf16 in / out, one code byte and fp32 scales
        "quantize_blockwise": 2 * numel + numel + 4 * (numel // BS8),
        "quantize_blockwise_dynamic": 2 * numel + numel + 4 * (numel // BS8),
        "dequantize_blockwise": numel + 4 * (numel // BS8) + 2 * numel,
        # embedding gather: the gathered rows' codes, scale codes and group
        # scales, the indices and the bf16 output rows
        "embedding_4bit": EMB_T * (K // 2 + K // BS + 4 * (K // BS) // BS2 + 8 + 2 * K),
    }


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


GEMV_SOURCES = ["quantized_matvec_amd/csrc/qmv_gemv.hip", "quantized_matvec_amd/csrc/qmv_device.hpp",
                "quantized_matvec_amd/csrc/qmv_launch.hpp"]


def measured_traffic():
    """HBM bytes per gemv launch from the committed rocprofv3 counter summary
    (lines "key: value"), or None when the kernel source changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", "gemv_4bit_nf4_14336x4096_m1_traffic.txt")
    d = {}
    try:
        with open(path) as f:
            for line in f:
                k, sep, v = line.partition(":")
                if sep and k.strip() and not k.startswith(("#", " ")):
                    d[k.strip()] = v.strip()
    except OSError:
        return None
    if d.get("kernel_source_sha256") != source_hash(GEMV_SOURCES):
        return None
    try:
        return int(float(d["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def timed_loop(fn, iters, stream, torch):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(iters):
        fn(i)
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters * 1e3   # microseconds per call


def cpu_baseline(W_cpu, x_cpu, budget_s=15.0, rows=256):
    """The oracle's gemv on a bounded sample: the first `rows` output rows of
    the weight, single-threaded.  Untimed set-up: block scales of the whole
    weight (the double-quant mean needs all of them), double quant, and the
    oracle quantize of the sampled rows.  Timed, repeated until `budget_s`:
    scale reconstruction of the sampled blocks, dequantization and the float64
    matmul.  Bytes are counted per output row exactly as for the GPU kernel."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle as O
    W64 = W_cpu.to(torch.float64).numpy()
    x64 = x_cpu.to(torch.float64).numpy()
    with threadpool_limits(limits=1):
        absmax = O.block_absmax(W64, BS).astype(np.float32)
        q, a2, off = O.double_quant(absmax, BS2)
        packed, _ = O.quantize_4bit(W64[:rows], BS, "nf4")
        nbs = rows * K // BS
        passes, t0 = 0, time.perf_counter()
        while True:
            ahat = O.dequant_absmax(q[:nbs], a2[:-(-nbs // BS2)], off, None, BS2)
            O.matmul_4bit(x64, packed, ahat, rows, K, BS, "nf4")
            passes += 1
            t = time.perf_counter() - t0
            if t >= budget_s:
                break
    per_row = K // 2 + K // BS * (1 + 4 / BS2) + 2 * M_GEMV      # packed + DQ scales + y
    gbs = passes * rows * per_row / t / 1e9
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle gemv (DQ scale decode + dequantize + float64 matmul) over the first "
                      f"{rows} of {N} output rows, {passes} passes in {t:.1f} s on one thread; "
                      f"bytes per row counted as for the GPU kernel"}


COPY_BYTES = 1 << 30


def measured_ceilings(torch, dev, reps=20):
    """Streaming ceilings of this GPU, to read the kernels' GB/s against: a
    plain 128-bit read of 1 GiB (the library's stream_read probe) and torch's
    device copy of 1 GiB (bytes read + written).  Event-timed on torch's
    current stream, the probe's launch stream, after two warm-up passes."""
    from quantized_matvec_amd import qmv
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {}
    for name, fn, nbytes in (("read_gbs", lambda: qmv.stream_read(src, sink), COPY_BYTES),
                             ("copy_gbs", lambda: dst.copy_(src), 2 * COPY_BYTES)):
        for _ in range(2):
            fn()
        st = torch.cuda.current_stream(dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        b.synchronize()
        us = a.elapsed_time(b) / reps * 1e3
        out[name] = round(nbytes / us / 1e3, 1)
    del src, dst
    out["method"] = ("stream_read probe over 1 GiB (128-bit loads, grid-stride) and torch copy_ of 1 GiB "
                     "(bytes read + written), event-timed")
    return out


def host_info():
    """The host side of the cpu_baseline: CPU model, usable and total cores,
    numpy's BLAS thread pools."""
    import os
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": d.get("internal_api"), "threads": d.get("num_threads")} for d in threadpool_info()]
    except Exception:  # noqa: BLE001 - informational only
        blas = []
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "cpu_count": os.cpu_count(), "blas_pools": blas}


def counters_run(name, fns, n_copies, dev, torch):
    """A short program for rocprofv3 counter passes: a plain 1 GiB device copy
    (its FETCH_SIZE / WRITE_SIZE per byte calibrate the counters), then ten
    launches of one kernel, each on a different weight copy."""
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy of {COPY_BYTES} bytes done", flush=True)
    for i in range(10):
        fns[name](i % n_copies)
    torch.cuda.synchronize()
    print(f"10 launches of {name} done", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--kernel-iters", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters", choices=["gemv_4bit", "gemm_4bit", "dequantize_4bit", "quantize_4bit"],
                    help="for hardware-counter runs: one 1 GiB copy (the calibration kernel), "
                         "then 10 launches of the named kernel over distinct weight copies")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_matvec_amd import build as qbuild
    from quantized_matvec_amd import qmv, synth
    if not os.path.exists(qmv.library_path):
        qbuild.build()
    qmv.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)      # default priority
    ab = algorithmic_bytes()

    W_cpu = synth.weight(3, 0)                   # [14336, 4096] bf16 with outliers
    x_cpu = synth.activations(3, 0, M_GEMV)
    A_cpu = synth.gaussian((M_GEMM, K), 1.0, 100 * 4 + 2, "bf16")

    with torch.cuda.stream(stream):
        W = W_cpu.to(dev)
        x = x_cpu.to(dev)
        A = A_cpu.to(dev)
        packed0, st0 = qmv.quantize_4bit(W, BS, "nf4", double_quant=True, blocksize2=BS2)
        # distinct copies so repeated launches stream from HBM, not the cache
        n_w = max(2, -(-ROTATE_BYTES // (W.numel() * 2)))
        n_p = max(2, -(-ROTATE_BYTES // packed0.numel()))
        Ws = [W] + [W.clone() for _ in range(n_w - 1)]
        packs = [packed0] + [packed0.clone() for _ in range(n_p - 1)]
        states = [st0] + [qmv.QuantState(st0.shape, st0.dtype, BS, "nf4", None, st0.absmax_q.clone(),
                                         st0.absmax2.clone(), st0.offset.clone(), st0.code2.clone(), BS2)
                          for _ in range(n_p - 1)]
        wout = [torch.empty(N, K, dtype=torch.bfloat16, device=dev) for _ in range(n_w)]
        y = torch.empty(M_GEMV, N, dtype=torch.bfloat16, device=dev)
        C = torch.empty(M_GEMM, N, dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()

        def step(i):
            p, st = qmv.quantize_4bit(Ws[i % n_w], BS, "nf4", double_quant=True, blocksize2=BS2)
            qmv.dequantize_4bit(p, st, out=wout[i % n_w])
            qmv.gemv_4bit(x, p, st, out=y)
            qmv.gemm_4bit(A, p, st, out=C)

        if args.counters:
            counters_run(args.counters, dict(gemv_4bit=lambda i: qmv.gemv_4bit(x, packs[i], states[i], out=y),
                                             gemm_4bit=lambda i: qmv.gemm_4bit(A, packs[i], states[i], out=C),
                                             dequantize_4bit=lambda i: qmv.dequantize_4bit(
                                                 packs[i], states[i], out=wout[i % n_w]),
                                             quantize_4bit=lambda i: qmv.quantize_4bit(
                                                 Ws[i % n_w], BS, "nf4")), n_p, dev, torch)
            return

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        us_step = timed_loop(step, args.steps, stream, torch)
        torch.cuda.synchronize()
        wall_step_ms = (time.perf_counter() - t0) * 1e3 / args.steps

        kiters = args.kernel_iters
        kern = {}
        # per-kernel loops call the C ABI directly with prepared arguments,
        # so the host keeps ahead of kernels of a few microseconds
        L = qmv.lib()
        s_h = stream.cuda_stream
        structs = [st._c() for st in states]          # kept alive for the byref handles
        scs = [ctypes.byref(c) for c in structs]
        p_ptr = [p.data_ptr() for p in packs]
        x_ptr, y_ptr, A_ptr, C_ptr = x.data_ptr(), y.data_ptr(), A.data_ptr(), C.data_ptr()
        w_ptr = [w.data_ptr() for w in wout]

        def run_gemv(i):
            L.qmv_gemv_4bit(x_ptr, 2, M_GEMV, N, K, p_ptr[i % n_p], scs[i % n_p], BS, 0, y_ptr, 2, None,
                            s_h)

        def run_gemm(i):
            L.qmv_gemm_4bit(A_ptr, 2, M_GEMM, N, K, p_ptr[i % n_p], scs[i % n_p], BS, 0, C_ptr, 2, None,
                            s_h)

        def run_deq(i):
            L.qmv_dequantize_4bit(p_ptr[i % n_p], scs[i % n_p], N * K, BS, 0, w_ptr[i % n_w], 2, s_h)

        qbuf = [torch.empty_like(packed0) for _ in range(n_w)]
        abuf = [torch.empty_like(st0.absmax_q, dtype=torch.float32) for _ in range(n_w)]

        def run_quant(i):      # the raw entry point (no allocation inside the loop)
            L.qmv_quantize_4bit(Ws[i % n_w].data_ptr(), 2, N * K, BS, 0, qbuf[i % n_w].data_ptr(),
                                abuf[i % n_w].data_ptr(), s_h)

        dq_out = [(torch.empty_like(st0.absmax_q), torch.empty_like(st0.absmax2),
                   torch.empty_like(st0.offset), torch.empty_like(st0.code2)) for _ in range(n_w)]
        nbk = N * K // BS
        ws = torch.zeros(L.qmv_double_quant_workspace(nbk), dtype=torch.uint8, device=dev)

        def run_dq(i):
            q, a2, off, c2 = dq_out[i % n_w]
            L.qmv_double_quant(abuf[i % n_w].data_ptr(), nbk, BS2, None, q.data_ptr(), a2.data_ptr(),
                               off.data_ptr(), c2.data_ptr(), ws.data_ptr(), ws.numel(), s_h)

        # gemm_4bit_backward (dX = dY @ W_hat) on the same weight, dY [512, 14336]
        dY = synth.gaussian((M_GEMM, N), 1.0, 100 * 4 + 3, "bf16").to(dev)
        dX = torch.empty(M_GEMM, K, dtype=torch.bfloat16, device=dev)
        dY_ptr, dX_ptr = dY.data_ptr(), dX.data_ptr()

        def run_bwd(i):
            L.qmv_gemm_4bit_backward(dY_ptr, 2, M_GEMM, N, K, p_ptr[i % n_p], scs[i % n_p], BS, 0,
                                     dX_ptr, 2, s_h)

        # the 8-bit blockwise codec on the same bf16 weights (blocksize 4096),
        # with the default linear table and with the dynamic-tree table
        q8 = [torch.empty(N * K, dtype=torch.uint8, device=dev) for _ in range(n_w)]
        a8 = [torch.empty(N * K // BS8, dtype=torch.float32, device=dev) for _ in range(n_w)]
        tree = (ctypes.c_float * 256)(*qmv.dynamic_tree_code())
        tree_p = ctypes.cast(tree, ctypes.c_void_p)

        def run_q8(i, code=None):
            L.qmv_quantize_blockwise(Ws[i % n_w].data_ptr(), 2, N * K, BS8, code, q8[i % n_w].data_ptr(),
                                     a8[i % n_w].data_ptr(), s_h)

        def run_dq8(i):
            L.qmv_dequantize_blockwise(q8[i % n_w].data_ptr(), a8[i % n_w].data_ptr(), N * K, BS8, None,
                                       w_ptr[i % n_w], 2, s_h)

        # embedding_4bit: EMB_T random rows of a [EMB_V, K] NF4 table (block 64,
        # double-quantized scales) to bf16
        # (the table is drawn on the device: torch's seeded normal generator)
        g = torch.Generator(device=dev).manual_seed(100 * 4 + 6)
        E = torch.randn((EMB_V, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        pe, ste = qmv.quantize_4bit(E, BS, "nf4", double_quant=True, blocksize2=BS2)
        del E
        eidx = torch.randint(0, EMB_V, (EMB_T,), generator=g, device=dev, dtype=torch.int64)
        eout = torch.empty(EMB_T, K, dtype=torch.bfloat16, device=dev)
        ec = ste._c()

        def run_emb(i):
            L.qmv_embedding_4bit(eidx.data_ptr(), EMB_T, EMB_V, K, pe.data_ptr(), ctypes.byref(ec), BS, 0,
                                 eout.data_ptr(), 2, s_h)

        for name, fn, iters in (("gemv_4bit", run_gemv, kiters), ("gemm_4bit", run_gemm, kiters // 4),
                                ("gemm_4bit_backward", run_bwd, kiters // 8),
                                ("dequantize_4bit", run_deq, kiters // 4),
                                ("quantize_4bit", run_quant, kiters // 4),
                                ("double_quant", run_dq, kiters // 4),
                                ("quantize_blockwise", run_q8, kiters // 4),
                                ("quantize_blockwise_dynamic", lambda i: run_q8(i, tree_p), kiters // 4),
                                ("dequantize_blockwise", run_dq8, kiters // 4),
                                ("embedding_4bit", run_emb, kiters // 4)):
            for i in range(5):
                fn(i)
            kern[name] = timed_loop(fn, iters, stream, torch)

    rep = {}
    for name, us in kern.items():
        e = {"us_per_launch": round(us, 3)}
        if name in ("gemm_4bit", "gemm_4bit_backward"):
            fl = 2.0 * M_GEMM * N * K
            e.update(flops=fl, tflops=round(fl / us / 1e6, 2),
                     mfma_frac=round(fl / us / 1e6 / BF16_PEAK_TFLOPS, 4))
        elif name in ab:
            b = ab[name]
            e.update(bytes=b, gbs=round(b / us / 1e3, 1), hbm_frac=round(b / us / 1e3 / HBM_PEAK_GBS, 4))
        rep[name] = e
    q_us = kern["quantize_4bit"] + kern["double_quant"]
    b = ab["quantize_4bit+double_quant"]
    rep["quantize_4bit+double_quant"] = {"us": round(q_us, 3), "bytes": b, "gbs": round(b / q_us / 1e3, 1),
                                         "hbm_frac": round(b / q_us / 1e3 / HBM_PEAK_GBS, 4)}

    gemv_us = kern["gemv_4bit"]
    gemv_gbs = ab["gemv_4bit"] / gemv_us / 1e3
    traffic = measured_traffic()
    ceil = measured_ceilings(torch, dev)
    out = {
        "metric": METRIC,
        "value": round(gemv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "LLM MLP up-projection 14336x4096 bf16 (0.1% x20 outliers), NF4 block 64, "
                               "double-quantized scales (256-groups); gemv M=1, gemm M=512",
                   "N": N, "K": K, "quant_type": "nf4", "blocksize": BS, "blocksize2": BS2,
                   "gemv_M": M_GEMV, "gemm_M": M_GEMM, "parallelism": "single-gpu",
                   "rotating_weight_copies": n_p},
        "roofline": {"bound": "hbm", "achieved": round(gemv_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "gemv_4bit",
                     "algorithmic_bytes_per_launch": ab["gemv_4bit"], "avg_launch_us": round(gemv_us, 3),
                     "frac_of_measured_read": round(gemv_gbs / ceil["read_gbs"], 4)},
        "ceilings": ceil,
        "env": {"torch": torch.__version__, "hip": torch.version.hip,
                "device": torch.cuda.get_device_name(dev),
                "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count},
        "kernels": rep,
        "step_wall_ms": round(wall_step_ms, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W_cpu, x_cpu)
        out["cpu_baseline"]["host"] = host_info()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
