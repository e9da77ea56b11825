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

The "configs" table then times every workload of the parity suite the same
way: the fp32 1024x1024 and bf16 4096x4096 NF4 weights; W_up 14336x4096 and
W_down 4096x14336 (NF4 and FP4, double-quantized scales); gemm_4bit at M =
8 ... 2048 on the 14336x4096 prefill weight with gemv_4bit at M = 1 and 8 for
the crossover; the 8192x28672 and 28672x8192 layers (NF4 and FP4, block 128,
double-quantized scales) with gemv_4bit at M = 1, 2, 4, 8.  Each row gives
microseconds per launch, algorithmic bytes (and flops for gemm), the fraction
of the HBM peak and of the measured read (gemv) or copy (codec) ceiling.

Before anything is timed, untimed steps run for --warm-seconds (2 s) so that
the GPU clocks have ramped up.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--warm-seconds S] [--no-cpu-baseline] [--no-configs]
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


def cpu_baseline(W_cpu, x_cpu, A_cpu, budget_s=12.0, rows=256):
    """The oracle as it stands, timed on bounded samples of the headline
    workload (W_up 14336 x 4096 bf16, NF4, block 64, double-quantized scales):
      quantize_4bit of the first 2048 weight rows; double_quant of all
      917504 block scales; dequantize_4bit (to bf16) of the first 4096 rows;
      gemv (scale decode + dequantize + float64 matmul) over the first `rows`
      output rows, repeated for `budget_s`; gemm of the 512 activation rows
      against the first 1024 output rows.
    Elementwise numpy runs on one thread, the float64 matmuls on all BLAS
    threads.  Bytes and flops are counted per unit exactly as for the GPU
    kernels.  The headline value is the gemv's."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O
    W64 = W_cpu.to(torch.float64).numpy()
    x64 = x_cpu.to(torch.float64).numpy()
    A64 = A_cpu.to(torch.float64).numpy()
    blas = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    ops = {}
    with threadpool_limits(limits=1):
        absmax = O.block_absmax(W64, BS).astype(np.float32)      # untimed set-up
        q, a2, off = O.double_quant(absmax, BS2, forms="threshold")
        t0 = time.perf_counter()
        O.quantize_4bit(W64[:2048], BS, "nf4", forms="threshold")
        t = time.perf_counter() - t0
        ops["quantize_4bit"] = {"gbs": round(2048 * K * (2 + 0.5 + 4 / BS) / t / 1e9, 5), "s": round(t, 3),
                                "sample": "2048 rows x 4096 (threshold form of the nearest-code search)"}
        t0 = time.perf_counter()
        O.double_quant(absmax, BS2, forms="threshold")
        t = time.perf_counter() - t0
        ops["double_quant"] = {"gbs": round(absmax.size * (4 + 1 + 4 / BS2) / t / 1e9, 5), "s": round(t, 3),
                               "sample": f"{absmax.size} scales (threshold form)"}
        drows = 4096
        packed_d, _ = O.quantize_4bit(W64[:drows], BS, "nf4", forms="threshold")
        nbd = drows * K // BS
        ahat_d = O.dequant_absmax(q[:nbd], a2[:-(-nbd // BS2)], off, None, BS2)
        t0 = time.perf_counter()
        O.dequantize_4bit(packed_d, ahat_d, drows * K, BS, "nf4", "bf16")
        t = time.perf_counter() - t0
        ops["dequantize_4bit"] = {"gbs": round(drows * K * (0.5 + 2 + (1 + 4 / BS2) / BS) / t / 1e9, 5),
                                  "s": round(t, 3), "sample": f"{drows} rows x 4096"}
        packed, _ = O.quantize_4bit(W64[:rows], BS, "nf4", forms="threshold")
        nbs = rows * K // BS
        ahat = O.dequant_absmax(q[:nbs], a2[:-(-nbs // BS2)], off, None, BS2)
    with threadpool_limits(limits=1, user_api="openmp"), threadpool_limits(limits=blas, user_api="blas"):
        passes, t0 = 0, time.perf_counter()
        while True:
            ah = O.dequant_absmax(q[:nbs], a2[:-(-nbs // BS2)], off, None, BS2)
            O.matmul_4bit(x64, packed, ah, rows, K, BS, "nf4")
            passes += 1
            t_gemv = time.perf_counter() - t0
            if t_gemv >= budget_s:
                break
        per_row = K // 2 + K // BS * (1 + 4 / BS2) + 2 * M_GEMV      # packed + DQ scales + y
        gbs = passes * rows * per_row / t_gemv / 1e9
        ops["gemv_4bit"] = {"gbs": round(gbs, 5), "s": round(t_gemv, 3),
                            "sample": f"{rows} output rows, {passes} passes"}
        grows = 1024
        packed_g, _ = O.quantize_4bit(W64[:grows], BS, "nf4", forms="threshold")
        nbg = grows * K // BS
        ahat_g = O.dequant_absmax(q[:nbg], a2[:-(-nbg // BS2)], off, None, BS2)
        t0 = time.perf_counter()
        O.matmul_4bit(A64, packed_g, ahat_g, grows, K, BS, "nf4")
        t = time.perf_counter() - t0
        ops["gemm_4bit"] = {"gflops": round(2 * A64.shape[0] * grows * K / t / 1e9, 4), "s": round(t, 3),
                            "sample": f"{A64.shape[0]} x {grows} outputs, K = 4096"}
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": blas, "kind": "oracle",
            "sample": f"oracle gemv (DQ scale decode + dequantize + float64 matmul) over the first "
                      f"{rows} of {N} output rows, {passes} passes in {t_gemv:.1f} s; elementwise steps on one "
                      f"thread, matmuls on {blas} BLAS threads; bytes per row counted as for the GPU kernel",
            "ops": ops}


def _copies(t, n):
    """n copies of t in one allocation, as views, each starting on a 256-byte
    boundary (the entry points refuse operands that are not 16-byte aligned)."""
    flat = t.reshape(-1)
    k = flat.numel()
    per = 256 // flat.element_size()
    stride = -(-k // per) * per
    big = flat.new_empty(n * stride)
    views = [big[i * stride:i * stride + k] for i in range(n)]
    for v in views:
        v.copy_(flat)
    return views


def _auto_timed(fn, stream, torch, target_us=30000.0, lo=20, hi=600):
    """Average microseconds per call of fn(i): a short trial sizes the loop
    to about target_us of GPU time.  fn returns the entry point's status,
    checked on the warm-up calls."""
    for i in range(3):
        _ok(fn(i))
    trial = timed_loop(fn, 8, stream, torch)
    iters = int(min(hi, max(lo, target_us / max(trial, 1e-3))))
    return timed_loop(fn, iters, stream, torch), iters


def graph_interval(fn, stream, torch, nodes=230, reps=15):
    """Microseconds per launch of fn(0 .. nodes - 1) captured once into a HIP
    graph and replayed reps times back to back: the GPU's own interval
    between consecutive launches, free of the host's per-call cost."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(nodes):
            fn(i)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(2):
            g.replay()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(reps):
            g.replay()
        end.record(stream)
    end.synchronize()
    del g
    return start.elapsed_time(end) / (reps * nodes) * 1e3


def _ok(rc):
    if rc != 0:
        from quantized_matvec_amd import qmv
        raise RuntimeError(f"entry point failed: {rc} ({qmv._status_string(rc)})")


def config_rows(torch, dev, stream, ceil):
    """Every workload of the parity suite, timed on the device: for each
    weight and quant type, quantize (with double quantization where the
    workload has it), dequantize to the weight's dtype and gemv / gemm at the
    workload's row counts.  Each op rotates over distinct copies of its
    operands (> 512 MB per rotation, twice the Infinity Cache) so the bytes
    come from HBM, and is timed with HIP events on the launch stream."""
    from quantized_matvec_amd import qmv, synth
    L = qmv.lib()
    s_h = stream.cuda_stream
    rows = []
    code = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    qcode = {"nf4": 0, "fp4": 1}
    read, copy = ceil["read_gbs"], ceil["copy_gbs"]
    extra_m = {4: (1, 8), 5: (1, 2, 4, 8)}
    gemm_m = {4: (8, 32, 128, 512, 1024, 2048)}
    for cfg in (1, 2, 3, 4, 5):
        wl = synth.WORKLOADS[cfg]
        for which, (Nw, Kw) in enumerate(wl.weights):
            W0 = synth.weight(cfg, which).to(dev)
            numel, wb = Nw * Kw, W0.element_size()
            bs, dq = wl.blocksize, wl.double_quant
            nb = numel // bs
            st_bytes = (nb + 4 * (-(-nb // BS2)) + 4 + 4 * 256) if dq else 4 * nb
            n_w = max(2, -(-ROTATE_BYTES // (numel * wb)))
            n_p = max(2, -(-ROTATE_BYTES // (numel // 2)))
            Ws = _copies(W0, n_w)
            wout = _copies(torch.empty_like(W0), n_w)
            for qt in wl.quant_types:
                tag = {"cfg": f"c{cfg}", "weight": f"{Nw}x{Kw}", "w_dtype": wl.w_dtype, "quant_type": qt,
                       "blocksize": bs, "double_quant": dq}
                p0, st0 = qmv.quantize_4bit(W0, bs, qt, double_quant=dq, blocksize2=BS2)
                packs = _copies(p0, n_p)
                if dq:
                    parts = [_copies(t, n_p) for t in (st0.absmax_q, st0.absmax2, st0.offset, st0.code2)]
                    states = [qmv.QuantState(st0.shape, st0.dtype, bs, qt, None, *[p[i] for p in parts], BS2)
                              for i in range(n_p)]
                else:
                    states = [qmv.QuantState(st0.shape, st0.dtype, bs, qt, a)
                              for a in _copies(st0.absmax, n_p)]
                cs = [st._c() for st in states]
                refs = [ctypes.byref(c) for c in cs]
                pp = [p.data_ptr() for p in packs]

                def add(op, us, iters, nbytes, ceiling, m=None, flops=None):
                    r = dict(tag, op=op, us=round(us, 3), launches_timed=iters, bytes=nbytes,
                             gbs=round(nbytes / us / 1e3, 1), hbm_frac=round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4))
                    if m is not None:
                        r["M"] = m
                    if ceiling:
                        r["ceiling"] = ceiling
                        r["ceiling_frac"] = round(nbytes / us / 1e3 / (read if ceiling == "read" else copy), 4)
                    if flops is not None:
                        r.update(flops=flops, tflops=round(flops / us / 1e6, 2),
                                 mfma_frac=round(flops / us / 1e6 / BF16_PEAK_TFLOPS, 4))
                    rows.append(r)

                # quantize (+ double quantization) into rotating outputs
                qb = _copies(torch.empty_like(p0), n_w)
                ab = _copies(torch.empty(nb, dtype=torch.float32, device=dev), n_w)
                if dq:
                    dqo = [_copies(t, n_w) for t in (torch.empty_like(st0.absmax_q), torch.empty_like(st0.absmax2),
                                                     torch.empty_like(st0.offset), torch.empty_like(st0.code2))]
                    ws = torch.zeros(max(16, L.qmv_double_quant_workspace(nb, BS2)), dtype=torch.uint8, device=dev)

                def run_q(i):
                    j = i % n_w
                    rc = L.qmv_quantize_4bit(Ws[j].data_ptr(), code[W0.dtype], numel, bs, qcode[qt],
                                             qb[j].data_ptr(), ab[j].data_ptr(), s_h)
                    if dq and rc == 0:
                        rc = L.qmv_double_quant(ab[j].data_ptr(), nb, BS2, None, dqo[0][j].data_ptr(),
                                                dqo[1][j].data_ptr(), dqo[2][j].data_ptr(), dqo[3][j].data_ptr(),
                                                ws.data_ptr(), ws.numel(), s_h)
                    return rc

                us, it = _auto_timed(run_q, stream, torch)
                add("quantize_4bit+double_quant" if dq else "quantize_4bit", us, it,
                    wb * numel + numel // 2 + st_bytes, "copy")

                def run_d(i):
                    return L.qmv_dequantize_4bit(pp[i % n_p], refs[i % n_p], numel, bs, qcode[qt],
                                          wout[i % n_w].data_ptr(), code[W0.dtype], s_h)

                us, it = _auto_timed(run_d, stream, torch)
                add("dequantize_4bit", us, it, numel // 2 + st_bytes + wb * numel, "copy")

                xfull = synth.activations(cfg, which).to(dev)
                xdt = xfull.dtype
                for m in extra_m.get(cfg, wl.ms):
                    x = xfull[:m].contiguous()
                    y = torch.empty(m, Nw, dtype=xdt, device=dev)

                    def run_v(i, x=x, y=y, m=m):
                        return L.qmv_gemv_4bit(x.data_ptr(), code[xdt], m, Nw, Kw, pp[i % n_p], refs[i % n_p], bs,
                                        qcode[qt], y.data_ptr(), code[xdt], None, s_h)

                    us, it = _auto_timed(run_v, stream, torch)
                    add("gemv_4bit", us, it, numel // 2 + st_bytes + x.element_size() * m * (Kw + Nw), "read", m=m)
                for m in gemm_m.get(cfg, ()):
                    A = (xfull[:m] if m <= xfull.shape[0] else
                         synth.gaussian((m, Kw), 1.0, 100 * cfg + 7, wl.x_dtype)).contiguous().to(dev)
                    C = torch.empty(m, Nw, dtype=xdt, device=dev)

                    def run_g(i, A=A, C=C, m=m):
                        return L.qmv_gemm_4bit(A.data_ptr(), code[xdt], m, Nw, Kw, pp[i % n_p], refs[i % n_p], bs,
                                        qcode[qt], C.data_ptr(), code[xdt], None, s_h)

                    us, it = _auto_timed(run_g, stream, torch, hi=200)
                    add("gemm_4bit", us, it, numel // 2 + st_bytes + A.element_size() * m * (Kw + Nw), None,
                        m=m, flops=2.0 * m * Nw * Kw)
                    del A, C
                torch.cuda.synchronize()
                print(f"[bench] c{cfg} {Nw}x{Kw} {qt} timed", file=sys.stderr, flush=True)
                del packs, states, cs, refs, qb, ab
            del Ws, wout, W0
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    return rows


COPY_BYTES = 1 << 30


def measured_ceilings(torch, dev, reps=20):
    """Streaming ceilings of this GPU, to read the kernels' GB/s against: a
    plain 128-bit read of 1 GiB (the library's stream_read probe), torch's
    fill of 1 GiB (write only) and torch's device copy of 1 GiB (bytes read +
    written).  Event-timed on torch's current stream, the probe's launch
    stream, after two warm-up passes."""
    from quantized_matvec_amd import qmv
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(8192, dtype=torch.int32, device=dev)
    out = {}
    for name, fn, nbytes in (("read_gbs", lambda: qmv.stream_read(src, sink), COPY_BYTES),
                             ("write_gbs", lambda: dst.fill_(1.0), COPY_BYTES),
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
    out["method"] = ("stream_read probe over 1 GiB (128-bit loads, grid-stride, one sink word per "
                     "workgroup), torch fill_ of 1 GiB (written bytes) and torch copy_ of 1 GiB (bytes "
                     "read + written), event-timed")
    return out


def clocks():
    """Current GPU clocks as the driver reports them (best effort)."""
    import glob
    import subprocess
    out = {}
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))[:1] + \
            sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_mclk"))[:1]:
        try:
            with open(path) as f:
                cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
            out[os.path.basename(path)] = cur[0] if cur else None
        except OSError:
            pass
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        lines = [ln.strip() for ln in r.stdout.splitlines() if "clock level" in ln.lower() or "Mhz" in ln]
        if lines:
            out["rocm_smi"] = lines[:8]
    except Exception:  # noqa: BLE001 - informational only
        pass
    return out or None


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
    ap.add_argument("--warm-seconds", type=float, default=2.0,
                    help="untimed steps for this long first, so the GPU clocks have ramped up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload table (every weight, quant type and row count)")
    ap.add_argument("--counters", choices=["gemv_4bit", "gemm_4bit", "gemm_4bit_backward", "dequantize_4bit",
                                           "quantize_4bit", "double_quant"],
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
        _, st0_plain = qmv.quantize_4bit(W, BS, "nf4")
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
            dY0 = synth.gaussian((M_GEMM, N), 1.0, 100 * 4 + 3, "bf16").to(dev)
            dX0 = torch.empty(M_GEMM, K, dtype=torch.bfloat16, device=dev)
            counters_run(args.counters, dict(gemv_4bit=lambda i: qmv.gemv_4bit(x, packs[i], states[i], out=y),
                                             gemm_4bit=lambda i: qmv.gemm_4bit(A, packs[i], states[i], out=C),
                                             gemm_4bit_backward=lambda i: qmv.gemm_4bit_backward(
                                                 dY0, packs[i], states[i], out=dX0),
                                             double_quant=lambda i: qmv.double_quant(st0_plain.absmax),
                                             dequantize_4bit=lambda i: qmv.dequantize_4bit(
                                                 packs[i], states[i], out=wout[i % n_w]),
                                             quantize_4bit=lambda i: qmv.quantize_4bit(
                                                 Ws[i % n_w], BS, "nf4")), n_p, dev, torch)
            return

        # the clocks ramp up under load over the first second or so (the same
        # kernel measured 15 % slower at the start of a run than after it):
        # run untimed steps for --warm-seconds, then the W warm-up steps
        tw = time.perf_counter()
        i = 0
        while time.perf_counter() - tw < args.warm_seconds:
            step(i)
            i += 1
            if i % 20 == 0:
                torch.cuda.synchronize()
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        us_step = timed_loop(step, args.steps, stream, torch)
        torch.cuda.synchronize()
        wall_step_ms = (time.perf_counter() - t0) * 1e3 / args.steps

        kern, kern_iters = {}, {}
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
            return L.qmv_gemv_4bit(x_ptr, 2, M_GEMV, N, K, p_ptr[i % n_p], scs[i % n_p], BS, 0, y_ptr, 2, None,
                                   s_h)

        def run_gemm(i):
            return L.qmv_gemm_4bit(A_ptr, 2, M_GEMM, N, K, p_ptr[i % n_p], scs[i % n_p], BS, 0, C_ptr, 2, None,
                                   s_h)

        def run_deq(i):
            return L.qmv_dequantize_4bit(p_ptr[i % n_p], scs[i % n_p], N * K, BS, 0, w_ptr[i % n_w], 2, s_h)

        qbuf = [torch.empty_like(packed0) for _ in range(n_w)]
        abuf = [torch.empty_like(st0.absmax_q, dtype=torch.float32) for _ in range(n_w)]

        def run_quant(i):      # the raw entry point (no allocation inside the loop)
            return L.qmv_quantize_4bit(Ws[i % n_w].data_ptr(), 2, N * K, BS, 0, qbuf[i % n_w].data_ptr(),
                                       abuf[i % n_w].data_ptr(), s_h)

        dq_out = [(torch.empty_like(st0.absmax_q), torch.empty_like(st0.absmax2),
                   torch.empty_like(st0.offset), torch.empty_like(st0.code2)) for _ in range(n_w)]
        nbk = N * K // BS
        ws = torch.zeros(L.qmv_double_quant_workspace(nbk, 256), dtype=torch.uint8, device=dev)

        def run_dq(i):
            q, a2, off, c2 = dq_out[i % n_w]
            return L.qmv_double_quant(abuf[i % n_w].data_ptr(), nbk, BS2, None, q.data_ptr(), a2.data_ptr(),
                                      off.data_ptr(), c2.data_ptr(), ws.data_ptr(), ws.numel(), s_h)

        # gemm_4bit_backward (dX = dY @ W_hat) on the same weight, dY [512, 14336]
        dY = synth.gaussian((M_GEMM, N), 1.0, 100 * 4 + 3, "bf16").to(dev)
        dX = torch.empty(M_GEMM, K, dtype=torch.bfloat16, device=dev)
        dY_ptr, dX_ptr = dY.data_ptr(), dX.data_ptr()
        bws_n = L.qmv_gemm_4bit_backward_workspace(M_GEMM, N, K, BS)
        bws = torch.empty(max(bws_n, 256), dtype=torch.uint8, device=dev)

        def run_bwd(i):
            return L.qmv_gemm_4bit_backward(dY_ptr, 2, M_GEMM, N, K, p_ptr[i % n_p], scs[i % n_p], BS, 0,
                                            dX_ptr, 2, bws.data_ptr(), bws.numel(), s_h)

        # the 8-bit blockwise codec on the same bf16 weights (blocksize 4096),
        # with the default linear table and with the dynamic-tree table
        q8 = [torch.empty(N * K, dtype=torch.uint8, device=dev) for _ in range(n_w)]
        a8 = [torch.empty(N * K // BS8, dtype=torch.float32, device=dev) for _ in range(n_w)]
        tree = (ctypes.c_float * 256)(*qmv.dynamic_tree_code())
        tree_p = ctypes.cast(tree, ctypes.c_void_p)

        def run_q8(i, code=None):
            return L.qmv_quantize_blockwise(Ws[i % n_w].data_ptr(), 2, N * K, BS8, code, q8[i % n_w].data_ptr(),
                                            a8[i % n_w].data_ptr(), s_h)

        def run_dq8(i):
            return L.qmv_dequantize_blockwise(q8[i % n_w].data_ptr(), a8[i % n_w].data_ptr(), N * K, BS8, None,
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
            return L.qmv_embedding_4bit(eidx.data_ptr(), EMB_T, EMB_V, K, pe.data_ptr(), ctypes.byref(ec), BS, 0,
                                        eout.data_ptr(), 2, s_h)

        # context for the gemv's figure: a plain 128-bit read of each rotating
        # copy's packed bytes (the same size, launched the same way), and the
        # interval of back-to-back launches that do almost nothing (one
        # workgroup reading 16 bytes), replayed from a HIP graph so that the
        # host's cost per call (about 3.5 us through ctypes) does not set it
        rsink = torch.zeros(8192, dtype=torch.int32, device=dev)
        pk_bytes = N * K // 2

        def run_read_same(i):
            return L.qmv_stream_read(p_ptr[i % n_p], pk_bytes, rsink.data_ptr(), s_h)

        def run_floor(i):
            return L.qmv_stream_read(p_ptr[0], 16, rsink.data_ptr(), s_h)

        _ok(run_floor(0))
        floor_graph_us = graph_interval(run_floor, stream, torch)
        gemv_graph_us = graph_interval(run_gemv, stream, torch)

        # each loop runs about 30 ms of launches (a short loop right after a
        # memory-bound one reads a compute-bound kernel up to 15 % slow)
        for name, fn in (("gemv_4bit", run_gemv), ("read_same_bytes", run_read_same), ("gemm_4bit", run_gemm), ("gemm_4bit_backward", run_bwd),
                         ("dequantize_4bit", run_deq), ("quantize_4bit", run_quant), ("double_quant", run_dq),
                         ("quantize_blockwise", run_q8), ("quantize_blockwise_dynamic", lambda i: run_q8(i, tree_p)),
                         ("dequantize_blockwise", run_dq8), ("embedding_4bit", run_emb)):
            us, it = _auto_timed(fn, stream, torch, hi=4000)
            kern[name] = us
            kern_iters[name] = it

    read_same_us = kern.pop("read_same_bytes")
    rep = {}
    for name, us in kern.items():
        e = {"us_per_launch": round(us, 3), "launches_timed": kern_iters[name]}
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
                     "frac_of_measured_read": round(gemv_gbs / ceil["read_gbs"], 4),
                     # the gemv's rate against a plain read of the same packed
                     # weight (29.4 MB per launch, same rotation and loop); the
                     # gemv's interval when its launches are replayed from a HIP
                     # graph; the interval below which no launch goes
                     "same_size_read_us": round(read_same_us, 3),
                     "frac_of_same_size_read": round(gemv_gbs / (N * K // 2 / read_same_us / 1e3), 4),
                     "graph_replay_us": round(gemv_graph_us, 3),
                     "launch_interval_floor_us": round(floor_graph_us, 3),
                     "note": "avg_launch_us is the interval between back-to-back launches (HIP events around "
                             "the whole loop); a rocprofv3 kernel trace reports the kernel's own duration, "
                             "shorter by the dispatch gap between consecutive kernels"},
        "ceilings": ceil,
        "env": {"torch": torch.__version__, "hip": torch.version.hip,
                "device": torch.cuda.get_device_name(dev),
                "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count},
        "kernels": rep,
        "step_wall_ms": round(wall_step_ms, 4),
        "clocks": clocks(),
    }
    if not args.no_configs:
        with torch.cuda.stream(stream):
            out["configs"] = config_rows(torch, dev, stream, ceil)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W_cpu, x_cpu, A_cpu)
        out["cpu_baseline"]["host"] = host_info()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
