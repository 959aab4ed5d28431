#!/usr/bin/env python3
"""Causal attention fwd+bwd throughput on one MI355X, with roofline and CPU-oracle baseline.

A step is one fa_forward + fa_backward over the workload's seeded inputs, which are resident
in HBM before the timed region starts. Counted work (the metric's convention): forward
4*B*H*N^2*d FLOPs, halved when causal; backward 2.5x forward.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-configs]

One JSON line. The run first measures every workload (`configs`, the headline's workload
last): fa_forward, fa_backward and both back to back, each timed with HIP events over 100 repetitions (20 for the 16384-row
workload) with a 512 MiB write before every repetition to flush L2 and the MALL (median,
p10, p90), plus one warm-cache figure; then the headline: W untimed steps and K timed steps
of the headline workload, back to back. The per-config block takes several seconds of GPU
work, so the headline runs at the clock the GPU holds under sustained load. Extra modes:
    --copy-calibration   run only a plain device copy of known size (HBM counter scaling)
    --sweep              forward / backward / end-to-end latency of these kernels against
                         plain PyTorch attention over sequence length x head dim x dtype
                         (a markdown table on stdout, no JSON line)
    --e2e                training steps of a toy decoder with plain attention, then with the
                         flash kernels monkey-patched in as its attention (two JSON lines)
    --atomic-dq          the backward with dQ from fp32 atomics against the deterministic
                         two-pass split, on --workload (one JSON line)
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

PUBLISHED_PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, as published
PEAK_HBM_GBPS = 8000.0
MFMA_BF16_FLOP_PER_CLK_PER_CU = 4096  # 4 SIMDs x one 32x32x16 MFMA (32768 FLOP) per 32 clk
DEFAULT_WORKLOAD = "b8_n4096_d64"
KERNEL_SOURCES = ["tiled_attention_causal_amd/csrc/fa_bf16.hip",
                  "tiled_attention_causal_amd/csrc/fa_common.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload flushed-cache block")
    ap.add_argument("--config-reps", type=int, default=100,
                    help="repetitions per measurement in the per-workload block (a fifth "
                         "of that for the 16384-row workload)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="run the oracle sample for at least this much CPU time")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--e2e", action="store_true",
                    help="training-step time of a toy decoder, plain vs flash attention")
    ap.add_argument("--atomic-dq", action="store_true",
                    help="backward time with dQ from fp32 atomics against the two-pass split")
    ap.add_argument("--sweep-n", default="128,256,512,1024,2048,4096,8192")
    ap.add_argument("--sweep-d", default="16,32,64,128")
    ap.add_argument("--sweep-dtypes", default="bf16,f32")
    ap.add_argument("--sweep-batch", type=int, default=1)
    ap.add_argument("--sweep-reps", type=int, default=20)
    ap.add_argument("--sweep-flash-only", action="store_true",
                    help="time only the flash kernels (e.g. past plain attention's memory)")
    ap.add_argument("--sweep-plain-only", action="store_true",
                    help="time only plain attention (e.g. to find where it runs out of memory)")
    return ap.parse_args()


def source_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_names(w, fwd_ws_bytes=0, bwd_ws_bytes=0):
    """(forward, backward) names of the attention kernels the library launches for workload
    `w` with these workspace sizes, from the library's own dispatch."""
    from seeded_inputs import torch_dtype
    from tiled_attention_causal_amd import kernel_names as lib_names
    return lib_names(torch_dtype(w.dtype), w.B, w.H, w.Nq, w.Nk, w.d, w.causal, fwd_ws_bytes,
                     bwd_ws_bytes)


def _loaded_hip_runtime():
    """The HIP runtime library this process already uses (so no second copy is loaded)."""
    import ctypes
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1]
            if "libamdhip64.so" in os.path.basename(path):
                return ctypes.CDLL(path)
    return ctypes.CDLL("libamdhip64.so")


def device_peak(dev_index=0):
    """bf16 dense MFMA peak of the device: compute units x peak engine clock x 4096 FLOP per
    clock per CU, from hipDeviceGetAttribute (hipDeviceAttributeMultiprocessorCount = 63,
    hipDeviceAttributeClockRate = 5, in kHz)."""
    import ctypes
    hip = _loaded_hip_runtime()
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    if (hip.hipDeviceGetAttribute(ctypes.byref(cus), 63, dev_index) != 0
            or hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, dev_index) != 0):
        raise RuntimeError("hipDeviceGetAttribute failed")
    tflops = cus.value * khz.value * 1e3 * MFMA_BF16_FLOP_PER_CLK_PER_CU / 1e12
    return {"bf16_tflops": round(tflops, 1), "compute_units": cus.value,
            "peak_clock_mhz": khz.value / 1000.0,
            "formula": f"{cus.value} CUs x {khz.value / 1000.0:g} MHz x "
                       f"{MFMA_BF16_FLOP_PER_CLK_PER_CU} FLOP/clk/CU",
            "published_bf16_tflops": PUBLISHED_PEAK_BF16_TFLOPS}


def read_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None
    when the summary is missing or was taken on a different kernel source."""
    stem = kernel.split("<")[0]
    path = os.path.join(ROOT, "profiles", f"{stem}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Workspace:
    """Device tensors and pre-marshalled C-ABI calls for one workload: forward (fa_forward,
    or fa_forward_with_workspace where the workload can use a workspace), the backward as
    fa_backward, and its two steps fa_backward_preprocess and fa_backward_main. Calls go
    straight through ctypes, so the host enqueues a launch in a few microseconds."""

    def __init__(self, w):
        import torch
        from seeded_inputs import workload_inputs
        from tiled_attention_causal_amd import (_lib, backward_workspace_bytes,
                                                forward_workspace_bytes)
        self.w = w
        dev = torch.device("cuda:0")
        inp = workload_inputs(w)
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        self.fws_bytes = forward_workspace_bytes(q, k, w.causal)
        self.bws_bytes = backward_workspace_bytes(q, k)
        fws = torch.empty(max(1, self.fws_bytes), dtype=torch.uint8, device=dev)
        bws = torch.empty(max(1, self.bws_bytes), dtype=torch.uint8, device=dev)
        self.tensors = (q, k, v, do, o, lse, dq, dk, dv, fws, bws)  # kept alive
        self.stream = torch.cuda.current_stream(dev)
        lib = _lib.load()
        self.ok = _lib.FA_SUCCESS
        self.err = _lib.FAError
        dt = _lib.FA_DTYPE_BF16 if w.dtype == "bf16" else _lib.FA_DTYPE_F32
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
        sp = self.stream.cuda_stream
        causal = int(bool(w.causal))
        fa = (dt, B, H, Nq, Nk, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), causal, w.scale,
              o.data_ptr(), lse.data_ptr())
        if self.fws_bytes:
            self.fwd = (lib.fa_forward_with_workspace, fa + (fws.data_ptr(), self.fws_bytes, sp))
        else:
            self.fwd = (lib.fa_forward, fa + (sp,))
        bw = (dt, B, H, Nq, Nk, d, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
              lse.data_ptr(), do.data_ptr(), causal, w.scale, dq.data_ptr(), dk.data_ptr(),
              dv.data_ptr(), bws.data_ptr(), self.bws_bytes, sp)
        self.bwd = (lib.fa_backward, bw)
        self.prep = (lib.fa_backward_preprocess,
                     (dt, B, H, Nq, d, o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                      bws.data_ptr(), self.bws_bytes, sp))
        self.main = (lib.fa_backward_main, bw)

    def call(self, which):
        fn, a = which
        st = fn(*a)
        if st != self.ok:
            raise self.err(st, fn.__name__)

    def step(self):
        self.call(self.fwd)
        self.call(self.bwd)


def _pct(ts, p):
    import numpy as np
    return float(np.percentile(np.asarray(ts), p))


def config_block(ws, reps, flush):
    """Flushed-cache medians (p10, p90) of fa_forward, fa_backward and both, over `reps`
    repetitions after 10 warm-up steps, each repetition preceded by a 512 MiB write that
    evicts L2 and the MALL (as triton.testing.do_bench clears the cache), plus the warm
    figure: the mean step of 5 chunks of 20 back-to-back steps, median chunk."""
    import torch
    w = ws.w
    fl = w.counted_flops()
    for _ in range(10):
        ws.step()
    torch.cuda.synchronize()
    out = {"workload": w.name, "reps": reps,
           "kernels": dict(zip(("fwd", "bwd"), kernel_names(w, ws.fws_bytes, ws.bws_bytes)))}
    runs = {"fwd": (lambda: ws.call(ws.fwd), fl["fwd"]),
            "bwd": (lambda: ws.call(ws.bwd), fl["bwd"]),
            "fwd_bwd": (ws.step, fl["total"])}
    for name, (fn, flops) in runs.items():
        ev = []
        for _ in range(reps):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(ws.stream)
            fn()
            e1.record(ws.stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) for a, b in ev]
        med = _pct(ts, 50)
        out[name] = {"median_ms": round(med, 5), "p10_ms": round(_pct(ts, 10), 5),
                     "p90_ms": round(_pct(ts, 90), 5),
                     "tflops": round(flops / (med * 1e-3) / 1e12, 2)}
    chunks = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(ws.stream)
        for _ in range(20):
            ws.step()
        e1.record(ws.stream)
        chunks.append((e0, e1))
    torch.cuda.synchronize()
    warm = sorted(a.elapsed_time(b) / 20 for a, b in chunks)[2]
    out["warm_fwd_bwd"] = {"ms": round(warm, 5),
                           "tflops": round(fl["total"] / (warm * 1e-3) / 1e12, 2),
                           "label": "warm cache: back-to-back steps, no flush"}
    return out


def time_workload(ws, steps, warmup):
    """The headline: `warmup` untimed steps, then exactly `steps` steps between two
    synchronisations (wall clock), then per-launch HIP-event durations of the step's three
    launches for the roofline."""
    import torch
    w = ws.w
    for _ in range(warmup):
        ws.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ws.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Per-launch durations with HIP events on the stream the kernels run on. Each of the
    # step's three launches (fa_forward, then fa_backward as its two steps
    # fa_backward_preprocess and fa_backward_main, exactly what fa_backward enqueues) is
    # repeated back to back between two events, in chunks of CHUNK launches, until `steps`
    # launches of each are timed; a chunk's elapsed time over CHUNK is the kernel's average
    # launch duration, so the events time the GPU, not the host's launch rate.
    launches = [ws.fwd, ws.prep, ws.main]
    CHUNK = 20
    nchunks = max(1, steps // CHUNK)
    per = [[] for _ in launches]
    for _ in range(nchunks):
        for i, which in enumerate(launches):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(ws.stream)
            for _ in range(CHUNK):
                ws.call(which)
            e1.record(ws.stream)
            per[i].append((e0, e1))
    torch.cuda.synchronize()

    def stat(i):
        t = sorted(a.elapsed_time(b) / CHUNK for a, b in per[i])
        return sum(t) / len(t), t[len(t) // 2]

    (fwd_mean, fwd_med), (prep_mean, prep_med), (main_mean, main_med) = (
        stat(0), stat(1), stat(2))
    names = kernel_names(w, ws.fws_bytes, ws.bws_bytes)
    return {
        "ms_per_step": wall * 1e3 / steps,
        "fwd_ms_mean": fwd_mean,
        "bwd_ms_mean": prep_mean + main_mean,
        "prep_ms_mean": prep_mean,
        "bwd_main_ms_mean": main_mean,
        "fwd_ms_median": fwd_med,
        "bwd_ms_median": prep_med + main_med,
        "kernels": names,
    }


def cpu_baseline(w, min_s, budget_s):
    """The fp64 oracle on whole heads of the same workload for about `min_s` seconds."""
    import numpy as np

    import oracle
    from seeded_inputs import to_f64, workload_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    inp = workload_inputs(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    # Whole heads in order, wrapping round, until at least `min_s` and at most `budget_s`
    # seconds of oracle work are done (a head is never cut short).
    while True:
        b, h = heads[done % len(heads)]
        a = [to_f64(inp[n][b, h]) for n in ("q", "k", "v", "do")]
        oracle.head_forward(a[0], a[1], a[2], w.causal, w.scale)
        oracle.head_backward(a[0], a[1], a[2], a[3], w.causal, w.scale)
        done += 1
        el = time.perf_counter() - t0
        per_head = el / done
        if el >= min_s or el + per_head > budget_s:
            break
    flops = w.counted_flops()["total"] * done / len(heads)
    del np
    # `cores`: the threads the oracle's work actually ran on (its BLAS pool; its elementwise
    # steps run on one of them). The host's cores available to this process are given apart.
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "blas_threads": int(threads), "host_cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{done} head passes over the {len(heads)} heads of the workload (one "
                      f"head: B=1,H=1,N={w.Nq},d={w.d}), fp64 forward + backward, {el:.1f} s; "
                      f"counted FLOPs as on the GPU"}


def plain_attention_forward(q, k, v, causal, scale, mask):
    """Attention as separate PyTorch operations, the baseline of "Systems and Parallelism"
    (CS336 field map, A2), problem pytorch_attention: S = Q K^T * scale, causal mask,
    softmax over the keys, O = P V. The N x N matrix P is kept for the backward."""
    import torch
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * scale
    if causal:
        s.masked_fill_(mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    del s
    return torch.matmul(p, v), p


def plain_attention_backward(q, k, v, p, do, scale):
    """Gradients of plain_attention_forward's graph, written out as autograd forms them
    (softmax backward dS = P (dP - rowsum(dP P))), with every transposed operand made
    contiguous before its batched product."""
    import torch
    dv = torch.matmul(p.transpose(-1, -2).contiguous(), do)
    dp = torch.matmul(do, v.transpose(-1, -2).contiguous())
    ds = p * (dp - (dp * p).sum(-1, keepdim=True))
    del dp
    dq = torch.matmul(ds, k) * scale
    dk = torch.matmul(ds.transpose(-1, -2).contiguous(), q) * scale
    return dq, dk, dv


def bench_ms(fn, reps, flush):
    """Median event time of fn() over `reps` runs after three warm-up runs, with the caches
    flushed (a 512 MiB fill) before every run, as triton.testing.do_bench does."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        flush.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    return times[len(times) // 2]


def sweep(args):
    """The flash_benchmarking comparison: these kernels against plain PyTorch attention,
    causal, batch `--sweep-batch`, one head, over sequence length x head dim x dtype.
    Latencies are medians in ms; plain attention that runs out of memory is reported as
    OOM, with its memory in use before the backward where it ran."""
    import torch
    from seeded_inputs import make_inputs
    from tiled_attention_causal_amd import backward_workspace_bytes, fa_backward, fa_forward

    dev = torch.device("cuda:0")
    flush = torch.empty(512 << 20, dtype=torch.int8, device=dev)
    B = args.sweep_batch
    ns = [int(x) for x in args.sweep_n.split(",")]
    ds = [int(x) for x in args.sweep_d.split(",")]
    print(f"| dtype | N | d | flash fwd | flash bwd | flash fwd+bwd | plain fwd | plain bwd "
          f"| plain fwd+bwd | fwd+bwd speed-up | plain memory before bwd |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for dtype in args.sweep_dtypes.split(","):
        for n in ns:
            mask = None
            for d in ds:
                inp = make_inputs(B, 1, n, n, d, dtype, index=7000 + n + d)
                q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
                scale = 1.0 / d ** 0.5
                row = [dtype, str(n), str(d)]
                fa = ["-"] * 3
                if not args.sweep_plain_only:
                    o, lse = fa_forward(q, k, v, True, scale)
                    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
                    ws = torch.empty(max(1, backward_workspace_bytes(q, k)), dtype=torch.uint8,
                                     device=dev)

                    def fa_fwd():
                        fa_forward(q, k, v, True, scale, out=o, lse=lse)

                    def fa_bwd():
                        fa_backward(q, k, v, o, lse, do, True, scale, dq=dq, dk=dk, dv=dv,
                                    workspace=ws)

                    def fa_e2e():
                        fa_fwd()
                        fa_bwd()

                    fa = [bench_ms(f, args.sweep_reps, flush) for f in (fa_fwd, fa_bwd, fa_e2e)]
                    del o, lse, dq, dk, dv, ws
                pl = ["-"] * 3
                mem = "-"
                if not args.sweep_flash_only:
                    try:
                        if mask is None:
                            mask = torch.ones(n, n, dtype=torch.bool, device=dev).triu_(1)
                        state = {}

                        def pl_fwd():
                            state["o"], state["p"] = plain_attention_forward(q, k, v, True,
                                                                             scale, mask)

                        def pl_bwd():
                            plain_attention_backward(q, k, v, state["p"], do, scale)

                        def pl_e2e():
                            pl_fwd()
                            pl_bwd()

                        pl_fwd()
                        torch.cuda.synchronize()
                        mem = f"{(torch.cuda.memory_allocated() - flush.numel()) / 2**20:.0f} MiB"
                        pl = [bench_ms(f, args.sweep_reps, flush)
                              for f in (pl_fwd, pl_bwd, pl_e2e)]
                        state.clear()
                    except torch.cuda.OutOfMemoryError:
                        state.clear()
                        pl = ["OOM"] * 3
                        torch.cuda.empty_cache()
                fmt = [f"{x:.4f}" if isinstance(x, float) else x for x in fa + pl]
                spd = (f"{pl[2] / fa[2]:.1f}x" if isinstance(pl[2], float)
                       and isinstance(fa[2], float) else "-")
                print("| " + " | ".join(row + fmt + [spd, mem]) + " |", flush=True)
                del q, k, v, do
            del mask
            torch.cuda.empty_cache()


class PlainAttention:
    """Plain attention as an autograd function (forward and backward of plain_attention_*),
    so that a model using it never has autograd form a batched product on a transposed
    view."""

    @staticmethod
    def apply(q, k, v, scale):
        import torch

        class _F(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v):
                n = q.shape[-2]
                masked = torch.ones(n, n, dtype=torch.bool, device=q.device).triu_(1)
                o, p = plain_attention_forward(q, k, v, True, scale, masked)
                ctx.save_for_backward(q, k, v, p)
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, p = ctx.saved_tensors
                return plain_attention_backward(q, k, v, p, do.contiguous(), scale)

        return _F.apply(q.contiguous(), k.contiguous(), v.contiguous())


def scaled_dot_product_attention(q, k, v, mask=None, is_causal=False, scale=None):
    """The toy model's attention function (module level, so it can be monkey-patched):
    plain attention under a causal keep-mask."""
    if mask is None and not is_causal:
        raise NotImplementedError("the toy model is causal")
    return PlainAttention.apply(q, k, v, scale if scale is not None else q.shape[-1] ** -0.5)


def toy_model(d_model, n_heads, d_ff, n_layers, dtype, device, seed=0):
    """A small pre-norm decoder stack (RMSNorm, causal multi-head attention, SwiGLU MLP) with
    random weights, calling this module's scaled_dot_product_attention for attention."""
    import torch

    g = torch.Generator().manual_seed(seed)

    def w(*shape):
        return (torch.randn(*shape, generator=g) * shape[-1] ** -0.5).to(device, dtype)

    class Block(torch.nn.Module):
        def __init__(self):
            super().__init__()
            self.wqkv = torch.nn.Parameter(w(3 * d_model, d_model))
            self.wo = torch.nn.Parameter(w(d_model, d_model))
            self.w1 = torch.nn.Parameter(w(d_ff, d_model))
            self.w3 = torch.nn.Parameter(w(d_ff, d_model))
            self.w2 = torch.nn.Parameter(w(d_model, d_ff))
            self.g1 = torch.nn.Parameter(torch.ones(d_model, device=device, dtype=dtype))
            self.g2 = torch.nn.Parameter(torch.ones(d_model, device=device, dtype=dtype))

        @staticmethod
        def rms(x, gain):
            xf = x.float()
            return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + 1e-5)).to(x.dtype) * gain

        def forward(self, x):
            B, N, _ = x.shape
            h = self.rms(x, self.g1).reshape(B * N, d_model)
            qkv = (h @ self.wqkv.t()).view(B, N, 3, n_heads, d_model // n_heads)
            q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
            keep = torch.ones(N, N, dtype=torch.bool, device=x.device).tril_()
            a = sys.modules[__name__].scaled_dot_product_attention(q, k, v, keep)
            a = a.transpose(1, 2).reshape(B * N, d_model)
            x = x + (a @ self.wo.t()).view(B, N, d_model)
            h = self.rms(x, self.g2).reshape(B * N, d_model)
            f = torch.nn.functional.silu(h @ self.w1.t()) * (h @ self.w3.t())
            return x + (f @ self.w2.t()).view(B, N, d_model)

    return torch.nn.Sequential(*[Block() for _ in range(n_layers)])


def atomic_dq(args):
    """The two dQ strategies of "Systems and Parallelism" (CS336 field map, A2), section
    1.3.3, on one workload: fa_backward (two-pass split, deterministic) and
    fa_backward_atomic (dQ from fp32 atomic additions), each launched back to back between
    HIP events after a warm-up, the median of five chunks of `steps // 5` launches."""
    import torch
    from seeded_inputs import WORKLOADS, workload_inputs
    from tiled_attention_causal_amd import (backward_atomic_workspace_bytes,
                                            backward_workspace_bytes, fa_backward,
                                            fa_backward_atomic, fa_forward)
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    inp = workload_inputs(w)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa_forward(q, k, v, w.causal, w.scale)
    ws = torch.empty(max(backward_workspace_bytes(q, k), backward_atomic_workspace_bytes(q, k)),
                     dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    runs = {
        "two_pass": lambda: fa_backward(q, k, v, o, lse, do, w.causal, w.scale, dq=dq, dk=dk,
                                        dv=dv, workspace=ws),
        "atomic": lambda: fa_backward_atomic(q, k, v, o, lse, do, w.causal, w.scale, dq=dq,
                                             dk=dk, dv=dv, workspace=ws),
    }
    for _ in range(max(1, args.warmup // 4)):
        for fn in runs.values():
            fn()
    torch.cuda.synchronize(dev)
    chunk = max(1, args.steps // 5)
    out = {}
    for name, fn in runs.items():
        t = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(chunk):
                fn()
            e1.record()
            e1.synchronize()
            t.append(e0.elapsed_time(e1) / chunk)
        ms = sorted(t)[2]
        out[name] = {"bwd_ms": round(ms, 5),
                     "bwd_tflops": round(w.counted_flops()["bwd"] / (ms * 1e-3) / 1e12, 2)}
    print(json.dumps({"atomic_dq": out, "workload": w.name, "deterministic": "two_pass"}))


def e2e(args):
    """Training steps of the toy decoder (forward, backward, AdamW) with plain attention and
    then with the flash kernels patched in as its attention function."""
    import torch
    from tiled_attention_causal_amd import integration

    dev = torch.device("cuda:0")
    B, N, d_model, H, d_ff, L = 4, 1024, 768, 12, 2048, 4
    model = toy_model(d_model, H, d_ff, L, torch.bfloat16, dev)
    opt = torch.optim.AdamW(model.parameters(), lr=1e-4)
    x = (torch.randn(B, N, d_model, generator=torch.Generator().manual_seed(1))
         .to(dev, torch.bfloat16))

    def step():
        opt.zero_grad(set_to_none=True)
        loss = model(x).float().pow(2).mean()
        loss.backward()
        opt.step()

    def timed(steps):
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    mod = sys.modules[__name__]
    t_plain = timed(args.steps)
    with integration.patched(mod, "scaled_dot_product_attention"):
        t_flash = timed(args.steps)
    cfg = {"B": B, "N": N, "d_model": d_model, "heads": H, "d_ff": d_ff, "layers": L,
           "dtype": "bf16", "causal": True}
    for name, t in (("plain", t_plain), ("flash", t_flash)):
        print(json.dumps({"e2e": name, "ms_per_step": round(t * 1e3, 4),
                          "tokens_per_s": round(B * N / t, 1), "config": cfg}))


def copy_calibration():
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    dev = torch.device("cuda:0")
    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the attention path is "
              "not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    from seeded_inputs import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (cuda:0 on ROCm)", file=sys.stderr)
        sys.exit(1)
    import tiled_attention_causal_amd
    tiled_attention_causal_amd.load()  # fail loudly if the HIP library is missing
    if args.sweep:
        sweep(args)
        return
    if args.e2e:
        e2e(args)
        return
    if args.atomic_dq:
        atomic_dq(args)
        return

    peak = device_peak()
    peak_tf = peak["bf16_tflops"]
    w = WORKLOADS[args.workload]
    # Every workload's inputs are drawn and placed on the GPU before anything is timed, so
    # the GPU runs the measurements back to back: after even a fraction of a second idle it
    # drops its clock and takes some milliseconds of work to regain it.
    spaces = {w.name: Workspace(w)}
    configs = None
    if not args.no_configs:
        for name, ww in WORKLOADS.items():
            if name not in spaces:
                spaces[name] = Workspace(ww)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
        torch.cuda.synchronize()
        configs = []
        # The headline's workload goes last, so the headline starts from the clock and cache
        # state its own back-to-back steps leave (the state a training loop runs in), not
        # from the power state another workload's warm chunks leave behind.
        order = [n for n in WORKLOADS if n != w.name] + [w.name]
        for name in order:
            ww = WORKLOADS[name]
            reps = max(1, args.config_reps // 5) if ww.Nq >= 16384 else args.config_reps
            c = config_block(spaces[name], reps, flush)
            configs.append(c)
            print(f"{name:18s} flushed median fwd {c['fwd']['median_ms']:.4f} ms, bwd "
                  f"{c['bwd']['median_ms']:.4f} ms, fwd+bwd {c['fwd_bwd']['median_ms']:.4f} ms "
                  f"({c['fwd_bwd']['tflops']:.1f} TF/s); warm {c['warm_fwd_bwd']['ms']:.4f} ms",
                  file=sys.stderr, flush=True)
        del flush

    fl = w.counted_flops()
    r = time_workload(spaces[w.name], args.steps, args.warmup)
    value = fl["total"] / (r["ms_per_step"] * 1e-3) / 1e12
    bwd_tf = fl["bwd"] / (r["bwd_ms_mean"] * 1e-3) / 1e12
    main_tf = fl["bwd"] / (r["bwd_main_ms_mean"] * 1e-3) / 1e12
    fwd_tf = fl["fwd"] / (r["fwd_ms_mean"] * 1e-3) / 1e12
    fwd_name, bwd_name = r["kernels"]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds, 3.0 * args.cpu_seconds)

    out = {
        "metric": "causal attention fwd+bwd TFLOP/s (bf16, d=64) and % of MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / peak_tf, 2),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "input_dtype": w.dtype},
        "peak": peak,
        "passes": {"fwd_kernel": fwd_name, "fwd_ms": round(r["fwd_ms_mean"], 5),
                   "fwd_tflops": round(fwd_tf, 2), "bwd_kernel": bwd_name,
                   "bwd_ms": round(r["bwd_ms_mean"], 5), "bwd_tflops": round(bwd_tf, 2),
                   "bwd_preprocess_ms": round(r["prep_ms_mean"], 5),
                   "bwd_main_ms": round(r["bwd_main_ms_mean"], 5)},
        "roofline": {"kernel": bwd_name, "bound": "mfma", "achieved": round(main_tf, 2),
                     "peak": peak_tf, "unit": "TFLOP/s",
                     "frac": round(main_tf / peak_tf, 4),
                     "traffic": read_traffic(w.name, bwd_name)},
        "cpu_baseline": cpu,
        "configs": configs,
        "order": ("per-workload flushed block (the headline's workload last), then the "
                  "headline's warm-up and timed steps" if configs is not None else "headline only"),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
