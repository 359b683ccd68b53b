#!/usr/bin/env python3
"""Benchmark of the fused chunked top-K KL loss, forward + backward, on one MI355X.

One step = fckl_forward + fckl_backward over the whole batch (N tokens) of the
GPT-OSS-20B-shaped workload at 32K tokens: N=32768, H=2880, V=201088, K=100, T=1,
bf16 h / W / teacher logits, fp32 accumulation.  Inputs are synthetic (seeded
generators in synth/, same shapes and distributions; the teacher cache is the exact
top-100 of a perturbed copy of the LM head) and resident in HBM before timing.

Prints one JSON line.  `value` is tokens/s of whole fwd+bwd steps.  `roofline` is
the dominant kernel's achieved bf16 MFMA rate: its algorithmic flops per launch
(2 * tokens * V * H) over its mean launch time, taken with HIP events that the
library records around each launch on its own stream during the timed steps.
`cpu_baseline` times the CPU oracle (fp64) on a small sample of the same tokens.
`single_call` times the same step done by fckl_forward_backward, which forms each
chunk's logits once (6 N V H flop); it is reported beside the main line, which times
the two passes of the method as defined (8 N V H flop).  `teacher_topk` times the
teacher-side extraction of the top-K cache from the same hidden states (fckl_topk), and
the same call with its first pass over the whole vocabulary.
`autograd_module` times FusedChunkedKLLoss as a training loop calls it (forward, then
loss.backward()), with the two passes and with single_call=True.
`full_teacher` times the online variant against the teacher's whole distribution
(fckl_full_forward_backward), with a teacher of the same shape (a seeded perturbed copy
of the student's hidden states and head, synth.full_teacher): 2 N V Ht + 6 N V H flop
per step.
`w_stream` gives, for each product that streams the LM head, its algorithmic W bytes per
launch (V H bf16, read once per launch) over the live launch time.  `memory_slope` runs
one step at N = 32K .. 256K tokens with the step's chunk and fits peak = a + b N: b is the
per-token cost of the inputs and outputs, with no N x V term.  `dense_baseline` is the
same loss with the N x V logits materialised in eager torch (peak memory and step time),
run last with only the inputs resident.
`library_gemm` is context for the roofline, not part of the loss: the platform BLAS
library's bf16 GEMM (torch.nn.functional.linear, which calls hipBLASLt) on one logit
product's shape, a chunk of h times W^T with bf16 output, timed on the same GPU with its
shader clock sampled as for the main measurement.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s fwd+bwd of fused top-K KL (MFMA % of peak) + peak GiB, N=32K V=201088"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
GiB = float(1 << 30)


class HipEvents:
    """hipEvent_t handles from libamdhip64 (the library records them on its stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = e.value
        return arr

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float(0)
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, arr):
        for e in arr:
            self.hip.hipEventDestroy(e)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c3", help="synth workload key (default c3: the 32K-token GPT-OSS-20B shape)")
    ap.add_argument("--tokens", type=int, default=0, help="override N (for quick runs)")
    ap.add_argument("--chunk", type=int, default=0, help="tokens per chunk (0 = library scheduler)")
    ap.add_argument("--cpu-tokens", type=int, default=256, help="oracle sample size for cpu_baseline (0 = skip)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense torch KL baseline (N x V logits materialised: peak memory and step time)")
    ap.add_argument("--no-slope", action="store_true",
                    help="skip the peak-memory fit over N = 32K .. 256K tokens")
    ap.add_argument("--no-single-call", action="store_true",
                    help="skip timing fckl_forward_backward (the single-call path) after the main measurement")
    ap.add_argument("--no-topk", action="store_true",
                    help="skip timing the teacher-side top-K extraction (fckl_topk) of the same hidden states")
    ap.add_argument("--sweep", default="4096",
                    help="comma-separated chunk sizes: also time the step and its peak memory at each (default "
                         "4096, the chunk at which the 32K-token step peaks under 7 GiB; '' = none)")
    ap.add_argument("--no-library-gemm", action="store_true",
                    help="skip timing the BLAS library's bf16 GEMM on one logit product's shape")
    ap.add_argument("--no-module", action="store_true",
                    help="skip the torch autograd module leg (FusedChunkedKLLoss, both modes)")
    ap.add_argument("--no-full", action="store_true",
                    help="skip the full-vocabulary teacher variant (fckl_full_forward_backward)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (reference dispatch for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import chunked_top_kl_chunk_amd as fckl
    import synth

    fckl.load()
    dev = torch.device("cuda:0")
    # the device's own count of free memory (hipMemGetInfo) before anything of this run
    free_start = torch.cuda.mem_get_info(dev)[0]
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    wl = synth.WORKLOADS[args.workload]
    if args.tokens:
        wl = wl.with_tokens(args.tokens)
    N, H, V, K, T = wl.N, wl.H, wl.V, wl.K, wl.T
    log("workload %s N=%d H=%d V=%d K=%d T=%g: generating inputs" % (wl.name, N, H, V, K, T))
    t0 = time.time()
    x = synth.make_inputs(wl, device=dev)
    log("inputs ready in %.1fs" % (time.time() - t0))
    torch.cuda.synchronize()
    # the generator's products leave torch's BLAS workspace allocated, which pins a cached
    # segment: release both, so that the step's own allocations are what the device sees
    if hasattr(torch._C, "_cuda_clearCublasWorkspaces"):
        torch._C._cuda_clearCublasWorkspaces()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    h = torch.from_numpy(x.h_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    W = torch.from_numpy(x.W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    idx = torch.from_numpy(np.ascontiguousarray(x.idx)).to(dev)
    tl = torch.from_numpy(x.tl_bits.view(np.int16)).to(dev).view(torch.bfloat16)

    desc = fckl.desc_for(h, W, idx, tl, T, args.chunk)
    chunk, ws_bytes = fckl.plan(desc) if args.chunk == 0 else (args.chunk, fckl.workspace_size(desc, args.chunk))
    nchunks = -(-N // chunk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    loss = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    dH = torch.empty(N, H, dtype=torch.float32, device=dev)
    dW = torch.empty(V, H, dtype=torch.float32, device=dev)
    log("chunk %d (%d chunks), workspace %.2f GiB" % (chunk, nchunks, ws_bytes / GiB))

    def step(profile=None):
        fckl.forward(h, W, idx, tl, T=T, chunk=chunk, ws=ws, loss_tok=loss, lse=lse, loss_mean=mean,
                     profile=profile)
        fckl.backward(h, W, idx, tl, lse, T=T, chunk=chunk, ws=ws, dH=dH, dW=dW, profile=profile)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log("warmup step %d done" % i)
    peak_bytes = torch.cuda.max_memory_allocated()
    # cross-check from the device side: the drop in free device memory since the start
    # of the run.  An upper bound of the peak: it also holds the allocator's rounding to
    # its segments, what input generation left reserved and the runtime's code objects.
    device_used = free_start - torch.cuda.mem_get_info(dev)[0]

    clock = {}
    ms_step, kernels = timed_steps(fckl, step, args.steps, nchunks, clock)
    tokens_per_s = N * 1e3 / ms_step
    log("timed %d steps: %.2f ms/step, %.0f tokens/s" % (args.steps, ms_step, tokens_per_s))
    # the two passes on their own (after the timed steps, so they do not enter `value`)
    reps = max(1, min(args.steps, 5))
    pass_ms = {}
    for name, call in (("forward", lambda: fckl.forward(h, W, idx, tl, T=T, chunk=chunk, ws=ws, loss_tok=loss,
                                                        lse=lse, loss_mean=mean)),
                       ("backward", lambda: fckl.backward(h, W, idx, tl, lse, T=T, chunk=chunk, ws=ws, dH=dH,
                                                          dW=dW))):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        pass_ms[name] = (time.perf_counter() - t0) * 1e3 / reps
    log("forward %.2f ms, backward %.2f ms" % (pass_ms["forward"], pass_ms["backward"]))
    gemms = ("fwd_logits", "bwd_logits", "dh", "dw")
    # the products that stream the LM head read the V H bf16 values of the vocabulary rows
    # they cover (the backward ones one slab at a time): W bytes per chunk
    w_bytes = 2.0 * V * H
    w_stream = {"bytes_per_chunk": w_bytes,
                "note": "algorithmic W bytes (W, W, W^T: 2 V H per chunk each, the backward's launches one "
                        "vocabulary slab at a time) over the kernel's live time; the L2-miss bytes "
                        "per launch (FETCH_SIZE / TCC_EA0_RDREQ_DRAM count requests to the memory side, which the "
                        "256 MB MALL serves in part, so an upper bound on HBM bytes: no counter on this GPU "
                        "separates MALL hits from HBM reads) are in profiles/hbm_bytes_<workload>.md"}
    for name in ("fwd_logits", "bwd_logits", "dh"):
        d = kernels[name]
        w_stream[name + "_gb_per_s"] = round(2.0 * H * d["vrows"] / (d["ms"] * 1e-3) / 1e9, 1)
    for name, d in kernels.items():
        d["avg_ms"] = d["ms"] / d["launches"]
        d["ms_per_step"] = d["ms"] / args.steps
        if name in gemms:
            # 2 flop per token, vocabulary row and hidden entry of each launch
            flops = 2.0 * d["token_rows"] * H
            d["tflops"] = flops / (d["ms"] * 1e-3) / 1e12
            d["mfma_frac"] = d["tflops"] / PEAK_BF16_TFLOPS
    dom = max(gemms, key=lambda n: kernels[n]["ms"])
    kd = kernels[dom]
    flops_per_launch = 2.0 * kd["token_rows"] / kd["launches"] * H
    achieved = flops_per_launch / (kd["avg_ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(wl.name, chunk, dom),
                "avg_launch_ms": round(kd["avg_ms"], 4),
                "flops_per_launch": flops_per_launch}
    if clock.get("mhz"):
        # the same rate against the dense bf16 peak at the shader clock measured during the
        # timed steps (the published 2.5 PFLOP/s assumes 2400 MHz)
        roofline["sustained_clock_mhz"] = round(clock["mhz"], 1)
        roofline["peak_at_sustained_clock"] = round(PEAK_BF16_TFLOPS * clock["mhz"] / 2400.0, 1)
        roofline["frac_at_sustained_clock"] = round(achieved / roofline["peak_at_sustained_clock"], 4)
    step_tflops = 8.0 * N * V * H / (ms_step * 1e-3) / 1e12

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "N": N, "H": H, "V": V, "K": K, "T": T, "chunk": chunk,
                   "chunks": nchunks},
        "roofline": roofline,
        "mfma_frac_step": round(step_tflops / PEAK_BF16_TFLOPS, 4),
        "forward_ms": round(pass_ms["forward"], 3), "backward_ms": round(pass_ms["backward"], 3),
        "step_tflops": round(step_tflops, 1),
        "peak_gib": round(peak_bytes / GiB, 3),
        "device_used_gib": round(device_used / GiB, 3),
        "workspace_gib": round(ws_bytes / GiB, 3),
        "w_stream": w_stream,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
    }

    if not args.no_single_call:
        # The same step as one fckl_forward_backward call: each chunk's logits are formed
        # once (6 N V H flop instead of 8).  Reported beside the main line, which times
        # the two passes the method defines.
        # its workspace also holds the chunk's kept exponentials (fckl_single_plan)
        sdesc = fckl.desc_for(h, W, idx, tl, T, chunk)
        sws_bytes = fckl.single_plan(sdesc)[1]
        del ws
        sws = torch.empty(sws_bytes, dtype=torch.uint8, device=dev)

        def single(profile=None):
            fckl.forward_backward(h, W, idx, tl, T=T, chunk=chunk, ws=sws, loss_tok=loss, lse=lse, loss_mean=mean,
                                  dH=dH, dW=dW, profile=profile)
        single()
        torch.cuda.synchronize()
        ms1, k1 = timed_steps(fckl, single, args.steps, nchunks)
        del sws
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        log("single call: %.2f ms/step, %.0f tokens/s" % (ms1, N * 1e3 / ms1))
        out["single_call"] = {
            "value": round(N * 1e3 / ms1, 1), "unit": "tokens/s", "ms_per_step": round(ms1, 3),
            "flops_per_step": 6.0 * N * V * H, "workspace_gib": round(sws_bytes / GiB, 3),
            "mfma_frac": round(6.0 * N * V * H / (ms1 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels": {k: {"launches": v["launches"], "ms_per_step": round(v["ms"] / args.steps, 4)}
                        for k, v in k1.items()},
        }

    if not args.no_library_gemm:
        out["library_gemm"] = library_gemm(h, W, chunk)
        log("library bf16 GEMM %s: %.3f ms, %.1f TFLOP/s" % (
            "x".join(str(out["library_gemm"][k]) for k in ("m", "n", "k")), out["library_gemm"]["ms"],
            out["library_gemm"]["tflops"]))

    if args.sweep:
        # The chunk scheduler's trade-off: the same step at other chunk sizes, each with
        # its own workspace, peak memory measured from the inputs and outputs alone.
        del ws
        ws = None
        sweep = []
        for c in [int(x) for x in args.sweep.split(",") if x]:
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            cws_bytes = fckl.workspace_size(fckl.desc_for(h, W, idx, tl, T, c), c)
            cws = torch.empty(cws_bytes, dtype=torch.uint8, device=dev)

            def sweep_step(profile=None):
                fckl.forward(h, W, idx, tl, T=T, chunk=c, ws=cws, loss_tok=loss, lse=lse, loss_mean=mean)
                fckl.backward(h, W, idx, tl, lse, T=T, chunk=c, ws=cws, dH=dH, dW=dW)
            sweep_step()
            torch.cuda.synchronize()
            reps = max(1, min(args.steps, 3))
            t0 = time.perf_counter()
            for _ in range(reps):
                sweep_step()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / reps
            peak = torch.cuda.max_memory_allocated()
            log("chunk %d: %.2f ms per step, peak %.2f GiB, workspace %.2f GiB" % (c, ms, peak / GiB, cws_bytes / GiB))
            sweep.append({"chunk": c, "ms_per_step": round(ms, 3), "tokens_per_s": round(N * 1e3 / ms, 1),
                          "peak_gib": round(peak / GiB, 3), "workspace_gib": round(cws_bytes / GiB, 3)})
            del cws
        out["chunk_sweep"] = sweep

    if not args.no_module:
        # The torch autograd module, as a training loop calls it (loss = module(...);
        # loss.backward(), gradients cast to the bf16 leaves by autograd): the two passes,
        # and single_call=True (gradients formed in the forward call, scaled in backward).
        from chunked_top_kl_chunk_amd.loss import FusedChunkedKLLoss
        hl = h.detach().clone().requires_grad_(True)
        Wl = W.detach().clone().requires_grad_(True)
        mod_ms = {}
        for single in (False, True):
            mod = FusedChunkedKLLoss(temperature=T, chunk=chunk, single_call=single)

            def module_step():
                hl.grad = None
                Wl.grad = None
                mod(hl, Wl, idx, tl).backward()
            module_step()
            torch.cuda.synchronize()
            reps = max(1, min(args.steps, 3))
            t0 = time.perf_counter()
            for _ in range(reps):
                module_step()
            torch.cuda.synchronize()
            mod_ms[single] = (time.perf_counter() - t0) * 1e3 / reps
        log("autograd module: %.2f ms per step, single_call %.2f ms" % (mod_ms[False], mod_ms[True]))
        out["autograd_module"] = {"ms_per_step": round(mod_ms[False], 3), "tokens_per_s": round(N * 1e3 / mod_ms[False], 1),
                                  "single_call_ms_per_step": round(mod_ms[True], 3),
                                  "single_call_tokens_per_s": round(N * 1e3 / mod_ms[True], 1)}
        del hl, Wl

    if not args.no_topk:
        # Teacher-side extraction of the cache the loss reads: top-K of h W^T in two
        # passes of the logit product, the first over every 4th vocabulary tile when that
        # gives at least 4 K slice maxima (2.5 N V H flop), else over all of it (4 N V H).
        nvt = -(-V // 256)
        partial = -(-nvt // 4) * 4 >= 4 * K
        tws = torch.empty(fckl.topk_workspace_size(fckl.make_desc(N, H, V, K)), dtype=torch.uint8, device=dev)
        ti = torch.empty(N, K, dtype=torch.int32, device=dev)
        tv = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
        reps = max(1, min(args.steps, 3))
        tk_ms = {}
        for full_first in (False, True):
            fckl.topk(h, W, K, ws=tws, topk_idx=ti, topk_logit=tv, full_first_pass=full_first)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                fckl.topk(h, W, K, ws=tws, topk_idx=ti, topk_logit=tv, full_first_pass=full_first)
            torch.cuda.synchronize()
            tk_ms[full_first] = (time.perf_counter() - t0) * 1e3 / reps
        ms_t = tk_ms[False]
        flops = (2.5 if partial else 4.0) * N * V * H
        log("teacher top-%d: %.2f ms per call (first pass over every tile: %.2f ms)" % (K, ms_t, tk_ms[True]))
        out["teacher_topk"] = {"K": K, "ms_per_call": round(ms_t, 3), "tokens_per_s": round(N * 1e3 / ms_t, 1),
                               "first_pass": "every 4th vocabulary tile" if partial else "every tile",
                               "flops_per_call": flops,
                               "mfma_frac": round(flops / (ms_t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                               "ms_per_call_full_first_pass": round(tk_ms[True], 3)}
        del tws, ti, tv

    if not args.no_full:
        # Online distillation against the full teacher distribution, teacher of the same
        # shape: a seeded perturbed copy of h and W, its logits formed chunk by chunk.
        tch = synth.full_teacher(wl, x)
        h_t = torch.from_numpy(tch.h_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        W_t = torch.from_numpy(tch.W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        del tch
        fdesc = fckl.make_desc(N, H, V, 1, T)
        fchunk, fws_bytes = fckl.full_plan(fdesc, H)
        del ws
        fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev)

        def full(profile=None):
            fckl.full_forward_backward(h, W, h_t, W_t, T=T, chunk=fchunk, ws=fws, loss_tok=loss, lse=lse,
                                       loss_mean=mean, dH=dH, dW=dW, profile=profile)
        full()
        torch.cuda.synchronize()
        nf = -(-N // fchunk)
        msf, kf = timed_steps(fckl, full, args.steps, nf)
        flops = 2.0 * N * V * H + 6.0 * N * V * H
        log("full teacher: %.2f ms/step, %.0f tokens/s (chunk %d)" % (msf, N * 1e3 / msf, fchunk))
        out["full_teacher"] = {
            "value": round(N * 1e3 / msf, 1), "unit": "tokens/s", "ms_per_step": round(msf, 3),
            "teacher_hidden": H, "chunk": fchunk, "workspace_gib": round(fws_bytes / GiB, 3),
            "flops_per_step": flops, "mfma_frac": round(flops / (msf * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels": {k: {"launches": v["launches"], "ms_per_step": round(v["ms"] / args.steps, 4)}
                        for k, v in kf.items()},
        }
        del fws, h_t, W_t
        ws = None

    if not args.no_slope:
        del ws
        ws = None
        out["memory_slope"] = memory_slope(W, K, chunk)

    if not args.no_dense:
        # the fused path's workspace and outputs are released first: the dense loss is
        # measured with only the inputs resident
        del ws, loss, lse, mean, dH, dW
        out["dense_baseline"] = dense_baseline(h, W, idx, tl, T)
        if out["dense_baseline"].get("ok"):
            out["dense_baseline"]["fused_peak_gib"] = out["peak_gib"]

    if args.cpu_tokens > 0:
        out["cpu_baseline"] = cpu_baseline(x, wl, args.cpu_tokens)
    print(json.dumps(out), flush=True)


def library_gemm(h, W, rows, reps=40):
    """The BLAS library's bf16 GEMM on one logit product's shape: h[:rows] W^T, bf16 in and
    out with fp32 accumulation, `reps` back-to-back calls between two events on torch's
    stream, the shader clock sampled meanwhile."""
    import torch
    import torch.nn.functional as F
    a = h[:rows]
    V, H = W.shape
    for _ in range(3):
        c = F.linear(a, W)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with ClockSampler() as cs:
        e0.record()
        for _ in range(reps):
            c = F.linear(a, W)
        e1.record()
        torch.cuda.synchronize()
    del c
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * rows * V * H / (ms * 1e-3) / 1e12
    res = {"op": "torch.nn.functional.linear (hipBLASLt), bf16 in and out, fp32 accumulation",
           "m": int(rows), "n": int(V), "k": int(H), "ms": round(ms, 4), "tflops": round(tf, 1),
           "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    mhz = cs.mean_mhz()
    if mhz:
        res["sustained_clock_mhz"] = round(mhz, 1)
        res["frac_at_sustained_clock"] = round(tf / (PEAK_BF16_TFLOPS * mhz / 2400.0), 4)
    return res


class ClockSampler:
    """Samples the GPU's current shader clock (the amdgpu driver's pp_dpm_sclk, its
    "S:" line or the level marked "*") every 50 ms on a background thread while the
    timed steps run.  mean_mhz() is None where the file is not readable."""

    def __init__(self, period_s=0.05):
        import glob
        import threading
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        import re
        try:
            text = open(self.path).read()
        except OSError:
            return None
        for line in text.splitlines():
            if "*" in line:
                m = re.search(r"(\d+)\s*Mhz", line, re.I)
                if m:
                    return int(m.group(1))
        return None

    def _run(self):
        while not self._stop.wait(self.period):
            v = self._read()
            if v is not None:
                self.samples.append(v)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.path:
            self._stop.set()
            self._thread.join()

    def mean_mhz(self):
        busy = [v for v in self.samples if v >= 500]     # samples taken while the GPU worked
        return sum(busy) / len(busy) if busy else None


def timed_steps(fckl, step, steps, nchunks, clock=None):
    """Time `steps` calls of step(profile) between two device syncs; the library records
    HIP events around each of its kernel launches on its stream.  Returns (ms per step,
    per-kernel {launches, ms, tokens})."""
    import torch
    ev = HipEvents()
    # the backward launches three of its kernels once per vocabulary slab
    per_step = nchunks * (len(fckl.KERNELS) + 3 * 16) + 4
    cap = per_step * max(steps, 1)
    events = ev.create(2 * cap)
    kid = (ctypes.c_int32 * cap)()
    work = (ctypes.c_int32 * cap)()
    vrows = (ctypes.c_int32 * cap)()
    prof = fckl.Profile((1 << len(fckl.KERNELS)) - 1, cap, 0, events, kid, work, vrows)
    torch.cuda.synchronize()
    sampler = ClockSampler() if clock is not None else None
    if sampler:
        sampler.__enter__()
    t_start = time.perf_counter()
    for _ in range(steps):
        step(prof)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    if sampler:
        sampler.__exit__(None, None, None)
        clock["mhz"] = sampler.mean_mhz()
        clock["samples"] = len(sampler.samples)
    kernels = {}
    for i in range(prof.count):
        name = fckl.KERNELS[kid[i]]
        d = kernels.setdefault(name, {"launches": 0, "ms": 0.0, "tokens": 0, "vrows": 0, "token_rows": 0})
        d["launches"] += 1
        d["ms"] += ev.elapsed_ms(events[2 * i], events[2 * i + 1])
        d["tokens"] += work[i]
        d["vrows"] += vrows[i]
        d["token_rows"] += work[i] * vrows[i]
    ev.destroy(events)
    return elapsed * 1e3 / steps, kernels


KERNEL_NAMES = {"fwd_logits": "forward_logits_kernel", "bwd_logits": "backward_logits_kernel",
                "dh": "dh_kernel", "dw": "dw_kernel"}


def measured_traffic(workload, chunk, kernel):
    """HBM bytes (read + written) per launch of `kernel`, from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs summarised in profiles/, scaled by the reference copy; None when no
    summary exists for this workload and chunk or the kernels changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_bytes_%s.json" % workload)
    src = os.path.join(ROOT, "chunked_top_kl_chunk_amd", "csrc", "fckl_kernels.hip")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("chunk") != chunk or rec.get("kernels_source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    for name, v in rec["kernels"].items():
        if name.startswith(KERNEL_NAMES[kernel]):
            return round(v["read_bytes"] + v["write_bytes"])
    return None


def memory_slope(W, K, chunk, Ns=(32768, 65536, 131072, 262144), seed=7):
    """Peak device memory of one fwd+bwd step at growing N with a fixed chunk, the head W
    resident throughout.  Inputs are drawn on the device from a seeded generator (their
    values do not change the memory): h ~ N(0,1), K distinct indices per token
    (a random offset plus k * (V // K), modulo V), logits N(0, 3^2) sorted descending.
    Fits peak = a + b N by least squares; b is the per-token cost, to compare with the
    inputs and outputs alone (2H + 4H + 6K + 8 bytes) and with the 4 V bytes per token
    that one fp32 logit row would add."""
    import numpy as np
    import torch
    import chunked_top_kl_chunk_amd as fckl
    dev = W.device
    V, H = W.shape
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    points = []
    for N in Ns:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        h = torch.randn(N, H, device=dev, dtype=torch.bfloat16, generator=gen)
        off = torch.randint(0, V, (N, 1), device=dev, generator=gen)
        idx = ((off + torch.arange(K, device=dev) * (V // K)) % V).to(torch.int32)
        tl = (torch.randn(N, K, device=dev, generator=gen) * 3.0).sort(dim=1, descending=True).values
        tl = tl.to(torch.bfloat16)
        t0 = time.perf_counter()
        _, lse, _ = fckl.forward(h, W, idx, tl, T=1.0, chunk=chunk)
        dH, dW = fckl.backward(h, W, idx, tl, lse, T=1.0, chunk=chunk)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        peak = torch.cuda.max_memory_allocated()
        points.append({"N": N, "peak_gib": round(peak / GiB, 3), "step_peak_minus_resident_gib":
                       round((peak - base) / GiB, 3), "ms_per_step": round(ms, 1)})
        log("memory slope: N=%d peak %.2f GiB (%.2f GiB above the resident head), %.1f ms" %
            (N, peak / GiB, (peak - base) / GiB, ms))
        del h, off, idx, tl, lse, dH, dW
    n = np.array([p["N"] for p in points], np.float64)
    y = np.array([p["peak_gib"] for p in points], np.float64) * GiB
    b, a = np.polyfit(n, y, 1)
    torch.cuda.empty_cache()
    return {"chunk": chunk, "points": points, "bytes_per_token": round(float(b), 1),
            "intercept_gib": round(float(a) / GiB, 3),
            "inputs_outputs_bytes_per_token": 2 * H + 4 * H + 6 * K + 8,
            "one_fp32_logit_row_bytes_per_token": 4 * V}


def dense_baseline(h, W, idx, tl, T, reps=2):
    """The dense loss in eager torch: the full N x V logits materialised, autograd
    backward.  Peak memory of one step, then the mean time of `reps` more steps."""
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    Wg = W.detach().clone().requires_grad_(True)
    hg = h.detach().clone().requires_grad_(True)

    def dense_step():
        Wg.grad = None
        hg.grad = None
        z = (hg @ Wg.t()).float() / T
        logq = torch.log_softmax(z, dim=1)
        logp = torch.log_softmax(tl.float() / T, dim=1)
        per_tok = (T * T) * (logp.exp() * (logp - torch.gather(logq, 1, idx.long()))).sum(1)
        per_tok.mean().backward()

    try:
        dense_step()
        torch.cuda.synchronize()
        res = {"peak_gib": round(torch.cuda.max_memory_allocated() / GiB, 3),
               "inputs_gib": round(base / GiB, 3), "ok": True}
        t0 = time.perf_counter()
        for _ in range(reps):
            dense_step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / reps
        res.update({"ms_per_step": round(ms, 2), "tokens_per_s": round(h.shape[0] * 1e3 / ms, 1)})
    except torch.cuda.OutOfMemoryError:
        res = {"ok": False, "error": "out of memory"}
    del Wg, hg
    torch.cuda.empty_cache()
    return res


def cpu_baseline(x, wl, S):
    """The CPU oracle (fp64, OpenMP) on S sampled tokens: forward, then backward with
    those tokens' dH rows and their dW contribution -- 8*V*H flop per token."""
    import numpy as np
    import oracle
    import synth
    rows = synth.sample_rows(wl, S)
    h64 = x.h.astype(np.float64)
    W64 = x.W.astype(np.float64)
    tl64 = x.tl.astype(np.float64)
    threads = oracle.num_threads()
    log("cpu baseline: oracle on %d tokens, %d threads" % (S, threads))
    t0 = time.perf_counter()
    oracle.forward(h64, W64, x.idx, tl64, wl.T, rows=rows)
    oracle.backward(h64, W64, x.idx, tl64, wl.T, rows=rows, n_norm=wl.N)
    dt = time.perf_counter() - t0
    return {"value": round(S / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d seeded-sampled tokens of the %d-token workload: forward and backward (dH rows and "
                      "their dW contribution), fp64, %.1f s" % (S, wl.N, dt)}


if __name__ == "__main__":
    main()
