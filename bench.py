"""Benchmark: causal bf16 attention forward + backward on one MI355X.

One step = the whole hot path once: fa_forward, then the three backward
steps fa_backward runs (D preprocess, dK/dV, dQ), called individually so that
HIP events between them time each kernel. Inputs are resident in HBM before
the timed region. Prints one JSON line.

Workload: B=2, H=16, N=8192, d=128, causal, bf16 (the N=8K headline shape);
the N=32K, d=80 shape, the other three configurations (the fp32 N=256
forward, the bf16 N=2048 d=64 causal forward and the N=65536 causal
forward + backward with dropout 0.1; forward-only ones time the forward
alone) and a packed batch of sixteen causal sequences of
512..8192 tokens (with the time the same sequences take padded to the
longest), and a block-sparse N=32K sequence (local window plus global key
blocks, with the dense time on the same shape), and the split-KV forward on a
decode shape and a small-batch prefill, and the forward with FP8 scores on
the N=8K shape are reported alongside under "also".
FLOP convention: forward 4*B*H*N^2*d, halved for causal; backward 2.5x.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import (SPARSE_WORKLOADS, SPLITKV_WORKLOADS, VARLEN_WORKLOADS, WORKLOADS,  # noqa: E402
                       block_mask_local_global, counted_flops, counted_flops_varlen, make_cross_inputs,
                       make_inputs, make_varlen_inputs)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 matrix-core peak (published)
PEAK_FP32_MFMA_TFLOPS = 157.3    # MI355X dense fp32 matrix-core peak (published)
METRIC = "attention fwd+bwd TFLOP/s & % of bf16 MFMA peak, causal, N=8K/32K"


def _device_inputs(w, torch):
    inp = make_inputs(w, with_grad=True)
    if w.dtype == "f32":
        dev = {k: torch.from_numpy(v[0]).cuda() for k, v in inp.items()}
    else:
        dev = {k: torch.from_numpy(v[0].view(np.int16)).view(torch.bfloat16).cuda() for k, v in inp.items()}
    return dev


def kernel_units(w):
    """Algorithmic MFMA FLOPs per launch of each kernel: 2*d per matrix
    product per counted score element (B*H*N^2, halved when causal).
    forward: S and P V (2 products); dK/dV: S, dP, dV, dK (4);
    dQ: S, dP, dQ (3). The D preprocess is bandwidth-bound: its bytes are
    O and dO read plus D written."""
    elems = w.B * w.H * float(w.N) * w.N / (2.0 if w.causal else 1.0)
    tensor_bytes = w.B * w.N * w.H * w.d * 2
    if w.dtype == "f32":
        # fp32 runs on the fp32 matrix cores (v_mfma_f32_32x32x2_f32)
        return {"forward": ("mfma_f32", 2 * 2 * w.d * elems)}
    return {
        "forward": ("mfma", 2 * 2 * w.d * elems),
        "bwd_preprocess": ("hbm", 2 * tensor_bytes + 4 * w.B * w.H * w.N),
        "bwd_dkdv": ("mfma", 4 * 2 * w.d * elems),
        "bwd_dq": ("mfma", 3 * 2 * w.d * elems),
    }


class ClockStamps:
    """Mean shader clock of each XCD over the timed steps: clock-stamp
    kernels (libfa_clock.so, fa_clock_stamp) enqueued on the benchmark's
    stream right before the first timed step and right after the last one
    read each XCD's shader-cycle counter (s_memtime) and the fixed 100 MHz
    real-time counter (s_memrealtime). Per XCD, clock = 100 MHz * cycles /
    real-time ticks between the two stamps (work-groups matched by the XCD id
    they read). The stamps lie outside the HIP-event brackets of the steps.
    Reports None with the reason if the library is missing."""

    MIN_REGION_MS = 2.0

    def __init__(self, torch, blocks=256):
        import ctypes
        self.torch = torch
        self.blocks = blocks
        self.error = None
        path = os.path.join(ROOT, "exact_io_aware_72_amd", "libfa_clock.so")
        try:
            self.lib = ctypes.CDLL(path)
            self.lib.fa_clock_stamp.restype = ctypes.c_int
            self.lib.fa_clock_stamp.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        except OSError as e:
            self.lib, self.error = None, f"{path}: {e}"
        self.bufs = [torch.zeros(4 * blocks, dtype=torch.int64, device="cuda") for _ in range(2)]
        self._ctypes = ctypes

    def stamp(self, i):
        if self.lib is None:
            return
        stream = self._ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        if self.lib.fa_clock_stamp(self.bufs[i].data_ptr(), self.blocks, stream) != 0:
            self.error = "fa_clock_stamp failed"

    def result(self):
        """Call after synchronising."""
        if self.lib is None or self.error:
            return {"mhz": None, "error": self.error}
        a, b = (x.cpu().numpy().reshape(-1, 4).astype(np.int64) for x in self.bufs)
        # Stamps of the two sides taken on the same CU (XCD and HW_ID CU
        # fields): each XCD's reading is the median over its matched CUs.
        end = {}
        for r1 in b:
            end.setdefault((int(r1[0]), int(r1[3])), r1)
        pairs = {}
        for r0 in a:
            r1 = end.get((int(r0[0]), int(r0[3])))
            if r1 is not None and r1[2] > r0[2]:
                pairs.setdefault(int(r0[0]), []).append(100.0 * float(r1[1] - r0[1]) / float(r1[2] - r0[2]))
        per = {x: float(np.median(v)) for x, v in sorted(pairs.items())}
        region_ms = float(np.median([(r1[2] - r0[2]) / 1e5 for r0, r1 in zip(a, b)]))
        # An XCD that idles between the stamps can stop or reset its cycle
        # counter (seen on sub-millisecond regions), so short regions are not
        # reported, and readings outside 100 MHz .. the 2.4 GHz peak engine
        # clock are left out of the median.
        if region_ms < self.MIN_REGION_MS:
            return {"mhz": None, "per_xcd_mhz": per, "region_ms": region_ms,
                    "error": f"timed region shorter than {self.MIN_REGION_MS} ms"}
        ok = {x: v for x, v in per.items() if 100.0 < v < 2450.0}
        bad = {x: v for x, v in per.items() if x not in ok}
        if not ok:
            return {"mhz": None, "per_xcd_mhz": per, "error": "no plausible per-XCD reading"}
        return {"mhz": float(np.median(list(ok.values()))), "per_xcd_mhz": ok, "xcds_used": len(ok),
                "excluded_xcd_readings": bad,
                "source": "s_memtime cycles / s_memrealtime (100 MHz) ticks between stamps enqueued "
                          "before the first and after the last timed step, matched by XCD and CU; "
                          "median over each XCD's CUs, then over the XCDs",
                "region_ms": region_ms}


def run_gpu(w, steps, warmup, torch, fa, keep_outputs=False, sample_clock=False):
    """One step = fa_forward, then (for workloads with a backward pass) the
    D preprocess, dK/dV and dQ kernels; HIP events between the calls time
    each kernel. Step and pass times are medians over the timed steps;
    kernel_ms holds each kernel's mean launch time (the roofline's average
    launch duration) and kernel_ms_median the medians."""
    dev = _device_inputs(w, torch)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    args = (w.causal, w.dropout_p, w.dropout_seed, w.scale)
    names = ("forward", "bwd_preprocess", "bwd_dkdv", "bwd_dq") if w.backward else ("forward",)
    nev = len(names) + 1

    def step(ev=None):
        if ev:
            ev[0].record()
        fa.forward(q, k, v, *args, out=o, lse=lse)
        if ev:
            ev[1].record()
        if not w.backward:
            return
        fa.backward_preprocess(o, do, workspace=ws)
        if ev:
            ev[2].record()
        fa.backward_dkdv(q, k, v, do, lse, ws, *args, dk=dk, dv=dv)
        if ev:
            ev[3].record()
        fa.backward_dq(q, k, v, do, lse, ws, *args, dq=dq)
        if ev:
            ev[4].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    clock = ClockStamps(torch) if sample_clock else None
    t0 = time.perf_counter()
    if clock:
        clock.stamp(0)
    for i in range(steps):
        step(evs[i])
    if clock:
        clock.stamp(1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock_info = clock.result() if clock else None
    # Per step: first to last event of that step; the line reports the median
    # step and keeps the mean (first event of the first step to the last of
    # the last, over the step count) beside it.
    step_ms = [e[0].elapsed_time(e[-1]) for e in evs]
    ms_step = float(np.median(step_ms))
    ms_step_mean = evs[0][0].elapsed_time(evs[-1][-1]) / steps
    launch = {n: [e[j].elapsed_time(e[j + 1]) for e in evs] for j, n in enumerate(names)}
    per = {n: float(np.mean(t)) for n, t in launch.items()}
    per_median = {n: float(np.median(t)) for n, t in launch.items()}
    fwd_f, bwd_f = counted_flops(w.B, w.H, w.N, w.d, w.causal, w.backward)
    fwd_ms = per_median["forward"]
    bwd_ms = (per_median["bwd_preprocess"] + per_median["bwd_dkdv"] + per_median["bwd_dq"]
              if w.backward else None)
    return {
        "ms_per_step": ms_step,
        "ms_per_step_mean": ms_step_mean,
        "wall_s": wall,
        "clock": clock_info,
        "tflops": (fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "fwd_tflops": fwd_f / (fwd_ms * 1e-3) / 1e12,
        "bwd_tflops": bwd_f / (bwd_ms * 1e-3) / 1e12 if w.backward else None,
        "kernel_ms": per,
        "kernel_ms_median": per_median,
        "outputs": ({"O": o, "LSE": lse, "dQ": dq, "dK": dk, "dV": dv} if w.backward else
                    {"O": o, "LSE": lse}) if keep_outputs else None,
    }


def _mfma_roofline(tflops):
    return {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / PEAK_BF16_TFLOPS}


def run_gpu_varlen(wv, steps, warmup, torch, fa):
    """Packed variable-length batch: forward_varlen + backward_varlen per step,
    FLOPs counted per sequence. Also times the same sequences padded to the
    longest one as a fixed-length batch (what padding would cost)."""
    cu, inp = make_varlen_inputs(wv)
    dev = {k: torch.from_numpy(v[0].view(np.int16)).view(torch.bfloat16).cuda() for k, v in inp.items()}
    cu_d = torch.from_numpy(cu).cuda()
    lengths = np.diff(cu)
    maxlen = int(lengths.max())
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    total = q.shape[0]
    o = torch.empty_like(q)
    lse = torch.empty((wv.H, total), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty((wv.H, total), dtype=torch.float32, device="cuda")
    args = (wv.causal, wv.dropout_p, wv.dropout_seed, wv.scale)

    def step(ev=None):
        if ev:
            ev[0].record()
        fa.forward_varlen(q, k, v, cu_d, maxlen, *args, out=o, lse=lse)
        if ev:
            ev[1].record()
        fa.backward_varlen(q, k, v, o, do, lse, cu_d, maxlen, *args, dq=dq, dk=dk, dv=dv,
                           workspace=ws)
        if ev:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    # medians over the timed steps (the mean step beside them)
    ms_step = float(np.median([e[0].elapsed_time(e[2]) for e in evs]))
    ms_step_mean = evs[0][0].elapsed_time(evs[-1][2]) / steps
    fwd_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    fwd_f, bwd_f = counted_flops_varlen(lengths, wv.H, wv.d, wv.causal, True)
    del dev, q, k, v, do, o, dq, dk, dv
    torch.cuda.empty_cache()
    padded = WORKLOADS[3].with_(B=len(lengths), H=wv.H, N=maxlen, d=wv.d, causal=wv.causal,
                                dropout_p=wv.dropout_p)
    rp = run_gpu(padded, max(2, steps // 2), 1, torch, fa)
    return {
        "workload": wv.name, "num_seqs": len(lengths), "total_tokens": int(total),
        "max_seqlen": maxlen, "tflops": (fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12,
        "ms_per_step": ms_step, "ms_per_step_mean": ms_step_mean,
        "pct_of_peak": 100.0 * (fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "fwd_tflops": fwd_f / (fwd_ms * 1e-3) / 1e12, "bwd_tflops": bwd_f / (bwd_ms * 1e-3) / 1e12,
        "padded_fixed_length_ms_per_step": rp["ms_per_step"],
        "roofline": _mfma_roofline((fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12),
    }


def kept_score_elements(mask, N, causal):
    """Score elements a block mask (and the causal mask) leave in, per head."""
    blk = 128
    nb = mask.shape[-1]
    size = np.minimum(blk, N - blk * np.arange(nb))  # rows (= columns) per block
    full = np.outer(size, size).astype(np.float64)
    if causal:
        # below the diagonal every element counts, above none, on it a triangle
        tri = size * (size + 1) / 2.0
        full = np.tril(full, -1) + np.diag(tri)
    return float(np.sum(full * (mask != 0)))


def run_gpu_sparse(name, steps, warmup, torch, fa):
    """Block-sparse fwd + bwd on a long sequence; FLOPs counted on the kept
    score elements (4*d per element forward, 2.5x backward). Also times the
    dense kernels on the same shape."""
    w, kw = SPARSE_WORKLOADS[name]
    mask_np = block_mask_local_global(w.N, **kw)
    dev = _device_inputs(w, torch)
    m = torch.from_numpy(mask_np).cuda()
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    args = (w.causal, w.dropout_p, w.dropout_seed, w.scale)

    def step(ev=None):
        if ev:
            ev[0].record()
        fa.forward_blocksparse(q, k, v, m, *args, out=o, lse=lse)
        if ev:
            ev[1].record()
        fa.backward_blocksparse(q, k, v, o, do, lse, m, *args, dq=dq, dk=dk, dv=dv, workspace=ws)
        if ev:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    # medians over the timed steps (the mean step beside them)
    ms_step = float(np.median([e[0].elapsed_time(e[2]) for e in evs]))
    ms_step_mean = evs[0][0].elapsed_time(evs[-1][2]) / steps
    fwd_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    elems = kept_score_elements(mask_np, w.N, w.causal) * w.B * w.H
    fwd_f = 4.0 * w.d * elems
    bwd_f = 2.5 * fwd_f
    del dev, q, k, v, do, o, dq, dk, dv
    torch.cuda.empty_cache()
    rd = run_gpu(w, max(2, steps // 2), 1, torch, fa)
    return {
        "workload": w.name, "mask": f"local window +-{kw['window']} blocks + {kw['n_global']} global key blocks",
        "density": float(np.mean(mask_np != 0)), "tflops": (fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12,
        "ms_per_step": ms_step, "ms_per_step_mean": ms_step_mean,
        "pct_of_peak": 100.0 * (fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "fwd_tflops": fwd_f / (fwd_ms * 1e-3) / 1e12, "bwd_tflops": bwd_f / (bwd_ms * 1e-3) / 1e12,
        "dense_ms_per_step": rd["ms_per_step"],
        "roofline": _mfma_roofline((fwd_f + bwd_f) / (ms_step * 1e-3) / 1e12),
    }


def run_gpu_splitkv(name, steps, warmup, torch, fa):
    """Split-KV forward: HIP-event time per call with the automatic part count
    and with one part. Decode is bound by reading K and V (reported in GB/s of
    K, V, Q, O and LSE bytes); prefill by the matrix cores (TFLOP/s)."""
    w = SPLITKV_WORKLOADS[name]
    inp = make_cross_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed)
    dev = {k: torch.from_numpy(v[0].view(np.int16)).view(torch.bfloat16).cuda() for k, v in inp.items()}
    q, k, v = dev["q"], dev["k"], dev["v"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    res = {"workload": w.name}
    for label, ns in (("auto", fa.splitkv_num_splits(w.B, w.H, w.Nq, w.Nk, w.d)), ("one_part", 1)):
        ws = torch.empty(fa.splitkv_workspace_bytes(w.B, w.H, w.Nq, w.d, ns) // 4, dtype=torch.float32,
                         device="cuda")
        for _ in range(warmup):
            fa.forward_splitkv(q, k, v, w.causal, ns, w.scale, out=o, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fa.forward_splitkv(q, k, v, w.causal, ns, w.scale, out=o, lse=lse, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        kv_bytes = 2.0 * w.B * w.Nk * w.H * w.d * 2
        io_bytes = kv_bytes + 2.0 * (w.B * w.Nq * w.H * w.d * 2) + 4.0 * w.B * w.H * w.Nq
        elems = w.B * w.H * float(w.Nq) * w.Nk
        if w.causal:
            elems = w.B * w.H * float(sum(min(w.Nk, i + 1 + w.Nk - w.Nq) for i in range(w.Nq)))
        res[label] = {"num_splits": ns, "ms": ms, "GB/s": io_bytes / (ms * 1e-3) / 1e9,
                      "tflops": 4.0 * w.d * elems / (ms * 1e-3) / 1e12}
        del ws
    if w.Nq == 1:
        res["roofline"] = {"bound": "hbm", "achieved": res["auto"]["GB/s"], "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": res["auto"]["GB/s"] / PEAK_HBM_GBS}
    else:
        res["roofline"] = {"bound": "mfma", "achieved": res["auto"]["tflops"], "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": res["auto"]["tflops"] / PEAK_BF16_TFLOPS}
    return res


def run_gpu_fp8(cfg, steps, warmup, torch, fa):
    """Forward with FP8 scores on a fixed-length workload: HIP-event times of
    the two quantisation launches (Q per 128 rows, K per 64 rows) and of the
    forward, against the bf16 forward on the same inputs."""
    w = WORKLOADS[cfg]
    dev = _device_inputs(w, torch)
    q, k, v = dev["q"], dev["k"], dev["v"]
    q8, qs = fa.quantize_fp8(q, 128)
    k8, ks = fa.quantize_fp8(k, 64)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    fwd_f, _ = counted_flops(w.B, w.H, w.N, w.d, w.causal, False)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_quant = timed(lambda: (fa.quantize_fp8(q, 128, out=q8, scales=qs),
                              fa.quantize_fp8(k, 64, out=k8, scales=ks)))
    ms_fp8 = timed(lambda: fa.forward_fp8_quantized(q8, k8, v, qs, ks, w.causal, w.scale, out=o,
                                                    lse=lse))
    ms_bf16 = timed(lambda: fa.forward(q, k, v, w.causal, 0.0, 0, w.scale, out=o, lse=lse))
    # QK^T runs on the FP8 matrix cores (5.0 PFLOP/s dense), P V on bf16 (2.5):
    # half the counted forward FLOPs each, so the bound is 2 / (1/5 + 1/2.5).
    peak_mixed = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
    tf8 = fwd_f / (ms_fp8 * 1e-3) / 1e12
    return {"workload": w.name + "_fp8_scores_fwd", "forward_fp8_ms": ms_fp8,
            "roofline": {"bound": "mfma", "achieved": tf8, "peak": peak_mixed, "unit": "TFLOP/s",
                         "frac": tf8 / peak_mixed},
            "forward_fp8_tflops": fwd_f / (ms_fp8 * 1e-3) / 1e12, "quantize_q_k_ms": ms_quant,
            "forward_bf16_ms": ms_bf16, "forward_bf16_tflops": fwd_f / (ms_bf16 * 1e-3) / 1e12}


def kernel_source_digest():
    """SHA-256 over the attention library's sources (comments and blank lines
    removed, so that only code counts; the benchmark's clock-stamp source is
    not part of it) and the build flags: HBM traffic figures recorded under
    profiles/ are valid only for this digest."""
    import hashlib
    import re
    from exact_io_aware_72_amd import build as fa_build
    h = hashlib.sha256()
    for name in sorted(os.listdir(fa_build.CSRC)):
        if name in fa_build.CLOCK_SOURCES:
            continue
        with open(os.path.join(fa_build.CSRC, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(name.encode() + b"\0" + code.encode())
    h.update(" ".join(f for f in fa_build.COMMON_FLAGS if not f.startswith("/")).encode())
    return h.hexdigest()


def recorded_traffic(workload_name, kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) that
    profiles/hbm_traffic_*.txt records for this kernel and workload, or None
    when none is recorded or the kernels changed since it was measured."""
    import glob
    digest = kernel_source_digest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "hbm_traffic_*.txt"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("kernel="):
                    continue
                kv = dict(tok.split("=", 1) for tok in line.split())
                if kv.get("kernel") == kernel and kv.get("workload") == workload_name:
                    if kv.get("digest") != digest:
                        return None
                    return {"fetch_bytes": float(kv["fetch_bytes"]), "write_bytes": float(kv["write_bytes"]),
                            "source": os.path.relpath(path, ROOT)}
    return None


def roofline(w, kernel_ms):
    units = kernel_units(w)
    name = max(kernel_ms, key=kernel_ms.get)
    bound, work = units[name]
    sec = kernel_ms[name] * 1e-3
    if bound == "mfma":
        achieved, peak, unit = work / sec / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    elif bound == "mfma_f32":
        bound = "mfma"
        achieved, peak, unit = work / sec / 1e12, PEAK_FP32_MFMA_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = work / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    rec = recorded_traffic(w.name, name)
    return {"kernel": name, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "avg_ms": kernel_ms[name], "work_per_launch": work,
            "traffic": None if rec is None else rec["fetch_bytes"] + rec["write_bytes"],
            "traffic_detail": rec}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, seconds, gpu_out=None):
    """The fp64 oracle (as it stands) on whole heads of the same workload,
    one head at a time until about `seconds` have passed. With `gpu_out`
    (the timed run's output tensors), each head the oracle computed is also
    compared with the GPU's, element by element, outside the timed region:
    max and mean absolute error per tensor against the bar (bf16: 2e-2 and
    1e-3; fp32: 1e-5)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = None
    inp = make_inputs(w, with_grad=True)
    vals = {k: v[1] for k, v in inp.items()}
    fwd_f, bwd_f = counted_flops(1, 1, w.N, w.d, w.causal, True)
    done, el = 0, 0.0
    err = {}  # name -> [max abs, sum abs, count]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in heads:
        t0 = time.perf_counter()
        o, lse = oracle.forward(vals["q"], vals["k"], vals["v"], w.scale, w.causal, w.dropout_p,
                                w.dropout_seed, heads=[(b, h)])
        dq, dk, dv, _ = oracle.backward(vals["q"], vals["k"], vals["v"], vals["do"], w.scale, w.causal,
                                        w.dropout_p, w.dropout_seed, heads=[(b, h)], check_d=False)
        el += time.perf_counter() - t0
        done += 1
        if gpu_out is not None:
            ref = {"O": o[b, :, h], "LSE": lse[b, h], "dQ": dq[b, :, h], "dK": dk[b, :, h], "dV": dv[b, :, h]}
            for name, t in gpu_out.items():
                g = (t[b, h] if name == "LSE" else t[b, :, h]).float().cpu().numpy().astype(np.float64)
                e = np.abs(g - ref[name])
                acc = err.setdefault(name, [0.0, 0.0, 0])
                acc[0] = max(acc[0], float(e.max()))
                acc[1] += float(e.sum())
                acc[2] += e.size
        if el >= seconds:
            break
    res = {"value": done * (fwd_f + bwd_f) / el / 1e12, "unit": "TFLOP/s",
           "cores": threads, "kind": "oracle",
           "sample": f"{done} of {len(heads)} heads (full N={w.N}, fwd+bwd, fp64 numpy) in {el:.1f} s",
           "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model()}
    if gpu_out is not None:
        max_tol, mean_tol = (1e-5, None) if w.dtype == "f32" else (2e-2, 1e-3)
        per = {n: {"max_abs": a[0], "mean_abs": a[1] / a[2]} for n, a in err.items()}
        res["parity"] = {
            "heads": done, "tensors": per, "max_abs_bar": max_tol, "mean_abs_bar": mean_tol,
            "within": all(v["max_abs"] <= max_tol and (mean_tol is None or v["mean_abs"] <= mean_tol)
                          for v in per.values()),
        }
    return res

# Power and clock sampler for --power-sample: a separate process, started
# before this process touches the GPU, that reads the power cap once
# (`rocm-smi --showmaxpower`), then polls `amd-smi metric` (socket power,
# shader clock of each XCD) and appends "time power_w mean_clock_mhz" lines
# to a file until a stop file appears.
_SAMPLER = r"""
import json, os, subprocess, sys, time
out, stop = sys.argv[1], sys.argv[2]
def smi(tool, args):
    try:
        r = subprocess.run([tool] + args, capture_output=True, text=True, timeout=20)
        return json.loads(r.stdout) if r.returncode == 0 else None
    except Exception:
        return None
with open(out, "w") as f:
    cap = smi("rocm-smi", ["--showmaxpower", "--json"]) or {}
    lim = {k: float(v) for c in cap.values() if isinstance(c, dict) for k, v in c.items()
           if "power" in k.lower() and v.replace(".", "", 1).isdigit()}
    f.write("#limits " + json.dumps(lim) + "\n")
    f.flush()
    while not os.path.exists(stop):
        t = time.time()
        m = smi("amd-smi", ["metric", "-g", "0", "-p", "-c", "--json"])
        try:
            g = m["gpu_data"][0]
            pw = float(g["power"]["socket_power"]["value"])
            clk = [float(v["clk"]["value"]) for k, v in g["clock"].items() if k.startswith("gfx_")]
            f.write(f"{(t + time.time()) / 2:.3f} {pw:.1f} {sum(clk) / len(clk):.1f}\n")
            f.flush()
        except Exception:
            time.sleep(0.5)
        time.sleep(0.05)
"""


def power_sample_leg(seconds, sampler, torch, fa):
    """Socket power and shader clock (amd-smi, sampled by a separate
    process) while the headline step runs back to back for `seconds` on its
    random inputs and then on constant inputs (every element of Q, K, V and
    dO equal to 1), after an idle interval. Returns one dict per phase."""
    proc, out, stop = sampler
    t_wait = time.time()
    while time.time() - t_wait < 60:  # first sample (amd-smi starts slowly)
        with open(out) as f:
            if any(not ln.startswith("#") for ln in f):
                break
        time.sleep(0.2)
    w = WORKLOADS[3]
    dev = _device_inputs(w, torch)
    ones = {k: torch.ones_like(v) for k, v in dev.items()}
    o = torch.empty_like(dev["q"])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(dev["q"]) for _ in range(3))
    args = (w.causal, w.dropout_p, w.dropout_seed, w.scale)
    fwd_f, bwd_f = counted_flops(w.B, w.H, w.N, w.d, w.causal, True)

    def step(x):
        fa.forward(x["q"], x["k"], x["v"], *args, out=o, lse=lse)
        fa.backward(x["q"], x["k"], x["v"], o, x["do"], lse, *args, dq=dq, dk=dk, dv=dv)

    phases = []
    try:
        torch.cuda.synchronize()
        t0 = time.time()
        time.sleep(min(5.0, seconds / 2))
        phases.append({"phase": "idle", "t0": t0, "t1": time.time(), "steps": 0})
        for name, x in (("random inputs", dev), ("constant inputs", ones)):
            for _ in range(20):
                step(x)
            torch.cuda.synchronize()
            t0 = time.time()
            n = 0
            while time.time() - t0 < seconds:
                for _ in range(50):
                    step(x)
                torch.cuda.synchronize()
                n += 50
            t1 = time.time()
            # forward and backward separately: event-timed medians over 20
            # more steps, right after the timed window (same clock regime)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(20)]
            for e in ev:
                e[0].record()
                fa.forward(x["q"], x["k"], x["v"], *args, out=o, lse=lse)
                e[1].record()
                fa.backward(x["q"], x["k"], x["v"], o, x["do"], lse, *args, dq=dq, dk=dk, dv=dv)
                e[2].record()
            torch.cuda.synchronize()
            fms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
            bms = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
            print(f"power leg: {name}: {n} steps in {t1 - t0:.1f} s", file=sys.stderr, flush=True)
            phases.append({"phase": name, "t0": t0, "t1": t1, "steps": n, "fwd_ms": fms, "bwd_ms": bms})
    finally:
        # the sampler always stops, also when the GPU work raised
        with open(stop, "w"):
            pass
        try:
            proc.wait(timeout=60)
        except Exception:
            proc.kill()
            proc.wait()
    limits, samples = {}, []
    with open(out) as f:
        for ln in f:
            if ln.startswith("#limits "):
                limits = json.loads(ln[len("#limits "):])
            elif ln.strip():
                t, pw, clk = (float(x) for x in ln.split())
                samples.append((t, pw, clk))
    res = []
    for ph in phases:
        # skip the first second of each phase (clock and power settle)
        sel = [(pw, clk) for t, pw, clk in samples if ph["t0"] + 1.0 <= t <= ph["t1"]]
        d = {"phase": ph["phase"], "seconds": round(ph["t1"] - ph["t0"], 2), "samples": len(sel),
             "socket_power_w": float(np.median([p for p, _ in sel])) if sel else None,
             "gfx_clock_mhz": float(np.median([c for _, c in sel])) if sel else None}
        if ph["steps"]:
            ms = (ph["t1"] - ph["t0"]) * 1e3 / ph["steps"]
            d.update({"steps": ph["steps"], "ms_per_step": ms, "tflops": (fwd_f + bwd_f) / (ms * 1e-3) / 1e12,
                      "fwd_ms": ph["fwd_ms"], "fwd_tflops": fwd_f / (ph["fwd_ms"] * 1e-3) / 1e12,
                      "bwd_ms": ph["bwd_ms"], "bwd_tflops": bwd_f / (ph["bwd_ms"] * 1e-3) / 1e12})
        res.append(d)
    return {"power_sample": {"workload": w.name, "phases": res, "power_limits_w": limits,
                             "source": "amd-smi metric (socket power, mean GFX clock over the XCDs), "
                                       "medians over each phase after its first second"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--also", type=int, nargs="*", default=[4, 1, 2, 5])
    ap.add_argument("--also-varlen", nargs="*", default=["varlen16"])
    ap.add_argument("--also-sparse", nargs="*", default=["local_global"])
    ap.add_argument("--also-splitkv", nargs="*", default=["decode", "prefill_small"])
    ap.add_argument("--also-fp8", type=int, nargs="*", default=[3])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB mebibytes (three times), "
                         "the reference kernel for scaling HBM traffic counters, and exit")
    ap.add_argument("--power-sample", type=float, default=0.0, metavar="SECONDS",
                    help="only run the headline step back to back for SECONDS on random and then on "
                         "constant inputs while a separate process samples socket power and shader "
                         "clock with amd-smi, print one JSON line, and exit")
    a = ap.parse_args()
    sampler = None
    if a.power_sample:
        # Started before anything here touches the GPU.
        import subprocess
        import tempfile
        tmp = tempfile.mkdtemp(prefix="fa_power_")
        out, stop = os.path.join(tmp, "samples.txt"), os.path.join(tmp, "stop")
        open(out, "w").close()
        sampler = (subprocess.Popen([sys.executable, "-c", _SAMPLER, out, stop]), out, stop)

        def _stop_sampler(proc=sampler[0], stop=stop):
            if proc.poll() is None:
                open(stop, "w").close()
                try:
                    proc.wait(timeout=60)
                except Exception:
                    proc.kill()
                    proc.wait()

        import atexit
        atexit.register(_stop_sampler)  # also on early exits (no GPU, library missing)
    if a.gpus != 1:
        print("bench.py measures one GPU: the attention kernels run on a single device and this build "
              "has no multi-GPU path (heads or sequence chunks would be sharded across GPUs); "
              "run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_io_aware_72_amd as fa

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    fa.lib()  # fails loudly if the HIP library is missing

    if sampler is not None:
        print(json.dumps(power_sample_leg(a.power_sample, sampler, torch, fa)), flush=True)
        return

    if a.copy_calibration:
        n = a.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return

    w = WORKLOADS[a.workload]
    r = run_gpu(w, a.steps, a.warmup, torch, fa, keep_outputs=not a.no_cpu_baseline, sample_clock=True)
    line = {
        "metric": METRIC,
        "value": r["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": r["ms_per_step"],
        "ms_per_step_mean": r["ms_per_step_mean"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "dropout_p": w.dropout_p, "global_batch": w.B, "seq_len": w.N,
                   "parallelism": "single-gpu"},
        "pct_of_peak": 100.0 * r["tflops"] / PEAK_BF16_TFLOPS,
        "fwd_ms": r["fwd_ms"], "bwd_ms": r["bwd_ms"],
        "fwd_tflops": r["fwd_tflops"], "bwd_tflops": r["bwd_tflops"],
        "kernel_ms": r["kernel_ms"],
        "kernel_ms_median": r["kernel_ms_median"],
        "clock": r["clock"],
        "roofline": roofline(w, r["kernel_ms"]),
    }
    also = []
    for cfg in a.also:
        wa = WORKLOADS[cfg]
        ra = run_gpu(wa, max(3, a.steps // 4) if wa.backward else a.steps, 2, torch, fa, sample_clock=True)
        peak = PEAK_FP32_MFMA_TFLOPS if wa.dtype == "f32" else PEAK_BF16_TFLOPS
        also.append({"workload": wa.name, "dtype": wa.dtype, "passes": "fwd+bwd" if wa.backward else "fwd",
                     "tflops": ra["tflops"], "ms_per_step": ra["ms_per_step"],
                     "pct_of_peak": 100.0 * ra["tflops"] / peak,
                     "fwd_tflops": ra["fwd_tflops"], "bwd_tflops": ra["bwd_tflops"],
                     "kernel_ms": ra["kernel_ms"], "clock": ra["clock"],
                     "roofline": roofline(wa, ra["kernel_ms"])})
        torch.cuda.empty_cache()
    for name in a.also_varlen:
        also.append(run_gpu_varlen(VARLEN_WORKLOADS[name], max(3, a.steps // 4), 2, torch, fa))
        torch.cuda.empty_cache()
    for name in a.also_sparse:
        also.append(run_gpu_sparse(name, max(3, a.steps // 4), 2, torch, fa))
        torch.cuda.empty_cache()
    for name in a.also_splitkv:
        also.append(run_gpu_splitkv(name, max(5, a.steps), 3, torch, fa))
        torch.cuda.empty_cache()
    for cfg in a.also_fp8:
        also.append(run_gpu_fp8(cfg, max(5, a.steps // 2), 2, torch, fa))
        torch.cuda.empty_cache()
    line["also"] = also
    line["cpu_baseline"] = None if a.no_cpu_baseline else cpu_baseline(w, a.cpu_seconds, r["outputs"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
