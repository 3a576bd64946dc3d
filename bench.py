#!/usr/bin/env python
"""Weight-stream benchmark of the block-quantized decode GEMV on one MI355X.

Default workload: Q4_K fused gate+up decode GEMV of Qwen3.8-27B's MLP
(M = 1, N = 2 x 17,408, K = 5,120; 100,270,080 packed weight bytes per call),
synthetic seeded weights and activations already resident in HBM.  A step is one
call of the hot path (quant_gemv).  The weights are rotated over enough distinct
copies (>= 1 GiB in total) that every call streams from HBM, not from the
256 MB Infinity Cache.

Printed: one JSON line with the weight-stream rate (GB/s of packed weight bytes),
the kernel's roofline position against MI355X's 8 TB/s HBM peak and against a
plain streaming read of 1 GiB on the same box, and the CPU oracle timed on a
bounded sample of the same workload.  --all adds every workload shape (the
parity configurations) as a "sweep" list; launch-bound shapes also report the
rate of their rotated calls replayed from one HIP graph.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
TOKEN_BYTES_GB = 16.39         # per-token weight read of the 27B Q4_K_M artifact, embedding gather excluded
ROTATE_BYTES = 1 << 30
LAUNCH_BOUND_BYTES = 16 << 20  # below this a call is dominated by launch latency
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")
COPY_ELEMS = 64 << 20  # fp32 elements of the calibration copy: 256 MiB read, 256 MiB written


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Workload:
    def __init__(self, name, fmt, N, K, M, seed, E=1, moe=None, block=None):
        self.name, self.fmt, self.N, self.K, self.M, self.seed, self.E = name, fmt, N, K, M, seed, E
        self.moe = moe  # (tokens, topk) for the grouped workload
        self.block = block  # (down format, F, tokens, topk) for the MoE block: N = 2F, K = D


def workloads():
    import gemm_block_quant_amd as qg
    return {
        "q8_0_1024": Workload("Q8_0 GEMV 1024x1024", qg.Q8_0, 1024, 1024, 1, 1),
        "q4k_gateup": Workload("Q4_K fused gate+up GEMV, N=34816 K=5120", qg.Q4_K, 2 * 17408, 5120, 1, 2),
        "q4k_gateup_m8": Workload("Q4_K fused gate+up, N=34816 K=5120", qg.Q4_K, 2 * 17408, 5120, 8, 2),
        "q4k_gateup_m512": Workload("Q4_K fused gate+up prefill, N=34816 K=5120", qg.Q4_K, 2 * 17408, 5120, 512, 2),
        "q5k_gateup": Workload("Q5_K fused gate+up GEMV, N=34816 K=5120", qg.Q5_K, 2 * 17408, 5120, 1, 6),
        "q5k_gateup_m8": Workload("Q5_K fused gate+up, N=34816 K=5120", qg.Q5_K, 2 * 17408, 5120, 8, 6),
        "q5k_gateup_m512": Workload("Q5_K fused gate+up prefill, N=34816 K=5120", qg.Q5_K, 2 * 17408, 5120, 512,
                                    6),
        "q6k_down_m1": Workload("Q6_K down-proj, N=5120 K=17408", qg.Q6_K, 5120, 17408, 1, 3),
        "q6k_down_m8": Workload("Q6_K down-proj, N=5120 K=17408", qg.Q6_K, 5120, 17408, 8, 3),
        "q6k_down_m512": Workload("Q6_K down-proj prefill, N=5120 K=17408", qg.Q6_K, 5120, 17408, 512, 3),
        "q6k_head_m1": Workload("Q6_K LM head, N=248320 K=5120", qg.Q6_K, 248320, 5120, 1, 3),
        "q6k_head_m8": Workload("Q6_K LM head, N=248320 K=5120", qg.Q6_K, 248320, 5120, 8, 3),
        "nvfp4_up_m1": Workload("NVFP4 MLP, N=17408 K=5120", qg.NVFP4, 17408, 5120, 1, 4),
        "nvfp4_up_m8": Workload("NVFP4 MLP, N=17408 K=5120", qg.NVFP4, 17408, 5120, 8, 4),
        "nvfp4_up_m512": Workload("NVFP4 MLP prefill, N=17408 K=5120", qg.NVFP4, 17408, 5120, 512, 4),
        "nvfp4_down_m1": Workload("NVFP4 MLP, N=5120 K=17408", qg.NVFP4, 5120, 17408, 1, 4),
        "nvfp4_down_m8": Workload("NVFP4 MLP, N=5120 K=17408", qg.NVFP4, 5120, 17408, 8, 4),
        "nvfp4_down_m512": Workload("NVFP4 MLP prefill, N=5120 K=17408", qg.NVFP4, 5120, 17408, 512, 4),
        "fp8_gateup": Workload("row-scaled FP8 fused gate+up GEMV, N=34816 K=5120", qg.FP8, 2 * 17408, 5120, 1, 7),
        "fp8_gateup_m8": Workload("row-scaled FP8 fused gate+up, N=34816 K=5120", qg.FP8, 2 * 17408, 5120, 8, 7),
        "fp8_gateup_m512": Workload("row-scaled FP8 fused gate+up prefill, N=34816 K=5120", qg.FP8, 2 * 17408, 5120,
                                    512, 7),
        "fp8_head_m1": Workload("row-scaled FP8 LM head, N=248320 K=5120", qg.FP8, 248320, 5120, 1, 7),
        "fp8_head_m8": Workload("row-scaled FP8 LM head, N=248320 K=5120", qg.FP8, 248320, 5120, 8, 7),
        "moe_gate": Workload("Q4_K grouped experts gate, E=288 N=2048 K=4096", qg.Q4_K, 2048, 4096, 128, 5, E=288,
                             moe=(16, 8)),
        "moe_down": Workload("Q4_K grouped experts down, E=288 N=4096 K=2048", qg.Q4_K, 4096, 2048, 128, 5, E=288,
                             moe=(16, 8)),
        "moe_block": Workload("Q4_K MoE block (gate|up, SwiGLU, down, combine), E=288 D=4096 F=2048, 16 tokens x "
                              "top-8", qg.Q4_K, 2 * 2048, 4096, 128, 5, E=288, block=(qg.Q4_K, 2048, 16, 8)),
    }


class Prepared:
    """Device buffers and a raw launcher for one workload."""

    def __init__(self, wl: Workload, rotate: bool = True):
        import torch

        import gemm_block_quant_amd as qg
        import synth
        self.wl = wl
        if wl.block is not None:
            self._prepare_block(wl)
            return
        tid_w = 0 if wl.moe is None or wl.K == 4096 else 4
        t0 = time.time()
        self.w_host = synth.weights(wl.fmt, synth.rng(wl.seed, tid_w), wl.E * wl.N, wl.K, E=wl.E)
        self.x_host = synth.x_bf16(synth.rng(wl.seed, 1 if wl.moe is None or wl.K == 4096 else 3), wl.M, wl.K)
        self.ids_host = synth.routing(synth.rng(wl.seed, 2), wl.moe[0], wl.moe[1], wl.E) if wl.moe else None
        self.wbytes_total = qg.quant_packed_bytes(wl.fmt, wl.E, wl.N, wl.K)
        log("[bench] %s: generated %.1f MB in %.1f s" % (wl.name, self.wbytes_total / 1e6, time.time() - t0))
        w0 = torch.from_numpy(self.w_host).cuda()
        if wl.moe is None:
            self.copies = max(1, -(-ROTATE_BYTES // self.wbytes_total)) if rotate else 1
            self.w = [w0] + [w0.clone() for _ in range(self.copies - 1)]
            self.bytes_per_call = self.wbytes_total
            self.distinct = 1
        else:
            self.copies = 1
            self.w = [w0]
            self.distinct = len(np.unique(self.ids_host))
            self.bytes_per_call = self.distinct * qg.quant_packed_bytes(wl.fmt, 1, wl.N, wl.K)
        self.x = torch.from_numpy(self.x_host.view(np.int16)).cuda()
        self.y = torch.empty((wl.M, wl.N), dtype=torch.float32, device="cuda")
        self.ids = torch.from_numpy(self.ids_host).cuda() if self.ids_host is not None else None
        self.ws = None
        L = qg.lib()
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        xp, yp = ctypes.c_void_p(self.x.data_ptr()), ctypes.c_void_p(self.y.data_ptr())
        wps = [ctypes.c_void_p(t.data_ptr()) for t in self.w]
        fmt, N, K, M, E = wl.fmt, wl.N, wl.K, wl.M, wl.E
        if wl.moe is not None:
            wsb = qg.quant_grouped_workspace_bytes(E, M)
            self.ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            ip, wsp = ctypes.c_void_p(self.ids.data_ptr()), ctypes.c_void_p(self.ws.data_ptr())
            fn = L.quant_grouped_gemm
            self.calls = [lambda s, wp=wp: fn(wp, fmt, E, N, K, M, xp, ip, yp, wsp, wsb, s) for wp in wps]
        elif M == 1:
            fn = L.quant_gemv
            self.calls = [lambda s, wp=wp: fn(wp, fmt, N, K, xp, yp, s) for wp in wps]
        else:
            fn = L.quant_gemm
            self.calls = [lambda s, wp=wp: fn(wp, fmt, N, K, M, xp, yp, s) for wp in wps]

    def _prepare_block(self, wl: Workload):
        """The MoE block: gate|up weight[E*2F, D], down weight[E*D, F].  Only the
        first 32 experts are drawn; experts e >= 32 repeat expert e % 32's bytes
        (same shapes and value distribution, distinct addresses), which keeps
        generation of the 4 GB layer to a fraction of a minute."""
        import torch

        import gemm_block_quant_amd as qg
        import synth
        fmt_dn, F, T, topk = wl.block
        D, E, base = wl.K, wl.E, min(wl.E, 32)
        assert wl.fmt != qg.NVFP4 and fmt_dn != qg.NVFP4, "the tiled generator needs self-contained blocks"
        t0 = time.time()
        reps = -(-E // base)
        gu = synth.weights(wl.fmt, synth.rng(wl.seed, 10), base * 2 * F, D)
        dn = synth.weights(fmt_dn, synth.rng(wl.seed, 11), base * D, F)
        self.w_gu = torch.from_numpy(gu).cuda().repeat(reps)[:qg.quant_packed_bytes(wl.fmt, E, 2 * F, D)].contiguous()
        self.w_dn = torch.from_numpy(dn).cuda().repeat(reps)[:qg.quant_packed_bytes(fmt_dn, E, D, F)].contiguous()
        self.x_host = synth.x_bf16(synth.rng(wl.seed, 12), T, D)
        self.idx_host = synth.routing(synth.rng(wl.seed, 13), T, topk, E).reshape(T, topk)
        self.wts_host = synth.routing_weights(synth.rng(wl.seed, 14), T, topk)
        self.distinct = len(np.unique(self.idx_host))
        self.bytes_per_call = self.distinct * (qg.quant_packed_bytes(wl.fmt, 1, 2 * F, D) +
                                               qg.quant_packed_bytes(fmt_dn, 1, D, F))
        self.wbytes_total = self.w_gu.numel() + self.w_dn.numel()
        log("[bench] %s: generated and placed %.1f MB in %.1f s" % (wl.name, self.wbytes_total / 1e6,
                                                                      time.time() - t0))
        self.copies = 1
        self.x = torch.from_numpy(self.x_host.view(np.int16)).cuda()
        self.idx = torch.from_numpy(self.idx_host).cuda()
        self.wts = torch.from_numpy(self.wts_host).cuda()
        self.y = torch.empty((T, D), dtype=torch.float32, device="cuda")
        wsb = qg.quant_moe_workspace_bytes(wl.fmt, fmt_dn, E, D, F, T, topk)
        self.ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        L = qg.lib()
        vp = lambda t: ctypes.c_void_p(t.data_ptr())
        args = (vp(self.w_gu), wl.fmt, vp(self.w_dn), fmt_dn, E, D, F, T, topk, vp(self.x), vp(self.idx),
                vp(self.wts), vp(self.y), vp(self.ws), wsb)
        self.calls = [lambda s: L.quant_moe_block(*args, s)]

    def call(self, i, stream=None):
        st = self.calls[i % len(self.calls)](self.stream if stream is None else stream)
        if st != 0:
            import gemm_block_quant_amd as qg
            raise qg.QuantGemmError(st, "bench launch")


def time_workload(p: Prepared, steps: int, warmup: int):
    """Two timed regions of `steps` calls on the launch stream (torch's current stream).

    The first has events only at its two ends: the whole-job time.  The second
    brackets every launch with its own event pair: the mean and median launch
    duration of the kernel(s) of one call.  (Events between launches add a few
    microseconds per call, so they stay out of the first region.)"""
    import torch
    for i in range(warmup):
        p.call(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(steps):
        p.call(i)
    t_end.record()
    torch.cuda.synchronize()
    total = t_start.elapsed_time(t_end) / 1e3
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        p.call(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) / 1e3 for a, b in ev]
    return total, float(np.mean(per)), float(np.median(per))


def graph_time(p: Prepared, reps: int = 5):
    """A launch-bound workload: one call per rotated weight copy captured in one
    HIP graph (torch's CUDAGraph), replayed `reps` times; seconds per call (the
    median replay)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st = ctypes.c_void_p(side.cuda_stream)
        for i in range(len(p.calls)):
            p.call(i, st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(len(p.calls)):
            p.call(i, st)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / 1e3 / len(p.calls))
    return float(np.median(times))


def achievable_read_gbs(reps: int = 5):
    """The plain streaming-read reference: quant_read_probe over 1 GiB (each
    16-byte granule read once, non-temporal loads, nothing written); GB/s of the
    median of `reps` runs."""
    import torch
    import gemm_block_quant_amd as qg
    t = torch.ones(ROTATE_BYTES // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    qg.quant_read_probe(t, sink)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        qg.quant_read_probe(t, sink)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / 1e3)
    del t
    torch.cuda.empty_cache()
    return ROTATE_BYTES / float(np.median(times)) / 1e9


def kernel_source_hash() -> str:
    """Hash of the HIP sources: HBM-traffic figures taken from counters are only
    reported while the kernels they were taken on are unchanged."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "gemm_block_quant_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(key: str):
    """Calibrated HBM bytes per call (fetched + written) from profiles/traffic.json, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)[key]
    except (OSError, KeyError, ValueError):
        return None
    if d.get("source_hash") != kernel_source_hash():
        return None
    return int(d["fetch_bytes"] + d["write_bytes"])


def copy_calibration():
    """A plain elementwise pass of known traffic (torch.neg over 256 MiB of fp32,
    into a second 256 MiB buffer), five times: the reference the FETCH_SIZE /
    WRITE_SIZE counters are scaled by."""
    import torch
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def _counter_means(out_dir: str, counter: str):
    """{kernel name: mean counter value per dispatch} from rocprofv3 counter CSVs under out_dir."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] == counter:
                    vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def pmc_summary(fetch_dir: str, write_dir: str, key: str, fetch_cmd: str, write_cmd: str):
    """Turn a FETCH_SIZE run and a WRITE_SIZE run (each over bench.py --calibrate-copy)
    into calibrated bytes per call, stored under `key` in profiles/traffic.json."""
    out = {"source_hash": kernel_source_hash(), "fetch_command": fetch_cmd, "write_command": write_cmd,
           "copy_bytes_each_way": COPY_ELEMS * 4}
    for name, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        means = _counter_means(d, counter)
        # the product kernels of one call (not the streaming-read reference)
        ours = {k: v for k, v in means.items() if "qg::" in k and "k_read_probe" not in k}
        copy = [v for k, v in means.items() if "neg" in k.lower() and "qg::" not in k]
        if not ours or not copy:
            raise SystemExit("pmc summary: no %s rows for %s in %s" % (counter, "our kernels" if not ours else "the copy", d))
        factor = COPY_ELEMS * 4 / (copy[0] * 1024)
        per_call_kib = sum(ours.values())
        out[name + "_kib_per_call_raw"] = round(per_call_kib, 3)
        out[name + "_copy_kib_raw"] = round(copy[0], 3)
        out[name + "_factor"] = round(factor, 5)
        out[name + "_bytes"] = int(round(per_call_kib * 1024 * factor))
        out[name + "_kernels"] = {k: round(v, 3) for k, v in ours.items()}
    try:
        with open(TRAFFIC_FILE) as f:
            allt = json.load(f)
    except (OSError, ValueError):
        allt = {}
    allt[key] = out
    os.makedirs(PROFILES, exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(allt, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out))


def cpu_baseline(p: Prepared, target_s: float = 12.0):
    """The oracle (as it stands) on a bounded sample of the same workload: the first
    output rows, doubling until one pass takes about target_s; when the whole
    matrix takes less, whole passes are repeated until target_s has elapsed."""
    import oracle
    wl = p.wl
    nthreads = oracle.max_threads()
    ids = p.ids_host if wl.moe else None
    rows_try = 64
    while True:
        cols = np.arange(min(rows_try, wl.N))
        t0 = time.time()
        oracle.gemm(wl.fmt, p.w_host, wl.N, wl.K, p.x_host, E=wl.E, cols=cols, ids=ids)
        dt = time.time() - t0
        if dt >= target_s or rows_try >= wl.N:
            break
        rows_try = int(min(wl.N, max(rows_try * 2, rows_try * target_s / max(dt, 1e-3) * 1.05)))
    passes = 1
    if dt < target_s:
        t0 = time.time()
        passes = 0
        while time.time() - t0 < target_s:
            oracle.gemm(wl.fmt, p.w_host, wl.N, wl.K, p.x_host, E=wl.E, cols=cols, ids=ids)
            passes += 1
        dt = time.time() - t0
    # the workload's weight bytes in proportion to the outputs computed (same unit as the GPU figure)
    pass_bytes = p.bytes_per_call * len(cols) / wl.N
    return {"value": round(pass_bytes * passes / dt / 1e9, 4), "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": "%d of %d output rows x M=%d (%.1f MB of packed weights per pass), %d pass(es) in %.2f s, "
                      "%d threads" % (len(cols), wl.N, wl.M, pass_bytes / 1e6, passes, dt, nthreads)}


def result_for(p: Prepared, steps: int, warmup: int):
    total, per_mean, per_med = time_workload(p, steps, warmup)
    wl = p.wl
    gbs = p.bytes_per_call * steps / total / 1e9
    kern_gbs = p.bytes_per_call / per_mean / 1e9
    r = {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K, "E": wl.E,
         "weight_bytes_per_call": p.bytes_per_call, "rotated_copies": p.copies,
         "ms_per_call": round(total / steps * 1e3, 5), "kernel_ms_mean": round(per_mean * 1e3, 5),
         "kernel_ms_median": round(per_med * 1e3, 5),
         "weight_GBps": round(gbs, 1), "kernel_weight_GBps": round(kern_gbs, 1),
         "pct_hbm_peak": round(100 * kern_gbs / HBM_PEAK_GBS, 2),
         "implied_tok_s": round(wl.M * gbs / TOKEN_BYTES_GB, 1)}
    if wl.moe or wl.block:
        r["distinct_experts"] = p.distinct
    if wl.M >= 32 and not wl.block:
        flops = 2.0 * wl.M * wl.N * wl.K
        r["TFLOPs"] = round(flops / per_mean / 1e12, 1)
        r["pct_bf16_mfma_peak"] = round(100 * flops / per_mean / 1e12 / BF16_MFMA_PEAK_TFLOPS, 2)
    if p.bytes_per_call < LAUNCH_BOUND_BYTES:
        # launch-bound: the rotated calls replayed from one graph
        gt = graph_time(p)
        r["graph_ms_per_call"] = round(gt * 1e3, 5)
        r["graph_weight_GBps"] = round(p.bytes_per_call / gt / 1e9, 1)
    return r, total, per_mean


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="q4k_gateup")
    ap.add_argument("--all", action="store_true", help="also time every workload shape (sweep)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sweep-out", default=None, help="write the sweep as JSON lines to this file")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed regions, run the known-size copy the HBM counters are scaled by")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="summarize two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/traffic.json")
    ap.add_argument("--pmc-commands", nargs=2, default=("", ""), help="the two commands, recorded with the summary")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload, *args.pmc_commands)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import gemm_block_quant_amd as qg
    qg.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wls = workloads()
    wl = wls[args.workload]
    achievable = achievable_read_gbs()
    log("[bench] plain streaming read of 1 GiB (quant_read_probe): %.1f GB/s" % achievable)
    p = Prepared(wl)
    torch.cuda.synchronize()
    r, total, per_mean = result_for(p, args.steps, args.warmup)
    r["pct_of_achievable"] = round(100 * r["weight_GBps"] / achievable, 2)
    log("[bench] %s" % json.dumps(r))
    sweep = []
    if args.all:
        for key, w2 in wls.items():
            if key == args.workload:
                sweep.append(r)
                continue
            try:
                p2 = Prepared(w2)
                steps = max(10, min(args.steps, int(2.0 / max(1e-6, p2.bytes_per_call / 5e12))))
                r2, _, _ = result_for(p2, steps, min(args.warmup, steps))
                r2["pct_of_achievable"] = round(100 * r2["weight_GBps"] / achievable, 2)
            except Exception as e:  # a workload the build cannot run yet is reported, not fatal
                r2 = {"workload": w2.name, "M": w2.M, "error": str(e)}
            log("[bench] %s" % json.dumps(r2))
            sweep.append(r2)
            del p2
            torch.cuda.empty_cache()
        if args.sweep_out:
            with open(args.sweep_out, "w") as f:
                for s in sweep:
                    f.write(json.dumps(s) + "\n")
    if args.calibrate_copy:
        copy_calibration()
    cpu = None
    if not args.no_cpu and not wl.block:
        cpu = cpu_baseline(p)
        log("[bench] cpu baseline %s" % json.dumps(cpu))
    value = p.bytes_per_call * args.steps / total / 1e9
    # the step is one launch of the product kernel: its average duration over the
    # timed region (events on the launch stream at the region's two ends)
    achieved = p.bytes_per_call / (total / args.steps) / 1e9
    out = {
        "metric": "weight-stream HBM GB/s and % of MI355X peak for quantized decode GEMV (M=1,8)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "format": {v: k for k, v in qg.FORMATS.items()}[wl.fmt], "M": wl.M,
                   "N": wl.N, "K": wl.K, "weight_bytes": p.bytes_per_call, "rotated_copies": p.copies,
                   "implied_tok_s": r["implied_tok_s"],
                   "ms_per_launch_with_per_launch_events": round(per_mean * 1e3, 5),
                   "achievable_read_GBps": round(achievable, 1),
                   "pct_of_achievable": round(100 * achieved / achievable, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(args.workload)},
        "cpu_baseline": cpu,
    }
    if sweep:
        out["sweep"] = sweep
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
