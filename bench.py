#!/usr/bin/env python
"""Weight-stream benchmark of the block-quantized decode GEMV on one MI355X.

Headline workload: Q4_K fused gate+up decode GEMV of Qwen3.8-27B's MLP
(M = 1, N = 2 x 17,408, K = 5,120; 100,270,080 packed weight bytes per call),
synthetic seeded weights and activations already resident in HBM.  A step is one
call of the hot path (quant_gemv).  The weights are rotated over enough distinct
copies (>= 1 GiB in total) that every call streams from HBM, not from the
256 MB Infinity Cache.

Printed: one JSON line with the headline's weight-stream rate (GB/s of packed
weight bytes), its roofline position against MI355X's 8 TB/s HBM peak, and a
"configs" list with every workload configuration of the method, each timed the
same way: Q8_0 1024 x 1024; Q4_K gate+up; Q6_K down projection and LM head at
M = 1 and 8; NVFP4 MLP shapes at M = 1, 8 and 512; the Q4_K 288-expert MoE layer
(gate, up, down grouped products over 16 tokens x top-8).  Each reports weight
GB/s, % of 8 TB/s, % of a plain streaming read of the same byte count (a
size-matched achievable ceiling), implied tokens/s, matrix-core TFLOP/s for
M = 512 and the HBM traffic measured by counters.  GPU clocks are read before,
under load and after; the CPU oracle is timed on a bounded sample, on all host
threads and on one.  --all adds the remaining workload shapes as a "sweep".
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
GRAPH_BYTES = 16 << 20  # below this a call is launch-bound: also timed replayed from a HIP graph
WARM_S = 0.1  # untimed back-to-back calls before each timed region, so the clocks have ramped up
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")
COPY_ELEMS = 64 << 20  # fp32 elements of the calibration copy: 256 MiB read, 256 MiB written


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Workload:
    def __init__(self, name, fmt, N, K, M, seed, E=1, moe=None, block=None, layer=False):
        self.name, self.fmt, self.N, self.K, self.M, self.seed, self.E = name, fmt, N, K, M, seed, E
        self.moe = moe  # (tokens, topk) for the grouped workload
        self.block = block  # (down format, F, tokens, topk) for the MoE block: N = 2F, K = D
        self.layer = layer  # grouped gate [E*N, K], up [E*N, K] and down [E*K, N] products per step


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
        "moe_prefill": Workload("Q4_K grouped experts prefill, E=8 N=2048 K=4096, 4096 tokens x top-4 "
                                "(about 2,048 rows per expert)", qg.Q4_K, 2048, 4096, 16384, 8, E=8, moe=(4096, 4)),
        "moe_block": Workload("Q4_K MoE block (gate|up, SwiGLU, down, combine), E=288 D=4096 F=2048, 16 tokens x "
                              "top-8", qg.Q4_K, 2 * 2048, 4096, 128, 5, E=288, block=(qg.Q4_K, 2048, 16, 8)),
        "moe_layer": Workload("Q4_K grouped MoE layer (gate, up, down products), E=288 experts of 4096x2048, "
                              "16 tokens x top-8", qg.Q4_K, 2048, 4096, 128, 5, E=288, moe=(16, 8), layer=True),
    }


# The workload configurations of the method, in order: (config id, workload key).
CONFIGS = [("1", "q8_0_1024"), ("2", "q4k_gateup"),
           ("3", "q6k_down_m1"), ("3", "q6k_down_m8"), ("3", "q6k_head_m1"), ("3", "q6k_head_m8"),
           ("4", "nvfp4_up_m1"), ("4", "nvfp4_up_m8"), ("4", "nvfp4_up_m512"),
           ("4", "nvfp4_down_m1"), ("4", "nvfp4_down_m8"), ("4", "nvfp4_down_m512"),
           ("5", "moe_layer")]
HEADLINE = "q4k_gateup"
LAYER_ROUTINGS = 8  # routing draws cycled by the MoE-layer workload


class Prepared:
    """Device buffers and a raw launcher for one workload."""

    def __init__(self, wl: Workload, rotate: bool = True):
        import torch

        import gemm_block_quant_amd as qg
        import synth
        self.wl = wl
        self.entry = None  # the entry point timed, where it is not the workload's usual one
        self.call_bytes = None  # bytes of call i (cycled), when calls differ
        if wl.block is not None:
            self._prepare_block(wl)
            return
        if wl.layer:
            self._prepare_layer(wl)
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
            # the 5120-row down projections at 512 rows leave resident workgroups
            # idle on the plain tile grid: the stream-K entry deals their work
            # evenly (quant_gemm_streamk is quant_gemm where it needs no workspace)
            wsb = qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, M)
            if wsb > 0:
                self.entry = "quant_gemm_streamk"
                self.ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
                wsp = ctypes.c_void_p(self.ws.data_ptr())
                fn = L.quant_gemm_streamk
                self.calls = [lambda s, wp=wp: fn(wp, fmt, N, K, M, xp, yp, wsp, wsb, s) for wp in wps]
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

    def _prepare_layer(self, wl: Workload):
        """The MoE layer: gate and up weight[E*N, K], down weight[E*K, N] (Q4_K), 16
        tokens routed to 8 distinct experts each (M = 128 rows), three grouped
        calls per step.  The routing cycles over LAYER_ROUTINGS draws so that
        consecutive steps read different expert sets from the 4 GB tower.  As for
        the MoE block, the first 32 experts are drawn and repeated for the others
        (same distributions, distinct addresses)."""
        import torch

        import gemm_block_quant_amd as qg
        import synth
        E, N, K, M = wl.E, wl.N, wl.K, wl.M
        tokens, topk = wl.moe
        base = min(E, 32)
        reps = -(-E // base)
        t0 = time.time()
        mats = []
        for tid, (rows, cols) in enumerate(((N, K), (N, K), (K, N))):
            hw = synth.weights(wl.fmt, synth.rng(wl.seed, 20 + tid), base * rows, cols)
            mats.append(torch.from_numpy(hw).cuda().repeat(reps)[:qg.quant_packed_bytes(wl.fmt, E, rows,
                                                                                          cols)].contiguous())
        self.w_gate, self.w_up, self.w_down = mats
        self.wbytes_total = sum(m.numel() for m in mats)
        self.x = torch.from_numpy(synth.x_bf16(synth.rng(wl.seed, 1), M, K).view(np.int16)).cuda()
        self.xd = torch.from_numpy(synth.x_bf16(synth.rng(wl.seed, 3), M, N).view(np.int16)).cuda()
        self.ids_list = [synth.routing(synth.rng(wl.seed, 100 + r), tokens, topk, E) for r in range(LAYER_ROUTINGS)]
        self.ids_dev = [torch.from_numpy(i).cuda() for i in self.ids_list]
        per_expert = 2 * qg.quant_packed_bytes(wl.fmt, 1, N, K) + qg.quant_packed_bytes(wl.fmt, 1, K, N)
        self.distinct_list = [len(np.unique(i)) for i in self.ids_list]
        self.call_bytes = [d * per_expert for d in self.distinct_list]
        self.bytes_per_call = sum(self.call_bytes) / len(self.call_bytes)
        self.distinct = sum(self.distinct_list) / len(self.distinct_list)
        self.copies = 1
        self.y_gate = torch.empty((M, N), dtype=torch.float32, device="cuda")
        self.y_up = torch.empty((M, N), dtype=torch.float32, device="cuda")
        self.y_down = torch.empty((M, K), dtype=torch.float32, device="cuda")
        wsb = qg.quant_grouped_workspace_bytes(E, M)
        self.ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        log("[bench] %s: generated and placed %.1f MB in %.1f s" % (wl.name, self.wbytes_total / 1e6,
                                                                      time.time() - t0))
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        L = qg.lib()
        vp = lambda t: ctypes.c_void_p(t.data_ptr())
        fmt = wl.fmt

        def step(s, ids):
            for w, xx, yy, n, k in ((self.w_gate, self.x, self.y_gate, N, K), (self.w_up, self.x, self.y_up, N, K),
                                    (self.w_down, self.xd, self.y_down, K, N)):
                st = L.quant_grouped_gemm(vp(w), fmt, E, n, k, M, vp(xx), vp(ids), vp(yy), vp(self.ws), wsb, s)
                if st != 0:
                    return st
            return 0
        self.calls = [lambda s, ids=ids: step(s, ids) for ids in self.ids_dev]

    def bytes_of(self, i):
        return self.call_bytes[i % len(self.call_bytes)] if self.call_bytes else self.bytes_per_call

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
    # and untimed calls until the clocks have ramped up (at least WARM_S of work)
    t0, i = time.time(), warmup
    while time.time() - t0 < WARM_S:
        for _ in range(16):
            p.call(i)
            i += 1
        torch.cuda.synchronize()
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
    """One call per rotated weight copy (at least 64 calls) captured in one HIP
    graph (torch's CUDAGraph), replayed `reps` times; seconds per call (the
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
    ncalls = max(64, len(p.calls))
    with torch.cuda.graph(g):
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(ncalls):
            p.call(i, st)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / 1e3 / ncalls)
    return float(np.median(times))


class ReadProbe:
    """The plain streaming-read reference (quant_read_probe: each 16-byte granule
    read once, non-temporal loads, nothing written).  One device buffer serves
    every size; a size is read from rotating slices of it (>= 1 GiB of distinct
    bytes per cycle, as the workloads rotate their weights) so that the rate is
    that of HBM, not of the last-level cache."""

    def __init__(self, max_bytes: int):
        import torch
        self.cap = max(2 * ROTATE_BYTES, 2 * max_bytes + ROTATE_BYTES // 8)
        self.buf = torch.ones(self.cap // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def gbs(self, nbytes: int, steps: int = 50, reps: int = 3) -> float:
        import torch
        import gemm_block_quant_amd as qg
        nbytes = (int(nbytes) + 255) // 256 * 256
        copies = max(2, -(-ROTATE_BYTES // nbytes))
        copies = min(copies, self.cap // nbytes)
        # raw C calls with prepared arguments, so that host overhead never limits the rate
        L = qg.lib()
        base = self.buf.data_ptr()
        ptrs = [ctypes.c_void_p(base + c * nbytes) for c in range(copies)]
        sink = ctypes.c_void_p(self.sink.data_ptr())
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        n = ctypes.c_size_t(nbytes)

        def call(i, stream=st):
            if L.quant_read_probe(ptrs[i % copies], n, sink, stream) != 0:
                raise RuntimeError("quant_read_probe failed")
        t0, i = time.time(), 0
        while time.time() - t0 < WARM_S:
            for _ in range(16):
                call(i)
                i += 1
            torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(steps):
                call(i)
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) / 1e3 / steps
            best = t if best is None else min(best, t)
        return nbytes / best / 1e9


def read_clocks():
    """Current GPU shader and memory clock levels (MHz) from sysfs, or None."""
    import glob
    out = {}
    for key, fname in (("sclk_MHz", "pp_dpm_sclk"), ("mclk_MHz", "pp_dpm_mclk")):
        for path in sorted(glob.glob("/sys/class/drm/card*/device/" + fname)):
            try:
                with open(path) as f:
                    for line in f:
                        if line.rstrip().endswith("*"):
                            out[key] = int(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
            except (OSError, ValueError, IndexError):
                continue
            if key in out:
                break
    return out or None


def clocks_under_load(p, seconds: float = 0.3):
    """Clock levels sampled while the workload's calls run back to back (these
    calls are outside every timed region)."""
    import threading
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            c = read_clocks()
            if c:
                samples.append(c)
            time.sleep(0.02)
    th = threading.Thread(target=sampler)
    th.start()
    t0, i = time.time(), 0
    while time.time() - t0 < seconds:
        for _ in range(64):
            p.call(i)
            i += 1
        torch.cuda.synchronize()
    stop.set()
    th.join()
    out = {}
    for key in ("sclk_MHz", "mclk_MHz"):
        v = [c[key] for c in samples if key in c]
        if v:
            out[key] = {"min": min(v), "max": max(v), "samples": len(v)}
    return out or None


def kernel_source_hash() -> str:
    """Hash of the HIP sources' code (comments and blank space left out): HBM-
    traffic figures taken from counters are only reported while the kernels
    they were taken on are unchanged."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "gemm_block_quant_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "r", encoding="utf-8") as fh:
            code = re.sub(r"/\*.*?\*/|//[^\n]*", " ", fh.read(), flags=re.S)
        h.update(" ".join(code.split()).encode())
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


def _counter_values(out_dir: str, counter: str):
    """{kernel name: [counter value of each dispatch]} from rocprofv3 counter CSVs under out_dir."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] == counter:
                    vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return vals


def pmc_summary(fetch_dir: str, write_dir: str, key: str, fetch_cmd: str, write_cmd: str):
    """Turn a FETCH_SIZE run and a WRITE_SIZE run (each over bench.py --calibrate-copy)
    into calibrated bytes per call, stored under `key` in profiles/traffic.json."""
    # Per step: the counters of every dispatch of the product kernels, divided by
    # the number of steps profiled.  A grouped call dispatches the bucketing once,
    # so the bucketing's dispatch count is the number of grouped calls; a step of
    # the MoE-layer workload is three of them (gate, up, down), a step of the MoE
    # block one.  Dense products dispatch one kernel per call.
    wl = workloads().get(key)
    calls = 3 if wl is not None and wl.layer else 1
    out = {"source_hash": kernel_source_hash(), "fetch_command": fetch_cmd, "write_command": write_cmd,
           "copy_bytes_each_way": COPY_ELEMS * 4, "calls_per_step": calls}
    for name, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        vals = _counter_values(d, counter)
        # the product kernels (not the streaming-read reference)
        ours = {k: v for k, v in vals.items() if "qg::" in k and "k_read_probe" not in k}
        copy = [sum(v) / len(v) for k, v in vals.items() if "neg" in k.lower() and "qg::" not in k]
        if not ours or not copy:
            raise SystemExit("pmc summary: no %s rows for %s in %s" % (counter, "our kernels" if not ours else "the copy", d))
        factor = COPY_ELEMS * 4 / (copy[0] * 1024)
        bucket = [len(v) for k, v in ours.items() if "k_bucket" in k]
        steps = (bucket[0] / calls) if bucket else max(len(v) for v in ours.values())
        per_call_kib = sum(sum(v) for v in ours.values()) / steps
        out[name + "_kib_per_call_raw"] = round(per_call_kib, 3)
        out[name + "_copy_kib_raw"] = round(copy[0], 3)
        out[name + "_factor"] = round(factor, 5)
        out[name + "_bytes"] = int(round(per_call_kib * 1024 * factor))
        out[name + "_kernels"] = {k: round(sum(v) / steps, 3) for k, v in ours.items()}
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p: Prepared, target_s: float = 10.0, single_s: float = 4.0):
    """The oracle (as it stands) on a bounded sample of the same workload, on all
    host threads and on one."""
    import oracle
    allt = _cpu_leg(p, target_s, 0)
    one = _cpu_leg(p, single_s, 1)
    allt["single_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"]}
    allt["cpu_model"] = cpu_model()
    allt["host_threads_available"] = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return allt


def _cpu_leg(p: Prepared, target_s: float, nthreads_req: int):
    """The first output rows, doubling until one pass takes about target_s; when
    the whole matrix takes less, whole passes are repeated until target_s has
    elapsed.  nthreads_req 0: every thread the oracle's OpenMP runtime uses."""
    import oracle
    wl = p.wl
    nthreads = oracle.max_threads() if nthreads_req <= 0 else nthreads_req
    ids = p.ids_host if wl.moe else None
    rows_try = 64
    while True:
        cols = np.arange(min(rows_try, wl.N))
        t0 = time.time()
        oracle.gemm(wl.fmt, p.w_host, wl.N, wl.K, p.x_host, E=wl.E, cols=cols, ids=ids, nthreads=nthreads)
        dt = time.time() - t0
        if dt >= target_s or rows_try >= wl.N:
            break
        rows_try = int(min(wl.N, max(rows_try * 2, rows_try * target_s / max(dt, 1e-3) * 1.05)))
    passes = 1
    if dt < target_s:
        t0 = time.time()
        passes = 0
        while time.time() - t0 < target_s:
            oracle.gemm(wl.fmt, p.w_host, wl.N, wl.K, p.x_host, E=wl.E, cols=cols, ids=ids, nthreads=nthreads)
            passes += 1
        dt = time.time() - t0
    # the workload's weight bytes in proportion to the outputs computed (same unit as the GPU figure)
    pass_bytes = p.bytes_per_call * len(cols) / wl.N
    return {"value": round(pass_bytes * passes / dt / 1e9, 4), "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": "%d of %d output rows x M=%d (%.1f MB of packed weights per pass), %d pass(es) in %.2f s, "
                      "%d threads" % (len(cols), wl.N, wl.M, pass_bytes / 1e6, passes, dt, nthreads)}


def result_for(p: Prepared, steps: int, warmup: int, key: str = None, probe: ReadProbe = None):
    """Time `steps` calls (whole job, events at the two ends) and the same calls
    with an event pair around each launch; the rates, roofline fractions and
    (when counters were taken on the current sources) the measured HBM traffic."""
    total, per_mean, per_med = time_workload(p, steps, warmup)
    wl = p.wl
    job_bytes = sum(p.bytes_of(i) for i in range(steps))
    gbs = job_bytes / total / 1e9
    kern_gbs = p.bytes_per_call / per_mean / 1e9
    r = {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K, "E": wl.E,
         "weight_bytes_per_call": int(round(p.bytes_per_call)), "rotated_copies": p.copies,
         "ms_per_call": round(total / steps * 1e3, 5), "kernel_ms_mean": round(per_mean * 1e3, 5),
         "kernel_ms_median": round(per_med * 1e3, 5),
         "weight_GBps": round(gbs, 1), "kernel_weight_GBps": round(kern_gbs, 1),
         "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
         "implied_tok_s": round(wl.M * gbs / TOKEN_BYTES_GB, 1)}
    if p.entry:
        r["entry"] = p.entry
    if wl.moe or wl.block:
        r["distinct_experts"] = p.distinct
    if wl.layer:
        r["grouped_calls_per_step"] = 3
        r["routings_cycled"] = LAYER_ROUTINGS
    if wl.M >= 32 and not wl.block and not wl.layer:
        flops = 2.0 * wl.M * wl.N * wl.K
        r["TFLOPs"] = round(flops / (total / steps) / 1e12, 1)
        r["pct_bf16_mfma_peak"] = round(100 * flops / (total / steps) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 2)
    if probe is not None:
        ach = probe.gbs(p.bytes_per_call)
        r["achievable_read_GBps"] = round(ach, 1)
        r["pct_of_achievable"] = round(100 * gbs / ach, 2)
    if key is not None:
        tr = traffic_for(key)
        r["traffic_bytes_per_call"] = tr
        r["traffic_ratio"] = round(tr / p.bytes_per_call, 4) if tr else None
    if p.bytes_per_call < GRAPH_BYTES and not wl.layer and not wl.block:
        # launch-bound: the rotated calls replayed from one graph
        gt = graph_time(p)
        r["graph_ms_per_call"] = round(gt * 1e3, 5)
        r["graph_weight_GBps"] = round(p.bytes_per_call / gt / 1e9, 1)
    return r, total, per_mean


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, help="headline workload (default: the Q4_K gate+up GEMV)")
    ap.add_argument("--only", action="store_true", help="time the headline workload only (no configs list)")
    ap.add_argument("--all", action="store_true", help="also time every other workload shape (sweep)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sweep-out", default=None, help="write the configs and sweep as JSON lines to this file")
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
    clocks = {"before": read_clocks()}
    probe = ReadProbe(1_042_944_000)
    achievable = probe.gbs(ROTATE_BYTES, steps=10)
    log("[bench] plain streaming read of 1 GiB (quant_read_probe): %.1f GB/s" % achievable)

    # the headline first: its timed region is the JSON line's value
    p = Prepared(wls[args.workload])
    torch.cuda.synchronize()
    r, total, per_mean = result_for(p, args.steps, args.warmup, args.workload, probe)
    clocks["under_load"] = clocks_under_load(p)
    log("[bench] %s" % json.dumps(r))
    headline_bytes = p.bytes_per_call
    cpu = None
    if not args.no_cpu and not p.wl.block and not p.wl.layer:
        cpu = cpu_baseline(p)
        log("[bench] cpu baseline %s" % json.dumps(cpu))
    if args.calibrate_copy:
        copy_calibration()
    del p
    torch.cuda.empty_cache()

    configs, sweep = [], []
    keys = [] if args.only else [(c, k) for c, k in CONFIGS]
    if args.all:
        listed = {k for _, k in CONFIGS}
        keys += [(None, k) for k in wls if k not in listed]
    for cfg, key in keys:
        if key == args.workload and cfg is not None:
            r2 = dict(r)
        else:
            try:
                p2 = Prepared(wls[key])
                # enough calls for a stable time, a few tenths of a second at most
                steps = max(20, min(args.steps, int(0.3 / max(1e-6, p2.bytes_per_call / 5e12))))
                r2, _, _ = result_for(p2, steps, min(args.warmup, steps), key, probe)
                del p2
            except Exception as e:  # a workload the build cannot run is reported, not fatal
                r2 = {"workload": wls[key].name, "M": wls[key].M, "error": str(e)}
            torch.cuda.empty_cache()
        r2["key"] = key
        if cfg is not None:
            r2["config"] = cfg
            configs.append(r2)
        else:
            sweep.append(r2)
        log("[bench] %s" % json.dumps(r2))
    clocks["after"] = read_clocks()
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            for x in configs + sweep:
                f.write(json.dumps(x) + "\n")

    value = headline_bytes * args.steps / total / 1e9
    # the step is one launch of the product kernel: its average duration over the
    # timed region (events on the launch stream at the region's two ends)
    achieved = headline_bytes / (total / args.steps) / 1e9
    wl = wls[args.workload]
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
                   "N": wl.N, "K": wl.K, "weight_bytes": int(headline_bytes), "rotated_copies": r["rotated_copies"],
                   "implied_tok_s": r["implied_tok_s"],
                   "ms_per_launch_with_per_launch_events": round(per_mean * 1e3, 5),
                   "achievable_read_GBps_1GiB": round(achievable, 1),
                   "achievable_read_GBps": r.get("achievable_read_GBps"),
                   "pct_of_achievable": r.get("pct_of_achievable")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(args.workload)},
        "cpu_baseline": cpu,
        "clocks": clocks,
        "configs": configs,
    }
    if sweep:
        out["sweep"] = sweep
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
