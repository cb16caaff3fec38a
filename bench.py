"""Benchmark of the W4A16 MoE path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one whole MoE layer: routing (top-8 of 128, expert offsets, token
sort), the gate/up grouped matmul with the fused GEGLU epilogue, the down
grouped matmul and the weighted combine, each through its own entry point of
libw4a16.so on torch's current stream.  Inputs are synthetic and seeded and
already resident in HBM when the timed region starts.  Three distinct weight
sets (3 x 428 MB, more than the 256 MB last-level cache) are used in turn so
that the weight bytes come from HBM.

Workloads (default: moe-decode, with moe-prefill measured in the same run):
  moe-decode    T=64 tokens, d_model 2816, 128 experts, expert hidden 704, top-8
  moe-prefill   T=4096 tokens, same experts, Zipf(1.1) expert popularity
  dense-decode  w4a16_linear, M in {1, 8, 16}, K=4096, N=14336
  dense-prefill w4a16_linear, M=4096, K=4096, N=14336 (TFLOP/s)
  repack-export repack of one layer exported with fp32 scales and bf16-rounded
                weights: bit-identical fraction, worst relative difference
  repack        q4_group_repack of 30 layers x 128 experts of on-grid bf16 weights
  e2e           repack of the 30 layers, then T=256 decode through all 30 layers
  fp8           the moe-decode and moe-prefill layers over FP8 (E4M3) experts, the
                comparison path (also measured in the default run)

Prints ONE JSON line.  value = touched-expert weight bytes per layer / layer
time (moe-decode); the roofline object is for the dominant kernel (the gate/up
grouped matmul), timed with HIP events around its launches inside the timed
region (the only events there: each record costs a few microseconds of stream
time, so the per-call breakdown comes from an instrumented pass afterwards).  cpu_baseline times the CPU oracle (test infrastructure) on a bounded
sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
import int4_group_quantized_q4_amd as w4  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, TFLOP/s
EXPERT_W1_BYTES = 1408 * 2816 // 2 + 1408 * 88 * 2   # 2,230,272
EXPERT_W2_BYTES = 2816 * 704 // 2 + 2816 * 22 * 2    # 1,115,136

# HBM bytes per launch of the two roofline kernels, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes over this bench (profiles/gemm_hbm_traffic.md): reads scaled
# by 2.000 and writes by 1.000, the factors a 512 MiB device copy gives.  They
# hold only for the code they were taken on (sha256 of the listed files in
# csrc/, in order, comments and blank lines removed: sources_sha256); once
# that code changes, the bench reports traffic as null.
TRAFFIC = {
    "decode_gmm1": {"sources": ("gemm_skinny.hip", "common.h", "internal.h"),
                    "sha256": "8ed30d9d7c51d6629fbed711f76b9ee8b1e817372d5a07ff715cf975866c3c70",
                    "read_bytes": 139715 * 2048, "write_bytes": 725 * 1024},
    "prefill_gmm1": {"sources": ("gemm_tiled.hip", "common.h", "internal.h"),
                     "sha256": "1297ca20c60924a20d5a114d81e548aebc010fe3668275c0cbb80123a0a7d019",
                     "read_bytes": 271193 * 2048, "write_bytes": 53697 * 1024},
    "dense_prefill": {"sources": ("gemm_tiled.hip", "common.h", "internal.h"),
                      "sha256": "1297ca20c60924a20d5a114d81e548aebc010fe3668275c0cbb80123a0a7d019",
                      "read_bytes": 275319 * 2048, "write_bytes": 119939 * 1024},
}


def traffic_source(key):
    rec = TRAFFIC[key]
    return ("rocprofv3 FETCH_SIZE and WRITE_SIZE counter passes (profiles/gemm_hbm_traffic.md) taken on kernel "
            "sources' code sha256 %s...; null once that code changes" % rec["sha256"][:12])


def sources_sha256(files):
    """sha256 of the listed csrc/ files with their comments and blank lines
    removed, so that only a change of code invalidates a counter figure."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "int4_group_quantized_q4_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(l.rstrip() for l in text.splitlines() if l.strip())
        h.update(code.encode())
    return h.hexdigest()


def traffic_of(key):
    """Counter-measured HBM bytes (read + write) per launch, or None when the
    kernel's code differs from the code the counters were taken on."""
    rec = TRAFFIC[key]
    if sources_sha256(rec["sources"]) != rec["sha256"]:
        return None
    return rec["read_bytes"] + rec["write_bytes"]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ MoE layer
class MoeLayerSet:
    """Several distinct MoE weight sets + inputs resident on the device."""

    def __init__(self, cfg, copies, seed, device):
        self.cfg = cfg
        T, d, I, E, k = cfg["T"], cfg["d"], cfg["I"], cfg["E"], cfg["k"]
        self.T, self.d, self.I, self.E, self.k = T, d, I, E, k
        g = gen.torch_generator(device, seed)
        self.layers = []
        for c in range(copies):
            self.layers.append({
                "w1q": gen.bytes_uniform_t(g, E * 2 * I * d // 2, device),
                # i.i.d. scales: drawn directly in the tile16 scale layout
                "w1s": gen.scales_loguniform_t(g, (E, 2 * I, d // 32), device),
                "w2q": gen.bytes_uniform_t(g, E * d * I // 2, device),
                "w2s": gen.scales_loguniform_t(g, (E, d, I // 32), device),
                "x": gen.bf16_normal_t(g, (T, d), device),
                "logits": gen.router_logits_t(g, T, E, device, cfg["router"], cfg.get("zipf_s", 1.1)),
            })
        R = T * k
        i32 = dict(dtype=torch.int32, device=device)
        self.ids = torch.empty(T, k, **i32)
        self.wts = torch.empty(T, k, dtype=torch.float32, device=device)
        self.offs = torch.empty(E + 1, **i32)
        self.srows = torch.empty(R, **i32)
        self.stoks = torch.empty(R, **i32)
        self.r2s = torch.empty(R, **i32)
        self.rws = torch.empty(max(16, w4.w4a16_moe_route_workspace(T, E, k)), dtype=torch.uint8, device=device)
        self.act = torch.empty(R, I, dtype=torch.bfloat16, device=device)
        self.o = torch.empty(R, d, dtype=torch.float32, device=device)
        self.y = torch.empty(T, d, dtype=torch.bfloat16, device=device)
        gws = max(w4.w4a16_moe_gmm_workspace(T, R, E, d, 2 * I), w4.w4a16_moe_gmm_workspace(R, R, E, I, d))
        self.gws = torch.empty(max(16, gws), dtype=torch.uint8, device=device)
        # decode batches take the streaming path of w4a16_moe_layer: the gate/up
        # matmul with the top-k from the logits, the down matmul over rows
        # found from the ids (a and o at the routed rows), the combine with the
        # identity row map
        self.streaming = not w4.w4a16_moe_layer_sorted(T, E, k, d, I)
        self.ident = torch.arange(R, dtype=torch.int32, device=device)

    def step(self, c, ev=None):
        """One layer, as w4a16_moe_layer runs it.  ev: None, 2 events (around
        the gate/up matmul only) or 5 (between the calls); each event record
        costs a few microseconds of stream time."""
        if self.streaming:
            return self.step_streaming(c, ev)
        L = self.layers[c]
        T, d, I, E, k = self.T, self.d, self.I, self.E, self.k
        R = T * k
        full = ev is not None and len(ev) == 5
        if full:
            ev[0].record()
        w4.w4a16_moe_route(L["logits"], k, self.ids, self.wts, self.offs, self.srows, self.stoks, self.r2s, self.rws)
        if ev is not None:
            ev[1 if full else 0].record()
        w4.w4a16_moe_gmm(L["x"], self.stoks, self.offs, E, R, d, 2 * I, L["w1q"], L["w1s"], w4.W4_EPI_GEGLU_TANH,
                         self.act, w4.W4_OUT_BF16, self.gws)
        if ev is not None:
            ev[2 if full else 1].record()
        w4.w4a16_moe_gmm(self.act, None, self.offs, E, R, I, d, L["w2q"], L["w2s"], w4.W4_EPI_NONE, self.o,
                         w4.W4_OUT_F32, self.gws)
        if full:
            ev[3].record()
        w4.w4a16_moe_combine(self.o, w4.W4_OUT_F32, self.r2s, self.wts, T, k, d, self.y)
        if full:
            ev[4].record()

    def step_streaming(self, c, ev=None):
        L = self.layers[c]
        T, d, I, E, k = self.T, self.d, self.I, self.E, self.k
        full = ev is not None and len(ev) == 5
        if full:
            ev[0].record()
        # (the top-k plan comes out of the gate/up call: up to 64 tokens its
        # workgroups rank the logits themselves, else it launches the top-k)
        if ev is not None:
            ev[1 if full else 0].record()
        w4.w4a16_moe_gmm_logits(L["x"], L["logits"], k, d, 2 * I, L["w1q"], L["w1s"], w4.W4_EPI_GEGLU_TANH,
                                self.act, self.ids, self.wts)
        if ev is not None:
            ev[2 if full else 1].record()
        w4.w4a16_moe_gmm_ids(self.act, self.ids, T, k, 1, E, I, d, L["w2q"], L["w2s"], w4.W4_EPI_NONE, self.o,
                             w4.W4_OUT_F32)
        if full:
            ev[3].record()
        w4.w4a16_moe_combine(self.o, w4.W4_OUT_F32, self.ident, self.wts, T, k, d, self.y)
        if full:
            ev[4].record()

    def touched(self, c):
        """Experts with at least one routed row in copy c (host-side, untimed)."""
        self.step(c)
        torch.cuda.synchronize()
        ids = self.ids.cpu().numpy().ravel()
        counts = np.bincount(ids, minlength=self.E)
        return int(np.count_nonzero(counts)), counts


class TimingEvent:
    """A HIP event used only for timing, created with hipEventDisableSystemFence:
    a default event's record ends with a system-scope release (cache writeback
    and invalidate) that slows the work queued after it by a few microseconds.
    Recorded on torch's current stream; read only after a device synchronize."""
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            torch.cuda.init()
            h = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch has loaded
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        self.ev = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self.ev), 0x20000000)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)

    def record(self):
        rc = self._lib().hipEventRecord(self.ev, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


WARMUP_MIN_S = 0.3


def warm_up(step, warmup):
    """At least `warmup` untimed steps and at least WARMUP_MIN_S seconds of
    them: the GPU's clocks reach their sustained level only after a few
    hundred milliseconds of load (the decode GEMM runs ~10% slower in the
    first ones)."""
    import time
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < WARMUP_MIN_S:
        step(n)
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


# every EVENT_STRIDE-th layer of the timed region carries the two events
# around its gate/up GEMM (each record adds about a microsecond of stream
# time, which the other layers are spared)
EVENT_STRIDE = 4


def time_moe(cfg, steps, warmup, copies=3, seed=1234):
    """Timed region: `steps` layers, every EVENT_STRIDE-th with HIP events
    around its gate/up GEMM (that GEMM's average launch time), and the
    whole-layer time.  Afterwards, an instrumented pass with events between
    all four calls gives the per-call breakdown (route, gate/up, down,
    combine), whose event records add a few microseconds to each call."""
    dev = torch.device("cuda:0")
    ls = MoeLayerSet(cfg, copies, seed, dev)
    touched = [ls.touched(c)[0] for c in range(copies)]
    warm_up(lambda i: ls.step(i % copies), warmup)
    timed = list(range(0, steps, EVENT_STRIDE))
    evs = {i: [TimingEvent() for _ in range(2)] for i in timed}
    torch.cuda.synchronize()
    start, stop = TimingEvent(), TimingEvent()
    start.record()
    for i in range(steps):
        ls.step(i % copies, evs.get(i))
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    g1 = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in timed])
    nb = min(steps, 30)
    evb = [[TimingEvent() for _ in range(5)] for _ in range(nb)]
    for i in range(nb):
        ls.step(i % copies, evb[i])
    torch.cuda.synchronize()
    parts = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evb])  # route, gmm1, gmm2, combine
    mean_touched = float(np.mean([touched[i % copies] for i in range(steps)]))
    # the same layers through the one w4a16_moe_layer call (its own workspace)
    lws = torch.empty(w4.w4a16_moe_layer_workspace(ls.T, ls.E, ls.k, ls.d, ls.I), dtype=torch.uint8, device=dev)
    yl = torch.empty(ls.T, ls.d, dtype=torch.bfloat16, device=dev)

    def layer_call(i):
        L = ls.layers[i % copies]
        w4.w4a16_moe_layer(L["x"], L["logits"], ls.k, ls.I, L["w1q"], L["w1s"], L["w2q"], L["w2s"],
                           w4.W4_EPI_GEGLU_TANH, yl, lws)
    warm_up(layer_call, 3)
    la, lb = TimingEvent(), TimingEvent()
    la.record()
    for i in range(steps):
        layer_call(i)
    lb.record()
    torch.cuda.synchronize()
    return {
        "layer_call_ms": la.elapsed_time(lb) / steps,
        "ms_per_step": total_ms / steps,
        "gmm1_ms": float(g1.mean()),
        "gmm1_ms_p10_p90": [float(np.percentile(g1, 10)), float(np.percentile(g1, 90))],
        "route_ms": float(parts[:, 0].mean()),
        "gmm2_ms": float(parts[:, 2].mean()),
        "combine_ms": float(parts[:, 3].mean()),
        "instrumented_ms": {k: round(float(parts[:, j].mean()), 5)
                            for j, k in enumerate(("route_ms", "gmm1_ms", "gmm2_ms", "combine_ms"))},
        "touched_experts": mean_touched,
        "layerset": ls,
    }


def moe_decode_report(steps, warmup):
    cfg = gen.MOE_DECODE
    r = time_moe(cfg, steps, warmup)
    wbytes = r["touched_experts"] * (EXPERT_W1_BYTES + EXPERT_W2_BYTES)
    w1bytes = r["touched_experts"] * EXPERT_W1_BYTES
    gmm_ms = r["gmm1_ms"] + r["gmm2_ms"]
    out = {
        "value": wbytes / (r["ms_per_step"] * 1e-3) / 1e9,
        "ms_per_step": r["ms_per_step"],
        "gmm_weight_GBs": wbytes / (gmm_ms * 1e-3) / 1e9,
        "gmm_frac_of_hbm": wbytes / (gmm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "weight_bytes_per_layer": wbytes,
        "touched_experts": r["touched_experts"],
        "kernel_ms": {k: round(r[k], 5) for k in ("route_ms", "gmm1_ms", "gmm2_ms", "combine_ms")},
        "gmm1_ms_p10_p90": r["gmm1_ms_p10_p90"],
        "kernel_ms_note": "gmm1 (the gate/up matmul, whose workgroups also rank the logits and write the "
                          "top-k plan) from the timed region; route (no launch of its own on this path), gmm2, "
                          "combine from an instrumented pass after it",
        "layer_ms_single_call": r["layer_call_ms"],
        "roofline": {
            "bound": "hbm",
            "kernel": "gate/up grouped matmul with its rows and the top-k plan from the router logits "
                      "(w4a16_moe_gmm_logits, GEGLU epilogue)",
            "achieved": w1bytes / (r["gmm1_ms"] * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": w1bytes / (r["gmm1_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": traffic_of("decode_gmm1"),
            "traffic_source": traffic_source("decode_gmm1"),
        },
    }
    return out, r["layerset"]


def moe_prefill_report(steps, warmup, keep=False):
    cfg = gen.MOE_PREFILL
    r = time_moe(cfg, steps, warmup)
    R = cfg["T"] * cfg["k"]
    d, I = cfg["d"], cfg["I"]
    flops1 = 2.0 * R * d * 2 * I
    flops2 = 2.0 * R * I * d
    gmm_ms = r["gmm1_ms"] + r["gmm2_ms"]
    tf = (flops1 + flops2) / (gmm_ms * 1e-3) / 1e12
    rep = {
        "workload": "moe-prefill: T=4096, d_model=2816, E=128, top-8 Zipf(1.1), expert hidden 704, int4 g32",
        "gmm_TFLOPs": tf,
        "gmm_frac_of_bf16_mfma": tf / BF16_MFMA_PEAK_TFLOPS,
        "layer_TFLOPs": (flops1 + flops2) / (r["ms_per_step"] * 1e-3) / 1e12,
        "ms_per_step": r["ms_per_step"],
        "useful_flops_per_layer": flops1 + flops2,
        "kernel_ms": {k: round(r[k], 5) for k in ("route_ms", "gmm1_ms", "gmm2_ms", "combine_ms")},
        "gmm1_ms_p10_p90": r["gmm1_ms_p10_p90"],
        "kernel_ms_note": "gmm1 from the timed region; route, gmm2, combine from an instrumented pass after it",
        "layer_ms_single_call": r["layer_call_ms"],
        "mfma_dtype": "fp16 MFMA on exact s*q weights and fp16 activation rows under a per-row power of two "
                      "(exact bf16 products; fp16 and bf16 share the dense peak)",
        "roofline": {
            "bound": "mfma",
            "kernel": "gate/up grouped matmul (w4a16_moe_gmm, GEGLU epilogue; fp16 MFMA on exact s*q)",
            "achieved": flops1 / (r["gmm1_ms"] * 1e-3) / 1e12,
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": flops1 / (r["gmm1_ms"] * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "traffic": traffic_of("prefill_gmm1"),
            "traffic_source": traffic_source("prefill_gmm1"),
        },
    }
    if keep:
        return rep, r["layerset"]
    return rep


def cpu_baseline_decode(layerset):
    """The oracle (as it stands) on copy 0 of the moe-decode layer: all 64 tokens."""
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import layout
    L = layerset.layers[0]
    E, I, d, k, T = layerset.E, layerset.I, layerset.d, layerset.k, layerset.T

    def codes_of(packed, rows, K):
        byte, shift = layout._index(rows, K)
        per = packed.cpu().numpy().reshape(E, rows * K // 2)
        v = (per[:, byte] >> shift[None]) & 0xF
        return (v.astype(np.int16) - 8).astype(np.int8)

    def scales_of(tiled, rows, K):
        t = tiled.cpu().numpy().view(np.uint16).reshape(E, -1)
        return np.stack([layout.decode_scales(t[e], rows, K) for e in range(E)])

    w1c = codes_of(L["w1q"], 2 * I, d)
    w2c = codes_of(L["w2q"], d, I)
    w1s = scales_of(L["w1s"], 2 * I, d)
    w2s = scales_of(L["w2s"], d, I)
    x = L["x"].view(torch.int16).cpu().numpy().view(np.uint16)
    logits = L["logits"].cpu().numpy()
    touched = int(np.count_nonzero(np.bincount(oracle.route(logits, k)["ids"].ravel(), minlength=E)))
    t0 = time.perf_counter()
    oracle.moe_layer(x, logits, w1c, w1s, w2c, w2s, k=k)
    dt = time.perf_counter() - t0
    wbytes = touched * (EXPERT_W1_BYTES + EXPERT_W2_BYTES)
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count()
    return {
        "value": wbytes / dt / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "one full moe-decode layer (64 tokens, %d touched experts), NumPy fp64, %.2f s" % (touched, dt),
    }


# --------------------------------------------------------------- FP8 (W8A8)
FP8_MFMA_PEAK_TFLOPS = 5033.2   # MI355X dense fp8 MFMA, TFLOP/s


def fp8_report(steps, warmup, w4_decode_ms=None, w4_prefill_ms=None):
    """The same MoE layers over FP8 experts (E4M3 codes, fp32 per-channel
    scales, per-row activation quantization) through w8a8_moe_layer, and the
    gate/up matmul alone, on the moe-decode and moe-prefill shapes."""
    dev = torch.device("cuda:0")
    out = {"workload": "the moe-decode and moe-prefill layers with E4M3 experts (1 byte per weight + fp32 "
                       "per-row scales), activations quantized per row at run time; w8a8_moe_layer and "
                       "w8a8_moe_gmm (16x16x128 FP8 MFMA)"}
    for name, cfg, copies in (("decode", gen.MOE_DECODE, 3), ("prefill", gen.MOE_PREFILL, 3)):
        T, d, I, E, k = cfg["T"], cfg["d"], cfg["I"], cfg["E"], cfg["k"]
        R = T * k
        g = gen.torch_generator(dev, 4321 + cfg["id"])
        layers = []
        for _ in range(copies):
            layers.append({"w1q": gen.fp8_codes_t(g, (E * 2 * I * d,), dev), "w1s": gen.fp8_scales_t(g, (E * 2 * I,), dev),
                           "w2q": gen.fp8_codes_t(g, (E * d * I,), dev), "w2s": gen.fp8_scales_t(g, (E * d,), dev),
                           "x": gen.bf16_normal_t(g, (T, d), dev),
                           "logits": gen.router_logits_t(g, T, E, dev, cfg["router"], cfg.get("zipf_s", 1.1))})
        nws = w4.w8a8_moe_layer_workspace(T, E, k, d, I)
        wss = [torch.empty(nws, dtype=torch.uint8, device=dev) for _ in range(copies)]
        y = torch.empty(T, d, dtype=torch.bfloat16, device=dev)

        def layer(i):
            L = layers[i % copies]
            w4.w8a8_moe_layer(L["x"], L["logits"], k, I, L["w1q"], L["w1s"], L["w2q"], L["w2s"],
                              w4.W4_EPI_GEGLU_TANH, y, wss[i % copies])
        warm_up(layer, warmup)
        a, b = TimingEvent(), TimingEvent()
        a.record()
        for i in range(steps):
            layer(i)
        b.record()
        torch.cuda.synchronize()
        layer_ms = a.elapsed_time(b) / steps
        # gate/up alone on each copy's plan, left in its workspace by the calls above
        p = w4.w8a8_moe_layer_plan(T, E, k, d, I)
        views = []
        for c in range(copies):
            ws = wss[c]
            views.append({"offs": ws[p[2]:p[2] + (E + 1) * 4].view(torch.int32),
                          "stoks": ws[p[4]:p[4] + R * 4].view(torch.int32),
                          "xq": ws[p[7]:p[7] + T * d].view(T, d),
                          "xs": ws[p[8]:p[8] + T * 4].view(torch.float32),
                          "act": ws[p[9]:p[9] + R * I * 2].view(torch.bfloat16).view(R, I)})
        touched = [int(torch.count_nonzero(v["offs"][1:] - v["offs"][:-1]).item()) for v in views]

        def gmm1(i):
            L, v = layers[i % copies], views[i % copies]
            w4.w8a8_moe_gmm(v["xq"], v["xs"], v["stoks"], v["offs"], E, R, d, 2 * I, L["w1q"], L["w1s"],
                            w4.W4_EPI_GEGLU_TANH, v["act"], w4.W4_OUT_BF16)
        warm_up(gmm1, warmup)
        a, b = TimingEvent(), TimingEvent()
        a.record()
        for i in range(steps):
            gmm1(i)
        b.record()
        torch.cuda.synchronize()
        g1_ms = a.elapsed_time(b) / steps
        mean_touched = float(np.mean([touched[i % copies] for i in range(steps)]))
        w1b = 2 * I * d + 4 * 2 * I
        wb = w1b + d * I + 4 * d
        rep = {"layer_ms": layer_ms, "gmm1_ms": g1_ms, "touched_experts": mean_touched}
        if name == "decode":
            rep.update({"weight_bytes_per_layer": mean_touched * wb,
                        "layer_weight_GBs": mean_touched * wb / (layer_ms * 1e-3) / 1e9,
                        "gmm1_weight_GBs": mean_touched * w1b / (g1_ms * 1e-3) / 1e9,
                        "gmm1_frac_of_hbm": mean_touched * w1b / (g1_ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
            if w4_decode_ms:
                rep["w4a16_layer_ms"] = w4_decode_ms
                rep["fp8_over_w4a16_layer_time"] = layer_ms / w4_decode_ms
        else:
            f1 = 2.0 * R * d * 2 * I
            rep.update({"gmm1_TFLOPs": f1 / (g1_ms * 1e-3) / 1e12,
                        "gmm1_frac_of_fp8_mfma": f1 / (g1_ms * 1e-3) / 1e12 / FP8_MFMA_PEAK_TFLOPS,
                        "layer_TFLOPs": 2.0 * R * d * 3 * I / (layer_ms * 1e-3) / 1e12})
            if w4_prefill_ms:
                rep["w4a16_layer_ms"] = w4_prefill_ms
                rep["fp8_over_w4a16_layer_time"] = layer_ms / w4_prefill_ms
        out[name] = rep
        del layers, wss, views
    return out


# ----------------------------------------------------------------- ceilings
def ceilings_report():
    """Measured machine ceilings on this GPU (libw4probe.so): a read-only
    stream of 2 GiB with 16-byte loads, and fp16 16x16x32 MFMAs with every
    operand in registers.  The kernels' rates are quoted against these as well
    as against the published peaks."""
    import ctypes
    path = os.path.join(ROOT, "int4_group_quantized_q4_amd", "libw4probe.so")
    if not os.path.exists(path):
        raise RuntimeError("%s is missing: run the build" % path)
    lp = ctypes.CDLL(path)
    lp.w4probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lp.w4probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    blocks = 256 * 16
    out = torch.zeros(blocks, dtype=torch.int32, device=dev)
    run = lambda i: lp.w4probe_stream(buf.data_ptr(), nbytes, out.data_ptr(), blocks, st)
    warm_up(run, 5)
    a, b = TimingEvent(), TimingEvent()
    a.record()
    for i in range(10):
        run(i)
    b.record()
    torch.cuda.synchronize()
    stream_gbs = nbytes / (a.elapsed_time(b) / 10 * 1e-3) / 1e9
    # the same stream over one dense-decode call's weight bytes (33,030,144)
    small = 33030144
    sblocks = small // 16 // 4 // 256   # 2016 blocks: every thread issues its 4 loads at once
    runs = lambda i: lp.w4probe_stream(buf.data_ptr() + (i % 16) * small, small, out.data_ptr(), sblocks, st)
    warm_up(runs, 20)
    a, b = TimingEvent(), TimingEvent()
    a.record()
    for i in range(200):
        runs(i)
    b.record()
    torch.cuda.synchronize()
    small_us = a.elapsed_time(b) / 200 * 1e3
    del buf
    mblocks, iters = 256 * 4, 4096
    mout = torch.empty(mblocks * 256, dtype=torch.float32, device=dev)
    runm = lambda i: lp.w4probe_mfma(mout.data_ptr(), mblocks, iters, st)
    warm_up(runm, 3)
    a, b = TimingEvent(), TimingEvent()
    a.record()
    for i in range(5):
        runm(i)
    b.record()
    torch.cuda.synchronize()
    flops = 2.0 * 16 * 16 * 32 * 8 * iters * 4 * mblocks
    mfma_tf = flops / (a.elapsed_time(b) / 5 * 1e-3) / 1e12
    return {"hbm_read_stream_GBs": stream_gbs, "hbm_read_stream_frac_of_peak": stream_gbs / HBM_PEAK_GBS,
            "read_stream_33MB_us": small_us, "read_stream_33MB_GBs": small / (small_us * 1e-6) / 1e9,
            "mfma_f16_TFLOPs": mfma_tf, "mfma_f16_frac_of_peak": mfma_tf / BF16_MFMA_PEAK_TFLOPS,
            "note": "read-only stream of 2 GiB (16-byte loads), the same over 33 MB back to back (one dense-decode "
                    "call's weight bytes, 16 rotating buffers), and register-only fp16 16x16x32 MFMA loops, "
                    "measured in this run"}


def cpu_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def cpu_baseline_extra(prefill_set=None):
    """The oracle on bounded samples of the repack and prefill workloads."""
    import oracle
    out = {}
    rng = gen.rng_for(5, 900)
    n_groups = 1 << 19
    src = gen.ongrid_source(rng, n_groups // 88 // 16 * 16 or 16, 2816, *gen.MOE_E2E["peak"])
    groups = src["w_bits"].size // 32
    t0 = time.perf_counter()
    oracle.repack_groups(src["w_bits"].reshape(-1, 32))
    dt = time.perf_counter() - t0
    out["repack"] = {"value": groups / dt, "unit": "groups/s", "cores": cpu_threads(), "kind": "oracle",
                     "sample": "%d on-grid groups (rows of 2816, peak level 4..8), %.2f s" % (groups, dt)}
    if prefill_set is not None:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import layout
        ls = prefill_set
        L = ls.layers[0]
        E, I, d, k = ls.E, ls.I, ls.d, ls.k
        toks = 24
        x = L["x"][:toks].view(torch.int16).cpu().numpy().view(np.uint16)
        logits = L["logits"][:toks].cpu().numpy()
        used = np.unique(oracle.route(logits, k)["ids"])

        def codes_of(packed, rows, K):
            byte, shift = layout._index(rows, K)
            per = packed.cpu().numpy().reshape(E, rows * K // 2)
            v = np.zeros((E, rows, K), dtype=np.int8)
            for e in used:
                v[e] = ((per[e][byte] >> shift) & 0xF).astype(np.int16) - 8
            return v

        def scales_of(tiled, rows, K):
            t = tiled.cpu().numpy().view(np.uint16).reshape(E, -1)
            s = np.zeros((E, rows, K // 32), dtype=np.uint16)
            for e in used:
                s[e] = layout.decode_scales(t[e], rows, K)
            return s

        w1c, w2c = codes_of(L["w1q"], 2 * I, d), codes_of(L["w2q"], d, I)
        w1s, w2s = scales_of(L["w1s"], 2 * I, d), scales_of(L["w2s"], d, I)
        t0 = time.perf_counter()
        oracle.moe_layer(x, logits, w1c, w1s, w2c, w2s, k=k)
        dt = time.perf_counter() - t0
        flops = 2.0 * toks * k * (d * 2 * I + I * d)
        out["moe_prefill"] = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cpu_threads(), "kind": "oracle",
                              "sample": "%d of the 4096 Zipf-routed prefill tokens (%d experts), NumPy fp64, %.2f s"
                                        % (toks, len(used), dt)}
    return out


# ------------------------------------------------------------- dense decode
def dense_decode_report(steps, warmup):
    dev = torch.device("cuda:0")
    cfg = gen.DENSE_DECODE
    K, N = cfg["K"], cfg["N"]
    g = gen.torch_generator(dev, 99)
    copies = 16   # 16 x 33 MB > 256 MB last-level cache
    qs = [gen.bytes_uniform_t(g, N * K // 2, dev) for _ in range(copies)]
    ss = [gen.scales_loguniform_t(g, (N, K // 32), dev) for _ in range(copies)]
    wbytes = N * K // 2 + N * (K // 32) * 2
    res = {}
    for M in cfg["Ms"]:
        x = gen.bf16_normal_t(g, (M, K), dev)
        y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(16, w4.w4a16_linear_workspace(M, K, N)), dtype=torch.uint8, device=dev)
        warm_up(lambda i: w4.w4a16_linear(x, qs[i % copies], ss[i % copies], N, y, ws), warmup)
        a, b = TimingEvent(), TimingEvent()
        a.record()
        for i in range(steps):
            w4.w4a16_linear(x, qs[i % copies], ss[i % copies], N, y, ws)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        res["M=%d" % M] = {"us_per_call": ms * 1e3, "weight_GBs": wbytes / (ms * 1e-3) / 1e9,
                           "frac_of_hbm": wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return res


def dense_prefill_report(steps, warmup):
    """w4a16_linear over a 4096-row prompt: 2*M*N*K flops per call against the
    bf16/fp16 MFMA peak."""
    dev = torch.device("cuda:0")
    cfg = gen.DENSE_PREFILL
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    g = gen.torch_generator(dev, 98)
    copies = 8   # 8 x 33 MB of weights > 256 MB last-level cache
    qs = [gen.bytes_uniform_t(g, N * K // 2, dev) for _ in range(copies)]
    ss = [gen.scales_loguniform_t(g, (N, K // 32), dev) for _ in range(copies)]
    x = gen.bf16_normal_t(g, (M, K), dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(16, w4.w4a16_linear_workspace(M, K, N)), dtype=torch.uint8, device=dev)
    warm_up(lambda i: w4.w4a16_linear(x, qs[i % copies], ss[i % copies], N, y, ws), warmup)
    a, b = TimingEvent(), TimingEvent()
    a.record()
    for i in range(steps):
        w4.w4a16_linear(x, qs[i % copies], ss[i % copies], N, y, ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    flops = 2.0 * M * N * K
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": "dense-prefill: w4a16_linear M=%d K=%d N=%d" % (M, K, N), "us_per_call": ms * 1e3,
            "TFLOPs": tf, "flops_per_call": flops,
            "roofline": {"bound": "mfma", "kernel": "w4a16_linear (prefill GEMM, fp16 MFMA on exact s*q)",
                         "achieved": tf, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / BF16_MFMA_PEAK_TFLOPS,
                         "traffic": traffic_of("dense_prefill"), "traffic_source": traffic_source("dense_prefill")}}


# ------------------------------------------------------------------- repack
def repack_layers(layers, dev, gen_seed=5):
    """Generate each layer's on-grid bf16 source on the device, repack it and
    keep only the packed weights.  Returns (packed layers, repack seconds,
    source bytes, off-grid total)."""
    cfg = gen.MOE_E2E
    d, I, E = cfg["d"], cfg["I"], cfg["E"]
    g = gen.torch_generator(dev, gen_seed)
    out = []
    rep_s = 0.0
    src_bytes = 0
    off = torch.zeros(2, dtype=torch.int64, device=dev)
    for l in range(layers):
        w1, _, _ = gen.ongrid_source_t(g, E * 2 * I, d, *cfg["peak"], dev)
        w2, _, _ = gen.ongrid_source_t(g, E * d, I, *cfg["peak"], dev)
        w1q = torch.empty(E * 2 * I * d // 2, dtype=torch.uint8, device=dev)
        w1s = torch.empty(E * 2 * I, d // 32, dtype=torch.bfloat16, device=dev)
        w2q = torch.empty(E * d * I // 2, dtype=torch.uint8, device=dev)
        w2s = torch.empty(E * d, I // 32, dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        a, b = TimingEvent(), TimingEvent()
        a.record()
        w4.q4_group_repack(w1, w1q, w1s, None, off)
        w4.q4_group_repack(w2, w2q, w2s, None, off)
        b.record()
        torch.cuda.synchronize()
        rep_s += a.elapsed_time(b) * 1e-3
        src_bytes += (w1.numel() + w2.numel()) * 2
        del w1, w2
        out.append((w1q, w1s.view(E, 2 * I, d // 32), w2q, w2s.view(E, d, I // 32)))
    return out, rep_s, src_bytes, int(off[0].item())


def repack_export_report():
    """The repack on a realistic export of one MoE layer (fp32 scales, weights
    rounded to bf16): off-grid groups, the fraction of values the repack's
    fp32 dequant reproduces bit for bit, and the worst relative difference --
    the figures the pages report for the real checkpoint (92.6% and 1.1e-2)."""
    dev = torch.device("cuda:0")
    cfg = gen.MOE_E2E
    d, I, E = cfg["d"], cfg["I"], cfg["E"]
    g = gen.torch_generator(dev, 6)
    stats = {"groups": 0, "off_grid_groups": 0, "identical": 0, "values": 0, "worst_rel": 0.0, "repack_s": 0.0}
    off = torch.zeros(2, dtype=torch.int64, device=dev)
    for rows, K in ((E * 2 * I, d), (E * d, I)):
        w, _, _ = gen.ongrid_source_t(g, rows, K, *cfg["peak"], dev, export=True)
        q = torch.empty(rows * K // 2, dtype=torch.uint8, device=dev)
        sc = torch.empty(rows * K // 32, dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        a, b = TimingEvent(), TimingEvent()
        a.record()
        w4.q4_group_repack(w, q, sc, None, off)
        b.record()
        torch.cuda.synchronize()
        stats["repack_s"] += a.elapsed_time(b) * 1e-3
        deq = torch.empty(rows, K, dtype=torch.float32, device=dev)
        w4.q4_group_dequant_f32(q, sc, rows, K, deq)
        src = w.float()
        stats["identical"] += int((deq == src).sum().item())
        stats["values"] += rows * K
        nz = src != 0
        stats["worst_rel"] = max(stats["worst_rel"], float(((deq - src).abs()[nz] / src.abs()[nz]).max().item()))
        stats["groups"] += rows * K // 32
        del w, q, sc, deq, src
    stats["off_grid_groups"] = int(off[0].item())
    stats["bit_identical_frac"] = stats["identical"] / stats["values"]
    stats["groups_per_s"] = stats["groups"] / stats["repack_s"]
    return stats


def repack_report():
    dev = torch.device("cuda:0")
    layers, rep_s, src_bytes, off = repack_layers(gen.MOE_E2E["layers"], dev)
    out_bytes = sum(q.numel() + s.numel() * 2 + q2.numel() + s2.numel() * 2 for q, s, q2, s2 in layers)
    groups = src_bytes // 64
    return {"repack_s": rep_s, "groups": groups, "groups_per_s": groups / rep_s,
            "GBs_read_plus_written": (src_bytes + out_bytes) / rep_s / 1e9, "off_grid_groups": off}


def e2e_report(steps, warmup):
    dev = torch.device("cuda:0")
    cfg = gen.MOE_E2E
    T, d, I, E, k = cfg["T"], cfg["d"], cfg["I"], cfg["E"], cfg["k"]
    layers, rep_s, src_bytes, off = repack_layers(cfg["layers"], dev)
    g = gen.torch_generator(dev, 77)
    x0 = gen.bf16_normal_t(g, (T, d), dev)
    logits = [gen.router_logits_t(g, T, E, dev) for _ in layers]
    ws = torch.empty(w4.w4a16_moe_layer_workspace(T, E, k, d, I), dtype=torch.uint8, device=dev)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=dev)

    x = torch.empty_like(x0)

    def forward():
        x.copy_(x0)
        for l, (w1q, w1s, w2q, w2s) in enumerate(layers):
            w4.w4a16_moe_layer(x, logits[l], k, I, w1q, w1s, w2q, w2s, w4.W4_EPI_GEGLU_TANH, y, ws)
            x.add_(y)   # residual (outside the library): one bf16 add, formed in fp32 and rounded once
        return x

    warm_up(lambda i: forward(), warmup)
    a, b = TimingEvent(), TimingEvent()
    a.record()
    for _ in range(steps):
        forward()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    wbytes = len(layers) * E * (EXPERT_W1_BYTES + EXPERT_W2_BYTES)
    return {"decode_ms_per_step_30_layers": ms, "weight_GBs": wbytes / (ms * 1e-3) / 1e9,
            "repack_s": rep_s, "repack_groups_per_s": (src_bytes // 64) / rep_s, "off_grid_groups": off}


# --------------------------------------------------------------------- main
def copy_report(steps, warmup):
    """A plain device copy of a known size: the reference for converting the
    memory-traffic counters (FETCH_SIZE / WRITE_SIZE) into bytes."""
    dev = torch.device("cuda:0")
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(7)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    warm_up(lambda i: dst.copy_(src), warmup)
    a, b = TimingEvent(), TimingEvent()
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    return {"bytes_read": n, "bytes_written": n, "ms_per_copy": ms, "GBs": 2 * n / (ms * 1e-3) / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="moe-decode",
                    choices=["moe-decode", "moe-prefill", "dense-decode", "dense-prefill", "repack", "repack-export", "e2e",
                             "copy", "fp8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip dense decode, e2e and the ceilings")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only (--gpus must be 1): there is no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    w4.lib()  # fail loudly if the library is not built

    line = {"metric": "MoE W4A16 GMM: weight-HBM GB/s (decode) and TFLOP/s (prefill), % of roofline",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "data": "synthetic (seeded), inputs resident in HBM"}
    if args.workload == "moe-decode":
        log("moe-decode")
        rep, ls = moe_decode_report(args.steps, args.warmup)
        line.update({"value": rep.pop("value"), "unit": "GB/s", "ms_per_step": rep.pop("ms_per_step"),
                     "dtype": "bf16 x int4 (fp32 accumulate)",
                     "config": {"workload": "moe-decode: T=64 tokens, d_model=2816, E=128 experts, top-8, "
                                            "expert hidden 704 (fused gate/up 2816->1408, down 704->2816), "
                                            "int4 group 32 + bf16 scales", "weight_sets_rotated": 3},
                     "roofline": rep.pop("roofline")})
        line["decode"] = rep
        pset = None
        if not args.no_prefill:
            log("moe-prefill")
            pre, pset = moe_prefill_report(max(10, args.steps // 5), max(2, args.warmup // 2), keep=True)
            line["prefill"] = pre
        if not args.no_extras:
            log("dense decode")
            line["dense_decode"] = {"workload": "w4a16_linear K=4096 N=14336, 33,030,144 weight bytes per call",
                                    **dense_decode_report(max(20, args.steps // 2), args.warmup)}
            log("e2e (30-layer repack, then 256-token decode)")
            line["e2e"] = e2e_report(3, 2)
            log("fp8 comparison")
            line["fp8"] = fp8_report(max(20, args.steps // 5), args.warmup, rep["layer_ms_single_call"],
                                     line["prefill"]["layer_ms_single_call"] if "prefill" in line else None)
            log("ceilings")
            line["ceilings"] = ceilings_report()
        if not args.no_cpu_baseline:
            log("cpu baseline (oracle)")
            line["cpu_baseline"] = cpu_baseline_decode(ls)
            line["cpu_baseline_extra"] = cpu_baseline_extra(pset)
    elif args.workload == "moe-prefill":
        pre = moe_prefill_report(args.steps, args.warmup)
        line.update({"value": pre["gmm_TFLOPs"], "unit": "TFLOP/s", "ms_per_step": pre["ms_per_step"],
                     "dtype": "bf16 x int4 (fp32 accumulate)", "config": {"workload": pre.pop("workload")},
                     "roofline": pre.pop("roofline"), "prefill": pre})
    elif args.workload == "dense-decode":
        res = dense_decode_report(args.steps, args.warmup)
        line.update({"value": res["M=16"]["weight_GBs"], "unit": "GB/s", "ms_per_step": res["M=16"]["us_per_call"] / 1e3,
                     "dtype": "bf16 x int4 (fp32 accumulate)",
                     "config": {"workload": "dense-decode: w4a16_linear K=4096 N=14336, M in {1,8,16}"},
                     "dense": res})
    elif args.workload == "dense-prefill":
        res = dense_prefill_report(args.steps, args.warmup)
        line.update({"value": res["TFLOPs"], "unit": "TFLOP/s", "ms_per_step": res["us_per_call"] / 1e3,
                     "dtype": "bf16 x int4 (fp32 accumulate)", "config": {"workload": res.pop("workload")},
                     "roofline": res.pop("roofline"), "dense": res})
    elif args.workload == "repack":
        res = repack_report()
        line.update({"value": res["groups_per_s"], "unit": "groups/s", "ms_per_step": res["repack_s"] * 1e3,
                     "dtype": "fp32 divide / fp64 least squares",
                     "config": {"workload": "repack: 30 layers x 128 experts on-grid bf16 (peak level 4..8)"},
                     "repack": res})
    elif args.workload == "repack-export":
        res = repack_export_report()
        line.update({"value": res["bit_identical_frac"], "unit": "fraction of values bit-identical",
                     "ms_per_step": res["repack_s"] * 1e3, "dtype": "fp32 divide / fp64 least squares",
                     "config": {"workload": "repack-export: one MoE layer (128 experts) exported with fp32 "
                                            "scales and bf16-rounded weights"},
                     "repack": res})
    elif args.workload == "fp8":
        res = fp8_report(args.steps, args.warmup)
        line.update({"value": res["decode"]["layer_weight_GBs"], "unit": "GB/s", "ms_per_step": res["decode"]["layer_ms"],
                     "dtype": "fp8 e4m3 x e4m3 (fp32 accumulate)",
                     "config": {"workload": "fp8: moe-decode and moe-prefill layers over E4M3 experts"}, "fp8": res})
    elif args.workload == "copy":
        res = copy_report(args.steps, args.warmup)
        line.update({"value": res["GBs"], "unit": "GB/s", "ms_per_step": res["ms_per_copy"], "dtype": "u8",
                     "config": {"workload": "copy: device-to-device copy of 512 MiB (counter calibration)"},
                     "copy": res})
    else:
        res = e2e_report(args.steps, args.warmup)
        line.update({"value": res["weight_GBs"], "unit": "GB/s", "ms_per_step": res["decode_ms_per_step_30_layers"],
                     "dtype": "bf16 x int4 (fp32 accumulate)",
                     "config": {"workload": "e2e: repack 30 layers x 128 experts, then T=256 decode through 30 layers"},
                     "e2e": res})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
