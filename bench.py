"""Layer throughput on one MI355X, plus the roofline of the dominant kernel and
the oracle's CPU rate.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only]

Headline workload: the Qwen2.5-7B-shaped layer, one decode step for batch 1
with a 1024-row KV cache (bf16 weights N(0, 0.02), biases N(0, 0.02), gammas
N(1, 0.05), cache and hidden rows N(0, 1); seeded synthetic data). One step =
one qlayer_decode call, i.e. every stage of the layer. The timed loop replays
a HIP graph that holds one call per weight copy, as consecutive layers of a
model run inside one decode-step graph (--eager launches each call directly). Two copies of the
weights and caches alternate between steps so that the 256 MB last-level cache
cannot serve the weight stream. `value` = tokens/s = batch / step time, timed
with events around exactly K steps on the layer's stream.

The other workloads of the config table (prefill and decode at their full
sizes) are timed the same way and reported under "secondary", each with a
per-stage breakdown taken from the library's stage events (eager calls, each
queued behind a short spin kernel so that host launch latency stays outside
the measured windows).

Beside the published peaks, "measured_peaks" gives reference rates taken on
the same GPU through torch (a plain device copy, the vendor library's bf16
matrix-vector and matrix products). MoE workloads also report the rows routed
to each expert in one call ("expert_rows": mean, sd, min, max).

One JSON line is printed on stdout.
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

from transformer_decoder_layer_qwen_amd import configs, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

METRIC = "layer tokens/s (prefill & decode) + % bf16 MFMA / HBM roofline, 1 GPU"
SPACER_CYCLES = 2_000_000   # spin queued ahead of each stage-timed call


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------ HIP events ----

class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        import torch
        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        lib.hipEventCreate.argtypes = [ctypes.POINTER(vp)]
        lib.hipEventSynchronize.argtypes = [vp]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        lib.hipEventDestroy.argtypes = [vp]
        lib.hipEventRecord.argtypes = [vp, vp]
        self.lib = lib

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e.value)
        return evs

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


# ------------------------------------------------------- algorithmic work ----

def stage_work(cfg, wl, stage, cache_len=None):
    """(algorithmic flops, algorithmic HBM bytes) of one stage of one call."""
    d, q, kv, f, dh = cfg.d, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim, cfg.head_dim
    N = wl.tokens
    es = 2
    w_bytes = {"qkv": (q + 2 * kv) * d * es + (2 * (q + 2 * kv) if cfg.qkv_bias else 0),
               "o_proj": d * q * es, "gate_up": 2 * f * d * es, "down": d * f * es}
    if stage in ("qkv", "o_proj", "gate_up", "down"):
        kdim, ncols = {"qkv": (d, q + 2 * kv), "o_proj": (q, d), "gate_up": (d, 2 * f),
                       "down": (f, d)}[stage]
        flops = 2 * N * kdim * ncols
        act = {"qkv": N * d * es + N * (q + 2 * kv) * 4,
               "o_proj": N * q * es + N * d * (es + 4),
               "gate_up": N * d * es + N * f * es,
               "down": N * f * es + N * d * (4 + es)}[stage]
        return flops, w_bytes[stage] + act
    if stage == "attention":
        if wl.kind == "prefill":
            S = wl.seq
            flops = wl.batch * 4 * dh * cfg.n_q_heads * S * (S + 1) // 2
            byts = wl.batch * (S * q * es * 2 + S * 2 * kv * es)
        else:
            L = cache_len + 1
            flops = wl.batch * 4 * dh * cfg.n_q_heads * L
            byts = wl.batch * (L * 2 * kv * es + 2 * q * es)
        return flops, byts
    if stage == "expert_gate_up":
        rows = N * cfg.top_k
        flops = 2 * rows * d * 2 * f
        touched = cfg.n_experts * (1 - (1 - cfg.top_k / cfg.n_experts) ** N)
        return flops, touched * 2 * f * d * es + rows * (d * es + f * es)
    if stage == "expert_down":
        rows = N * cfg.top_k
        flops = 2 * rows * f * d
        touched = cfg.n_experts * (1 - (1 - cfg.top_k / cfg.n_experts) ** N)
        return flops, touched * f * d * es + rows * (f * es + d * 4)
    sf = cfg.shared_ffn_dim
    if stage == "shared_gate_up":
        return 2 * N * d * 2 * sf, 2 * sf * d * es + N * (d * es + sf * es)
    if stage == "shared_down":
        return 2 * N * sf * d, d * sf * es + N * (sf * es + d * 4)
    return 0, 0


def layer_work(cfg, wl):
    stages = ["qkv", "attention", "o_proj"] + (
        ["expert_gate_up", "expert_down"] if cfg.is_moe else ["gate_up", "down"])
    if cfg.shared_ffn_dim:
        stages += ["shared_gate_up", "shared_down"]
    fl = by = 0
    for s in stages:
        a, b = stage_work(cfg, wl, s, cache_len=wl.seq)
        fl += a
        by += b
    if cfg.is_moe:
        by += cfg.n_experts * d_router(cfg)
    return fl, by


def d_router(cfg):
    return cfg.d * 2


# ------------------------------------------------------------- workloads ----

_WEIGHTS = {}


def host_weights(cid):
    """The seeded synthetic weights of a config (the tests' draws), kept for
    the config's other workloads."""
    cfg = configs.CONFIGS[cid]
    if cfg.name not in _WEIGHTS:
        _WEIGHTS.clear()
        t0 = time.time()
        _WEIGHTS[cfg.name] = synth.make_weights(cfg, configs.weight_seed(cid))
        log(f"[bench] {cfg.name}: weights generated in {time.time() - t0:.1f}s")
    return _WEIGHTS[cfg.name]


class Setup:
    """Device weights (n_copies) and inputs of one workload."""

    def __init__(self, cid, wl, n_copies=2):
        import torch
        from transformer_decoder_layer_qwen_amd import binding as B
        self.cfg = cfg = configs.CONFIGS[cid]
        self.wl = wl
        w_np = host_weights(cid)
        self.layers = []
        for _ in range(n_copies):
            self.layers.append(B.QLayer(cfg, B.device_weights(w_np),
                                        max_tokens=wl.tokens if wl.kind == "prefill" else 1,
                                        max_batch=wl.batch if wl.kind == "decode" else 1))
        self.inputs = []
        for c in range(n_copies):
            if wl.kind == "prefill":
                x = B.to_device(synth.make_prefill_input(cfg, wl.seed, wl.batch, wl.seq))
                kc = torch.zeros(wl.batch, wl.seq, cfg.n_kv_heads, cfg.head_dim,
                                 dtype=torch.bfloat16, device="cuda")
                self.inputs.append((x, kc, torch.zeros_like(kc), torch.empty_like(x)))
            else:
                x, kc, vc, lens = synth.make_decode_input(cfg, wl.seed, wl.batch, wl.seq)
                self.inputs.append((B.to_device(x), B.to_device(kc), B.to_device(vc),
                                    torch.from_numpy(lens).cuda(), lens.tolist(),
                                    torch.empty(wl.batch, cfg.d, dtype=torch.bfloat16,
                                                device="cuda")))
        torch.cuda.synchronize()

    def capture(self):
        """One HIP graph holding one full call on each weight copy in turn --
        the way consecutive layers of a model run inside one decode-step
        graph. One replay = len(layers) steps."""
        import torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(len(self.layers)):   # warm the captured code paths
                self.step(c)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(len(self.layers)):
                self.step(c)
        torch.cuda.synchronize()
        return g

    def step(self, i):
        c = i % len(self.layers)
        layer, inp = self.layers[c], self.inputs[c]
        if self.wl.kind == "prefill":
            x, kc, vc, y = inp
            layer.prefill(x, kc, vc, y=y)
        else:
            x, kc, vc, lens, _, y = inp
            layer.decode(x, lens, kc, vc, y=y)

    def close(self):
        for layer in self.layers:
            layer.close()
        self.layers, self.inputs = [], []


def time_steps(setup, hip, steps, warmup, graph=None):
    """Mean time of one call over exactly `steps` calls (a graph replay runs
    one call per weight copy), HIP events around the whole timed region on
    the stream the calls run on."""
    import torch
    n = len(setup.layers)
    if graph is not None:
        assert steps % n == 0, "steps must be a multiple of the number of weight copies"
        run, calls = (lambda i: graph.replay()), steps // n
        wcalls = max(1, warmup // n)
    else:
        run, calls, wcalls = setup.step, steps, warmup
    for i in range(wcalls):
        run(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    a, b = hip.create(2)
    torch.cuda.synchronize()
    hip.record(a, stream)
    for i in range(calls):
        run(i)
    hip.record(b, stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(a, b)
    hip.destroy([a, b])
    return ms / steps


def time_stage(setup, hip, stage, steps):
    """Mean duration of one stage: the library records events immediately
    before its first and after its last kernel, on the call's stream. Each
    call is queued behind a bounded spin kernel, so the host has enqueued the
    whole call before the GPU reaches it and no host launch gap falls inside
    the window."""
    import torch
    evs = hip.create(2 * steps)
    for i in range(steps):
        for layer in setup.layers:
            layer.set_stage_events(stage, evs[2 * i], evs[2 * i + 1])
        torch.cuda._sleep(SPACER_CYCLES)
        setup.step(i)
    torch.cuda.synchronize()
    for layer in setup.layers:
        layer.set_stage_events(None, None, None)
    tot = sum(hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps))
    hip.destroy(evs)
    return tot / steps


def time_stage_graph(setup, hip, stage, reps):
    """Mean duration of one stage inside graph replay: the library's stage
    events are captured into the graph with the calls (one event pair per
    weight copy), the graph is replayed `reps` times and each replay's pairs
    are read after it completes. No host launch gap can fall inside a
    window, and the kernels run back to back as in the timed loop."""
    import torch
    n = len(setup.layers)
    evs = hip.create(2 * n)
    for c, layer in enumerate(setup.layers):
        layer.set_stage_events(stage, evs[2 * c], evs[2 * c + 1])
    try:
        g = setup.capture()
    finally:
        for layer in setup.layers:
            layer.set_stage_events(None, None, None)
    tot, cnt = 0.0, 0
    for r in range(reps + 1):
        g.replay()
        torch.cuda.synchronize()
        if r == 0:
            continue   # the first replay warms up
        for c in range(n):
            tot += hip.elapsed_ms(evs[2 * c], evs[2 * c + 1])
            cnt += 1
    del g
    hip.destroy(evs)
    return tot / cnt


GEMV_MAX_ROWS = 4   # dense decode with this many rows or fewer folds RMSNorm2 into gate/up


def time_empty_span(hip, steps):
    """Mean span of two events recorded back to back behind the same spin
    kernel: the fixed cost that every stage span carries on top of its
    kernels. Stage times below are reported with it subtracted."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    evs = hip.create(2 * steps)
    for i in range(steps):
        torch.cuda._sleep(SPACER_CYCLES)
        hip.record(evs[2 * i], stream)
        hip.record(evs[2 * i + 1], stream)
    torch.cuda.synchronize()
    tot = sum(hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps))
    hip.destroy(evs)
    return tot / steps


def stages_of(cfg, kind, batch):
    # decode with at most GEMV_MAX_ROWS sequences fuses RMSNorm1 into the QKV
    # projection, QK-norm / RoPE / cache append into attention and (dense FFN)
    # RMSNorm2 into gate/up; prefill and larger decode batches run RMSNorm1 on
    # its own and do QK-norm, RoPE and the cache write in the QKV epilogue
    gemv = kind == "decode" and batch <= GEMV_MAX_ROWS
    s = (["qkv"] if gemv else ["rmsnorm1", "qkv"])
    s += ["attention", "o_proj"]
    if not (gemv and not cfg.is_moe):
        s += ["rmsnorm2"]
    s += (["router", "permute", "expert_gate_up", "expert_down"] if cfg.is_moe
          else ["gate_up", "down"])
    if cfg.shared_ffn_dim:
        s += ["shared_gate_up", "shared_down"]
    if cfg.is_moe:
        s += ["combine"]
    return s


# HBM bytes per launch from rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), scaled by what the same counters read for a plain 256 MiB device copy
# (FETCH_SIZE 131084.6 KiB, WRITE_SIZE 262144.0 KiB: factors 1.9998 and 1.0). Keyed by
# (workload, stage); each entry names the source file of the stage's kernels and the first
# 16 hex digits of the SHA-256 of that file with common.h and kernels.h when the counters
# were taken, and is reported only while they are unchanged (else traffic is null).
# Summary: profiles/hbm_counters_decode_workloads.md.
PMC_FETCH_SCALE = 262144.0 / 131084.4
PMC_WRITE_SCALE = 262144.0 / 262144.0
PMC_TRAFFIC_KIB = {
    # (workload, stage): (FETCH_SIZE KiB, WRITE_SIZE KiB, source file, sha256[:16]) per layer
    # call, the stage's kernels summed; profiles/hbm_counters_decode_workloads.md
    ("qwen2.5-7b decode B=1 cache=1024", "qkv"): (16212.3, 72.0, "gemv.hip", "6a126318354a6a7d"),
    ("qwen2.5-7b decode B=1 cache=1024", "attention"): (1766.4, 975.0, "attn_decode.hip", "5eaf26c64e4f6327"),
    ("qwen2.5-7b decode B=1 cache=1024", "o_proj"): (12643.6, 56.0, "gemv.hip", "6a126318354a6a7d"),
    ("qwen2.5-7b decode B=1 cache=1024", "gate_up"): (132730.4, 148.1, "gemv.hip", "6a126318354a6a7d"),
    ("qwen2.5-7b decode B=1 cache=1024", "down"): (66531.3, 56.0, "gemv.hip", "6a126318354a6a7d"),
    ("qwen2.5-7b decode B=32 cache=1024", "rmsnorm1"): (160.9, 448.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen2.5-7b decode B=32 cache=1024", "qkv"): (22392.5, 9152.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen2.5-7b decode B=32 cache=1024", "attention"): (37940.6, 8064.0, "attn_decode.hip", "5eaf26c64e4f6327"),
    ("qwen2.5-7b decode B=32 cache=1024", "o_proj"): (18577.4, 8896.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen2.5-7b decode B=32 cache=1024", "rmsnorm2"): (273.7, 448.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen2.5-7b decode B=32 cache=1024", "gate_up"): (140884.4, 15040.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen2.5-7b decode B=32 cache=1024", "down"): (79226.5, 8800.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-8b decode B=64 cache=4096", "rmsnorm1"): (308.9, 1024.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen3-8b decode B=64 cache=4096", "qkv"): (35060.0, 18944.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-8b decode B=64 cache=4096", "attention"): (532011.5, 5376.0, "attn_decode.hip", "5eaf26c64e4f6327"),
    ("qwen3-8b decode B=64 cache=4096", "o_proj"): (25491.5, 17408.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-8b decode B=64 cache=4096", "rmsnorm2"): (565.7, 1024.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen3-8b decode B=64 cache=4096", "gate_up"): (110272.2, 23552.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-8b decode B=64 cache=4096", "down"): (59540.8, 16896.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-30b-a3b decode B=128 cache=4096", "rmsnorm1"): (289.8, 1024.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen3-30b-a3b decode B=128 cache=4096", "qkv"): (32503.5, 20992.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-30b-a3b decode B=128 cache=4096", "attention"): (535739.6, 10752.0, "attn_decode.hip", "5eaf26c64e4f6327"),
    ("qwen3-30b-a3b decode B=128 cache=4096", "o_proj"): (17811.1, 17408.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-30b-a3b decode B=128 cache=4096", "rmsnorm2"): (545.7, 2048.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen3-30b-a3b decode B=128 cache=4096", "router"): (2652.9, 72.0, "moe.hip", "f52fec8eb3681e2a"),
    ("qwen3-30b-a3b decode B=128 cache=4096", "permute"): (4.9, 10.1, "moe.hip", "f52fec8eb3681e2a"),
    ("qwen3-30b-a3b decode B=128 cache=4096", "expert_gate_up"): (398320.1, 3073.4, "gemm.hip", "c4880637026b08aa"),
    ("qwen3-30b-a3b decode B=128 cache=4096", "expert_down"): (208941.1, 8192.0, "gemm.hip", "c4880637026b08aa"),
    ("qwen3-30b-a3b decode B=128 cache=4096", "combine"): (4645.6, 512.0, "moe.hip", "f52fec8eb3681e2a"),
    ("qwen3-30b-a3b decode B=128 cache=1024", "rmsnorm1"): (289.9, 1024.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen3-30b-a3b decode B=128 cache=1024", "qkv"): (32502.6, 20992.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-30b-a3b decode B=128 cache=1024", "attention"): (139268.4, 10752.0, "attn_decode.hip", "5eaf26c64e4f6327"),
    ("qwen3-30b-a3b decode B=128 cache=1024", "o_proj"): (17811.1, 17408.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-30b-a3b decode B=128 cache=1024", "rmsnorm2"): (545.7, 2048.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen3-30b-a3b decode B=128 cache=1024", "router"): (2652.9, 72.0, "moe.hip", "f52fec8eb3681e2a"),
    ("qwen3-30b-a3b decode B=128 cache=1024", "permute"): (4.9, 10.1, "moe.hip", "f52fec8eb3681e2a"),
    ("qwen3-30b-a3b decode B=128 cache=1024", "expert_gate_up"): (395321.6, 3073.7, "gemm.hip", "c4880637026b08aa"),
    ("qwen3-30b-a3b decode B=128 cache=1024", "expert_down"): (207405.2, 8192.1, "gemm.hip", "c4880637026b08aa"),
    ("qwen3-30b-a3b decode B=128 cache=1024", "combine"): (4645.5, 512.0, "moe.hip", "f52fec8eb3681e2a"),
    ("qwen3-32b decode B=32 cache=4096", "rmsnorm1"): (229.0, 640.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen3-32b decode B=32 cache=4096", "qkv"): (57594.7, 10496.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-32b decode B=32 cache=4096", "attention"): (270961.6, 9728.0, "attn_decode.hip", "5eaf26c64e4f6327"),
    ("qwen3-32b decode B=32 cache=4096", "o_proj"): (48161.9, 9344.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-32b decode B=32 cache=4096", "rmsnorm2"): (386.7, 640.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen3-32b decode B=32 cache=4096", "gate_up"): (265878.7, 17536.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen3-32b decode B=32 cache=4096", "down"): (140794.7, 9024.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("mixtral-like decode B=64 cache=2048", "rmsnorm1"): (308.8, 1024.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("mixtral-like decode B=64 cache=2048", "qkv"): (35057.3, 18944.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("mixtral-like decode B=64 cache=2048", "attention"): (267923.5, 5376.0, "attn_decode.hip", "5eaf26c64e4f6327"),
    ("mixtral-like decode B=64 cache=2048", "o_proj"): (25491.5, 17408.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("mixtral-like decode B=64 cache=2048", "rmsnorm2"): (565.7, 2048.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("mixtral-like decode B=64 cache=2048", "router"): (692.9, 3.0, "moe.hip", "f52fec8eb3681e2a"),
    ("mixtral-like decode B=64 cache=2048", "permute"): (3.2, 1.2, "moe.hip", "f52fec8eb3681e2a"),
    ("mixtral-like decode B=64 cache=2048", "expert_gate_up"): (266353.2, 2048.0, "gemm.hip", "c4880637026b08aa"),
    ("mixtral-like decode B=64 cache=2048", "expert_down"): (139305.1, 2048.0, "gemm.hip", "c4880637026b08aa"),
    ("mixtral-like decode B=64 cache=2048", "combine"): (1561.5, 512.0, "moe.hip", "f52fec8eb3681e2a"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "rmsnorm1"): (272.8, 896.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "qkv"): (28523.3, 18304.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "attention"): (72277.7, 8512.0, "attn_decode.hip", "5eaf26c64e4f6327"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "o_proj"): (24511.3, 17792.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "rmsnorm2"): (497.8, 1792.0, "rmsnorm.hip", "8b0d9a0232539a0f"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "router"): (1971.5, 24.2, "moe.hip", "f52fec8eb3681e2a"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "permute"): (3.9, 5.1, "moe.hip", "f52fec8eb3681e2a"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "expert_gate_up"): (1150526.8, 5120.0, "gemm.hip", "c4880637026b08aa"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "expert_down"): (594007.0, 7168.0, "gemm.hip", "c4880637026b08aa"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "shared_gate_up"): (158065.8, 29696.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "shared_down"): (98819.2, 18048.0, "gemm2.hip", "c99046ea5ffdae45"),
    ("qwen2-57b-a14b decode B=64 cache=1024", "combine"): (4067.5, 448.0, "moe.hip", "f52fec8eb3681e2a"),
}


def source_sha(name):
    """First 16 hex digits of the SHA-256 of a kernel source together with the
    headers every kernel includes (common.h, kernels.h): a change to either
    changes the kernel, and its counter readings no longer apply."""
    import hashlib
    csrc = os.path.join(ROOT, "transformer_decoder_layer_qwen_amd", "csrc")
    h = hashlib.sha256()
    for f in (name, "common.h", "kernels.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(wl, stage):
    t = PMC_TRAFFIC_KIB.get((wl.label, stage))
    if t is None or source_sha(t[2]) != t[3]:
        return None
    return int((t[0] * PMC_FETCH_SCALE + t[1] * PMC_WRITE_SCALE) * 1024)


def roofline_entry(cfg, wl, stage, ms):
    fl, by = stage_work(cfg, wl, stage, cache_len=wl.seq)
    hbm_bound = wl.kind == "decode" or fl / max(by, 1) < 315
    if hbm_bound:
        ach = by / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": pmc_traffic(wl, stage),
                "algorithmic_bytes": int(by), "kernel_ms": round(ms, 5), "stage": stage}
    ach = fl / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
            "algorithmic_flops": int(fl), "kernel_ms": round(ms, 5), "stage": stage}


def run_workload(cid, wl, hip, steps, warmup, stage_steps, breakdown=True, use_graph=True,
                 graph_stage_probe=False):
    setup = Setup(cid, wl)
    cfg = setup.cfg
    graph = setup.capture() if use_graph else None
    ms = time_steps(setup, hip, steps, warmup, graph)
    del graph
    out = {"workload": wl.label, "kind": wl.kind, "batch": wl.batch, "hip_graph": use_graph,
           "seq_or_cache": wl.seq, "tokens_per_step": wl.tokens,
           "ms_per_step": round(ms, 5), "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1)}
    fl, by = layer_work(cfg, wl)
    if wl.kind == "prefill":
        out["layer_tflops"] = round(fl / (ms * 1e-3) / 1e12, 1)
        out["layer_frac_mfma"] = round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    else:
        out["layer_gbs"] = round(by / (ms * 1e-3) / 1e9, 1)
        out["layer_frac_hbm"] = round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if breakdown:
        st = {}
        empty = time_empty_span(hip, max(stage_steps, 8))
        for s in stages_of(cfg, wl.kind, wl.batch):
            st[s] = round(max(time_stage(setup, hip, s, stage_steps) - empty, 1e-6), 5)
        out["stage_ms"] = st
        out["event_span_overhead_ms"] = round(empty, 5)
        if graph_stage_probe:
            out["stage_ms_graph"] = {s: round(time_stage_graph(setup, hip, s, stage_steps), 5)
                                     for s in st}
        dom = max(st, key=st.get)
        out["dominant"] = roofline_entry(cfg, wl, dom, st[dom])
        gemms = [s for s in ("qkv", "o_proj", "gate_up", "down", "expert_gate_up",
                             "expert_down", "shared_gate_up", "shared_down") if s in st]
        out["stage_roofline"] = {s: roofline_entry(cfg, wl, s, st[s]) for s in gemms + ["attention"]}
    if cfg.is_moe:
        out["expert_rows"] = expert_rows(setup)
    setup.close()
    return out, setup


def gpu_weights(cfg, seed):
    """A layer's synthetic weights drawn on the GPU (torch's generator, seeded),
    with synth's distributions: gammas N(gamma_mean, gamma_std), weights and
    biases N(0, w_std / b_std), router N(0, router_std), rounded to bf16. For
    the layer stack, whose 28 layers (13 GB) would take minutes to draw on the
    host; the single-layer workloads use synth's host draws."""
    import torch
    from transformer_decoder_layer_qwen_amd import synth as sy
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    out = {}
    for name, shape in sy.weight_shapes(cfg).items():
        if name.endswith("_g"):
            mean, std = cfg.gamma_mean, cfg.gamma_std
        elif name in ("bq", "bk", "bv"):
            mean, std = 0.0, cfg.b_std
        elif name == "w_router":
            mean, std = 0.0, cfg.router_std
        else:
            mean, std = 0.0, cfg.w_std
        t = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
        out[name] = (t * std + mean).to(torch.bfloat16).contiguous()
    return out


def run_stack(hip, n_layers, steps, warmup, cache_len=1024):
    """One decode step (batch 1) through a stack of `n_layers` Qwen2.5-7B
    layers, each with its own synthetic weights and KV cache, captured as one
    HIP graph and replayed: the single-stream decode of the model's trunk
    ("Qwen2.5-7B 结构拆解" §11: tokens/s is bounded by HBM bandwidth over the
    bytes read per step)."""
    import torch
    from transformer_decoder_layer_qwen_amd import binding as B
    cfg = configs.QWEN25_7B
    t0 = time.time()
    layers, ks, vs = [], [], []
    T_max = cache_len + 1
    for l in range(n_layers):
        layers.append(B.QLayer(cfg, gpu_weights(cfg, 20000 + l), max_tokens=1, max_batch=1))
        k = torch.randn(1, T_max, cfg.n_kv_heads, cfg.head_dim, device="cuda").to(torch.bfloat16)
        ks.append(k)
        vs.append(torch.randn_like(k, dtype=torch.float32).to(torch.bfloat16))
    x = torch.randn(1, cfg.d, device="cuda").to(torch.bfloat16)
    y, tmp = torch.empty_like(x), torch.empty_like(x)
    lens = torch.full((1,), cache_len, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] {n_layers}-layer stack: weights and caches in {time.time() - t0:.1f}s")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.decode_stack(layers, x, lens, ks, vs, y=y, tmp=tmp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.decode_stack(layers, x, lens, ks, vs, y=y, tmp=tmp)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    a, b = hip.create(2)
    hip.record(a, stream)
    for _ in range(steps):
        g.replay()
    hip.record(b, stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(a, b) / steps
    hip.destroy([a, b])
    wl = configs.Workload(2, 1, "decode", 1, cache_len)
    _, layer_bytes = layer_work(cfg, wl)
    step_bytes = n_layers * layer_bytes
    gbs = step_bytes / (ms * 1e-3) / 1e9
    for ly in layers:
        ly.close()
    del g, layers, ks, vs
    torch.cuda.empty_cache()
    return {"workload": f"qwen2.5-7b {n_layers}-layer decode stack B=1 cache={cache_len}",
            "kind": "decode_stack", "layers": n_layers, "hip_graph": True,
            "ms_per_step": round(ms, 5), "tokens_per_s": round(1.0 / (ms * 1e-3), 1),
            "bytes_per_step": int(step_bytes), "achieved_GBs": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "single_stream_bound_tokens_per_s": round(HBM_PEAK_GBS * 1e9 / step_bytes, 1),
            "weights": "per-layer synthetic, drawn on the GPU (torch generator, seeds 20000+l)"}


def expert_rows(setup):
    """Rows routed to each expert in one call: the router logits are tapped
    from the library (fp32, as the top-k reads them) and the top-k taken here.
    Returns mean, standard deviation, min and max over the experts."""
    import torch
    cfg, wl = setup.cfg, setup.wl
    lg = torch.empty(wl.tokens, cfg.n_experts, dtype=torch.float32, device="cuda")
    layer = setup.layers[0]
    layer.set_taps(logits=lg)
    setup.step(0)
    torch.cuda.synchronize()
    layer.set_taps()
    l = lg.cpu().numpy()
    top = np.argpartition(-l, cfg.top_k - 1, axis=1)[:, :cfg.top_k]
    cnt = np.bincount(top.ravel(), minlength=cfg.n_experts)
    return {"mean": round(float(cnt.mean()), 2), "sd": round(float(cnt.std()), 2),
            "min": int(cnt.min()), "max": int(cnt.max()), "experts": int(cfg.n_experts)}


def measured_peaks():
    """Reference rates measured on this GPU, beside the published peaks: a
    plain 1 GiB device copy (read + write bytes), the vendor library's bf16
    matrix-vector product on the headline gate/up weight shape (37888 x 3584,
    read bytes), and its bf16 8192^3 matrix product, all through torch. Best
    of 5, events on the current stream."""
    import torch
    def best_ms(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b))
        return min(t)
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    copy_ms = best_ms(lambda: dst.copy_(src))
    del src, dst
    rows, cols = 2 * 18944, 3584
    wmat = torch.randn(rows, cols, dtype=torch.bfloat16, device="cuda")
    xv = torch.randn(cols, dtype=torch.bfloat16, device="cuda")
    mv_ms = best_ms(lambda: torch.mv(wmat, xv))
    del wmat, xv
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    mm_ms = best_ms(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.empty_cache()
    return {"copy_GBs": round(2 * n / (copy_ms * 1e-3) / 1e9, 1),
            "vendor_gemv_GBs": round(2 * rows * cols / (mv_ms * 1e-3) / 1e9, 1),
            "bf16_matmul_TFLOPs": round(2 * m ** 3 / (mm_ms * 1e-3) / 1e12, 1),
            "method": "torch: 1 GiB copy_; mv bf16 37888x3584; matmul bf16 8192^3; best of 5"}


# ------------------------------------------------------------ CPU oracle ----

def cpu_info():
    model = "unknown"
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
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = len(os.sched_getaffinity(0))
    return model, int(cores)


def oracle_spec(cfg):
    from oracle import qlayer_ref as ref
    return ref.LayerSpec(d=cfg.d, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                         head_dim=cfg.head_dim, ffn_dim=cfg.ffn_dim, n_experts=cfg.n_experts,
                         top_k=cfg.top_k, norm_topk_prob=cfg.norm_topk_prob,
                         shared_ffn_dim=cfg.shared_ffn_dim, qkv_bias=cfg.qkv_bias,
                         qk_norm=cfg.qk_norm, eps=cfg.rms_eps, theta=cfg.rope_theta)


def cpu_oracle(cid, wl, seconds=3.0):
    """The fp64 oracle, as it stands, on a bounded sample of one workload:
    decode steps of up to 4 of its sequences (full cache length), or the
    prefill of the first min(S, 256) rows of one sequence; repeated for about
    `seconds`. Tokens per second of that sample (a baseline only)."""
    from oracle import qlayer_ref as ref
    cfg = configs.CONFIGS[cid]
    w = {k: synth.to_f32(v) for k, v in host_weights(cid).items()}
    spec = oracle_spec(cfg)
    if wl.kind == "prefill":
        S = min(wl.seq, 256)
        x = synth.to_f32(synth.make_prefill_input(cfg, wl.seed, 1, S))
        run, toks, what = (lambda: ref.layer_prefill(x, w, spec)), S, f"prefill of {S} rows"
    else:
        Bs = min(wl.batch, 4)
        x, kc, vc, lens = synth.make_decode_input(cfg, wl.seed, Bs, wl.seq)
        x, kc, vc = synth.to_f32(x), synth.to_f32(kc), synth.to_f32(vc)
        run, toks, what = (lambda: ref.layer_decode(x, kc, vc, lens, w, spec)), Bs, \
            f"decode step of {Bs} sequences at cache {wl.seq}"
    n, t0 = 0, time.time()
    while True:
        run()
        n += 1
        if time.time() - t0 >= seconds:
            break
    dt = time.time() - t0
    return {"value": round(n * toks / dt, 3), "unit": "tokens/s", "kind": "oracle",
            "sample": f"{n} x {what} in {dt:.1f}s"}

def cpu_baseline(seconds=12.0):
    """The fp64 oracle, as it stands, on the headline workload: repeated decode
    steps of the Qwen2.5-7B layer at batch 1 with a 1024-row cache."""
    from oracle import qlayer_ref as ref
    model, cores = cpu_info()
    cid, wl = 2, configs.WORKLOADS[2][0]
    cfg = configs.CONFIGS[cid]
    w = {k: synth.to_f32(v) for k, v in host_weights(cid).items()}
    x, kc, vc, lens = synth.make_decode_input(cfg, wl.seed, wl.batch, wl.seq)
    x, kc, vc = synth.to_f32(x), synth.to_f32(kc), synth.to_f32(vc)
    spec = ref.LayerSpec(d=cfg.d, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                         head_dim=cfg.head_dim, ffn_dim=cfg.ffn_dim, qkv_bias=cfg.qkv_bias,
                         qk_norm=cfg.qk_norm, eps=cfg.rms_eps, theta=cfg.rope_theta)
    n = 0
    t0 = time.time()
    while True:
        ref.layer_decode(x, kc, vc, lens, w, spec)
        n += 1
        if time.time() - t0 >= seconds:
            break
    dt = time.time() - t0
    return {"value": round(n * wl.batch / dt, 3), "unit": "tokens/s", "cores": int(cores),
            "cpu": model, "kind": "oracle",
            "sample": f"{n} decode steps of {wl.label} (fp64 NumPy oracle, weights pre-widened "
                      f"to fp32) in {dt:.1f}s"}


# ------------------------------------------------------------------ main ----

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-steps", type=int, default=10)
    ap.add_argument("--eager", action="store_true", help="no HIP graph replay")
    ap.add_argument("--stack-layers", type=int, default=28,
                    help="layers of the decode-stack workload (0: skip it)")
    ap.add_argument("--graph-stage-probe", action="store_true",
                    help="also time every stage with events captured in graph replay")
    ap.add_argument("--only", default=None,
                    help="time one workload CID:INDEX of the config table instead of the headline")
    ap.add_argument("--copy-ref", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (a known-size reference "
                         "for the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: "
              "data-parallel ranks each run their own sequences with no exchange, so the "
              "per-GPU kernels are exactly the ones measured here", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_ref:
        n = args.copy_ref << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy reference: 5 copies of {n} bytes")
        return
    hip = HipEvents()

    cid, wl = 2, configs.WORKLOADS[2][0]
    if args.only:
        c, i = (int(v) for v in args.only.split(":"))
        w = [x for x in configs.WORKLOADS[c] if x.index == i][0]
        r, _ = run_workload(c, w, hip, args.steps, args.warmup, args.stage_steps,
                            use_graph=not args.eager)
        print(json.dumps(r), flush=True)
        return
    head, _ = run_workload(cid, wl, hip, args.steps, args.warmup, args.stage_steps,
                           use_graph=not args.eager, graph_stage_probe=args.graph_stage_probe)
    log(f"[bench] headline {head['workload']}: {head['tokens_per_s']} tok/s, "
        f"{head['ms_per_step']} ms/step")
    secondary = []
    if not args.headline_only:
        # the graded configs (Qwen2.5-7B, Qwen3-8B, Qwen3-30B-A3B), then the
        # shape variants (Qwen3-32B, the Mixtral-like layer, Qwen2-57B-A14B)
        for c in (2, 3, 4, 5, 6, 7, 8):
            for w in configs.WORKLOADS[c]:
                if (c, w.index) == (cid, wl.index):
                    continue
                s_steps = max(6, args.steps // 5 // 2 * 2) if w.kind == "prefill" else args.steps
                r, _ = run_workload(c, w, hip, s_steps, max(2, args.warmup // 2),
                                    max(3, args.stage_steps // 2), use_graph=not args.eager)
                if not args.no_cpu_baseline:
                    r["cpu_oracle"] = cpu_oracle(c, w)
                log(f"[bench] {r['workload']}: {r['tokens_per_s']} tok/s, "
                    f"{r['ms_per_step']} ms/step")
                secondary.append(r)
                torch.cuda.empty_cache()
        if args.stack_layers:
            r = run_stack(hip, args.stack_layers, max(10, args.steps // 2), 3)
            log(f"[bench] {r['workload']}: {r['tokens_per_s']} tok/s, {r['achieved_GBs']} GB/s")
            secondary.append(r)

    cfg = configs.CONFIGS[cid]
    dom = dict(head["dominant"])
    roof = {k: dom[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof["kernel"] = dom["stage"]
    roof["kernel_ms"] = dom["kernel_ms"]
    peaks = measured_peaks()
    log(f"[bench] measured peaks: {peaks}")
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.label, "batch": wl.batch, "cache_len": wl.seq, "d": cfg.d,
                   "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "ffn_dim": cfg.ffn_dim, "qkv_bias": cfg.qkv_bias,
                   "weight_copies_rotated": 2, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer_frac_hbm": head.get("layer_frac_hbm"),
        "stage_ms": head.get("stage_ms"),
        "event_span_overhead_ms": head.get("event_span_overhead_ms"),
        "stage_ms_graph": head.get("stage_ms_graph"),
        "secondary": secondary,
        "measured_peaks": peaks,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
