#!/usr/bin/env python3
"""Benchmark of the mixed-head KV-cache attention path on one MI355X.

Decode leg (the headline number): Llama-3-8B-shaped decode, batch 8, 32768 valid tokens, 32 q / 8 kv
heads, 4 retrieval kv heads, sink 64 / recent 256, bf16, pages of 16. One step = append one token
per sequence (kv_append_circular) + duo_attn_decode. Four layers' caches are rotated so that every
step reads cache lines last touched >1.5 GB earlier (the 256 MB Infinity Cache cannot serve them).
value = algorithmic decode bytes per step / wall time per step.

Int8 and 4-bit decode legs: the same decode workload over the int8 cache (kv_append_circular_int8 +
duo_attn_decode_int8; 8-bit codes plus one fp32 scale per slot for K and V) and over the 4-bit cache
(kv_append_circular_int4 + duo_attn_decode_int4; 4-bit codes with per-channel scales), reported in
the same algorithmic GB/s (codes + scales + block table + q/out) and as step-time speedups over bf16.

Prefill leg: Llama-2-7B-shaped MHA chunked prefill, eight 4096-token chunks building a 32768-token
context, 8 of 32 heads retrieval, sink 128 / recent 1024. One pass = 8 x (append chunk + prefill).
Reported as algorithmic TFLOP/s (4 * head_dim per visible (query, key) pair).

Inputs are seeded synthetic tensors (synth/), already resident in HBM when timing starts.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "decode attn HBM GB/s + prefill TFLOP/s (% of MI355X roofline), mixed heads"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6   # dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk/CU)
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SAMPLES = 32              # decode launches timed with HIP events, in a pass of their own
FLUSH_BYTES = 1 << 30            # read before each sampled launch: more than L2 + Infinity Cache
_DECODE_SRC = ["decode.hip", "decode_body.h", "duo_common.h", "duo_kernels.h"]
_PREFILL_SRC = ["prefill.hip", "decode_body.h", "duo_common.h", "duo_kernels.h"]
KERNEL_SOURCES = {
    "decode": _DECODE_SRC,
    "decode_int8": _DECODE_SRC,
    "decode_int4": _DECODE_SRC,
    "prefill": _PREFILL_SRC,
    "dca": _PREFILL_SRC,
    "gemma": _DECODE_SRC,
    "1m": _DECODE_SRC,
    "cb": _PREFILL_SRC,
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "kv_cache_sparsity_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match the source."""
    try:
        with open(COUNTERS) as fh:
            c = json.load(fh).get(kernel)
    except (OSError, ValueError):
        return None
    if not c or c.get("source_sha") != source_sha(kernel):
        return None
    return c.get("hbm_bytes_per_launch")


# ---- algorithmic units ---------------------------------------------------------------------------
def visible_count(p: np.ndarray, retrieval: bool, sink: int, recent: int) -> np.ndarray:
    """Number of keys a query at position p sees (union of sinks and the recent window)."""
    p = np.asarray(p, dtype=np.int64)
    n = np.maximum(p + 1, 0)
    if retrieval:
        return n
    a = np.minimum(sink, n)                               # [0, min(sink, p+1))
    b_lo = np.maximum(p - recent + 1, 0)
    b = np.maximum(p + 1 - b_lo, 0)                       # [b_lo, p+1)
    overlap = np.maximum(np.minimum(sink, p + 1) - b_lo, 0)
    return a + b - overlap


def decode_bytes(w: synth.Workload, lens: np.ndarray, int8_cache: bool = False,
                 int4_cache: bool = False) -> int:
    """K+V rows each head must read + q + out + block-table entries. With the int8 cache a key's
    K+V row is 2 * head_dim one-byte codes plus its two fp32 scales; with the 4-bit cache it is
    head_dim bytes of codes, and the per-channel scales (2 * head_dim fp32 per kv head) are read
    once per call."""
    if int4_cache:
        row = w.head_dim
    elif int8_cache:
        row = 2 * w.head_dim + 2 * 4
    else:
        row = 2 * w.head_dim * w.elem_bytes
    total = 0
    for b in range(w.batch):
        L = int(lens[b])
        for h in range(w.num_kv_heads):
            ret = h in w.retrieval
            n = int(visible_count(np.array([L - 1]), ret, w.sink, w.recent)[0])
            total += n * row
            if ret:
                pages = -(-L // w.block_size)
            else:
                sink_pages = -(-min(w.sink, L) // w.block_size)
                lo = max(w.sink, L - w.recent)
                ring_pages = 0
                if L > w.sink:
                    ring_pages = (L - 1 - w.sink) // w.block_size - (lo - w.sink) // w.block_size + 1
                pages = sink_pages + ring_pages
            total += pages * 4
    total += 2 * w.batch * w.num_q_heads * w.head_dim * w.elem_bytes
    if int4_cache:
        total += 2 * w.num_kv_heads * w.head_dim * 4
    return total


def prefill_flops(w: synth.Workload, L: int, q_len: int) -> int:
    p = np.arange(L - q_len, L)
    total = 0
    for hq in range(w.num_q_heads):
        ret = (hq // w.group) in w.retrieval
        total += int(visible_count(p, ret, w.sink, w.recent).sum())
    return 4 * w.head_dim * total * w.batch


# ---- device helpers --------------------------------------------------------------------------
def event_pair(torch):
    """Two timing events, recorded once so that they exist, to hand to duo.profile_next_launch:
    the library's next attention launch records them at its kernel's own start and end."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    return a, b


def to_dev(torch, arr, dtype, device):
    if dtype == synth.F32:
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device)
    return t.view(torch.bfloat16 if dtype == synth.BF16 else torch.float16)


def logical_bits(w, L, which):
    out = np.empty((w.batch, w.num_kv_heads, L, w.head_dim), dtype=synth.storage_np_dtype(w.dtype))
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            out[b, h] = synth.f32_to_storage(synth.kv_tokens(w, which, b, h, 0, L), w.dtype)
    return out


def torch_dtype(torch, dtype):
    return {synth.F32: torch.float32, synth.F16: torch.float16, synth.BF16: torch.bfloat16}[dtype]


# ---- decode leg ------------------------------------------------------------------------------
def spread_us(times_s):
    """Median and 90th percentile of sampled kernel durations (seconds in, microseconds out)."""
    return {"kernel_us_median": round(float(np.median(times_s)) * 1e6, 2),
            "kernel_us_p90": round(float(np.percentile(times_s, 90)) * 1e6, 2),
            "kernel_samples": len(times_s)}


class Flusher:
    """Reads FLUSH_BYTES of device memory (a reduction over a buffer no leg uses), which pushes the
    decode's earlier lines out of the L2s and the 256 MB Infinity Cache. A read leaves no dirty
    lines behind, so the next kernel pays no write-backs of the flush."""

    def __init__(self, torch):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.sink = None

    def __call__(self):
        self.sink = self.buf.sum()


def sample_kernels(torch, step, first: int, n: int, flush):
    """n steps, each preceded by a flush (outside the events) and with HIP events attached to its
    attention dispatch; returns the kernel durations in seconds, in step order."""
    evs = [event_pair(torch) for _ in range(n)]
    for i, ev in enumerate(evs):
        flush()
        step(first + i, ev)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e-3 for a, b in evs]


def decode_leg(args, torch, duo):
    w = synth.llama3_8b_decode()
    dev = torch.device("cuda:0")
    L = w.context
    log(f"[decode] generating {w.name}")
    K = logical_bits(w, L, synth.S_K)
    V = logical_bits(w, L, synth.S_V)
    table_h, nblocks = synth.block_table(w)
    table = torch.from_numpy(table_h).to(dev)
    mask = w.retrieval_mask
    tdt = torch_dtype(torch, w.dtype)
    ks = (nblocks, w.block_size, w.head_dim)
    vs = (nblocks, w.head_dim, w.block_size)
    layers = []
    zero = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    after = torch.empty_like(zero)
    for li in range(args.layers):
        kp = torch.empty(ks, dtype=tdt, device=dev)
        vp = torch.empty(vs, dtype=tdt, device=dev)
        if li == 0:
            for s in range(0, L - 1, 8192):
                e = min(L - 1, s + 8192)
                kn = to_dev(torch, K[:, :, s:e].transpose(0, 2, 1, 3), w.dtype, dev)
                vn = to_dev(torch, V[:, :, s:e].transpose(0, 2, 1, 3), w.dtype, dev)
                lb = torch.full((w.batch,), s, dtype=torch.int32, device=dev)
                duo.kv_append_circular(kp, vp, table, kn, vn, lb, after, mask, w.sink, w.recent,
                                       w.ring_blocks)
        else:
            kp.copy_(layers[0][0])
            vp.copy_(layers[0][1])
        layers.append((kp, vp))
    # the token decoded at every step (position L-1) and its query
    k_tok = to_dev(torch, K[:, :, L - 1:L].transpose(0, 2, 1, 3), w.dtype, dev)
    v_tok = to_dev(torch, V[:, :, L - 1:L].transpose(0, 2, 1, 3), w.dtype, dev)
    q_bits = synth.f32_to_storage(synth.queries(w, 0, q_len=1)[:, 0], w.dtype)
    q = to_dev(torch, q_bits, w.dtype, dev)
    out = torch.empty_like(q)
    ws = duo.decode_workspace(q, table, w.block_size)
    lens_before = torch.full((w.batch,), L - 1, dtype=torch.int32, device=dev)
    lens = torch.empty_like(lens_before)
    torch.cuda.synchronize()

    def step(i, ev=None):
        kp, vp = layers[i % len(layers)]
        duo.kv_append_circular(kp, vp, table, k_tok, v_tok, lens_before, lens, mask, w.sink,
                               w.recent, w.ring_blocks)
        if ev is not None:
            duo.profile_next_launch(ev[0], ev[1])
        duo.duo_attn_decode(q, kp, vp, table, lens, mask, w.sink, w.recent, w.ring_blocks,
                            w.scale, out, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The timed steps run back to back without events, as a serving loop would; the kernel's own
    # duration comes from a separate pass of KERNEL_SAMPLES steps with HIP events on the decode
    # dispatch, each after a flush.
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    kern_all = sample_kernels(torch, step, args.warmup + args.steps, KERNEL_SAMPLES, args.flush)
    kern_s = float(np.mean(kern_all))
    nbytes = decode_bytes(w, np.full(w.batch, L))
    traffic = measured_traffic("decode")

    # The same step as one launch (duo_attn_append_decode: the append fused into the decode),
    # timed the same way, back to back.
    lens_fused = torch.empty_like(lens_before)

    def fused_step(i):
        kp, vp = layers[i % len(layers)]
        duo.duo_attn_append_decode(q, k_tok, v_tok, kp, vp, table, lens_before, lens_fused, mask,
                                   w.sink, w.recent, w.ring_blocks, w.scale, out, ws)

    for i in range(args.warmup):
        fused_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fused_step(args.warmup + i)
    torch.cuda.synchronize()
    fused_s = (time.perf_counter() - t0) / args.steps
    res = {
        "w": w, "K": K, "V": V, "q_bits": q_bits, "out": out,
        "value": nbytes / step_s / 1e9, "ms_per_step": step_s * 1e3, "bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(nbytes / kern_s / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / kern_s / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "duo::decode_kernel<bf16,128>",
                     "kernel_us": round(kern_s * 1e6, 2),
                     **spread_us(kern_all),
                     "cold": f"{FLUSH_BYTES >> 20} MiB read before each sampled launch",
                     "algorithmic_bytes_per_launch": nbytes},
        "fused_step": {"call": "duo_attn_append_decode (1 token/seq, one launch)",
                       "us_per_step": round(fused_s * 1e6, 2),
                       "GB/s": round(nbytes / fused_s / 1e9, 1)},
    }
    log(f"[decode] step {step_s * 1e6:.1f} us, kernel {kern_s * 1e6:.1f} us, "
        f"{res['value']:.0f} GB/s per step, {nbytes / kern_s / 1e9:.0f} GB/s kernel; "
        f"fused step {fused_s * 1e6:.1f} us")
    return res


def decode_shape_leg(args, torch, duo, w, lens_seq, n_layers, steps, tag):
    """Timing of append (one token per sequence) + decode on another decode workload.

    The pools are filled on the device with N(0,1) values (the workloads' distribution; the scores
    must be realistic, since the online softmax rescales only when the running max moves). Parity
    at these shapes, garbage past the valid lengths included, is covered by the GPU tests.
    lens_seq[k] = the lengths after step k's append. n_layers caches are rotated so that every
    step reads lines the Infinity Cache does not hold."""
    dev = torch.device("cuda:0")
    log(f"[{tag}] {w.name}: {n_layers} layer caches")
    identity = w.sink == 0 and len(w.retrieval) == w.num_kv_heads and w.num_kv_heads == 1
    table_h, nblocks = synth.block_table(w, identity=identity)
    table = torch.from_numpy(table_h).to(dev)
    mask = w.retrieval_mask
    tdt = torch_dtype(torch, w.dtype)
    layers = []
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    for _ in range(n_layers):
        kp = torch.randn((nblocks, w.block_size, w.head_dim), generator=g, device=dev).to(tdt)
        vp = torch.randn((nblocks, w.head_dim, w.block_size), generator=g, device=dev).to(tdt)
        layers.append((kp, vp))
    k_tok = torch.randn((w.batch, 1, w.num_kv_heads, w.head_dim), generator=g, device=dev).to(tdt)
    v_tok = torch.randn((w.batch, 1, w.num_kv_heads, w.head_dim), generator=g, device=dev).to(tdt)
    q = torch.randn((w.batch, w.num_q_heads, w.head_dim), generator=g, device=dev).to(tdt)
    out = torch.empty_like(q)
    ws = duo.decode_workspace(q, table, w.block_size)
    after = [torch.from_numpy(np.asarray(x, dtype=np.int32)).to(dev) for x in lens_seq]
    before = [a - 1 for a in after]
    lens_tmp = torch.empty_like(after[0])
    torch.cuda.synchronize()

    def step(i, ev=None):
        kp, vp = layers[i % n_layers]
        j = i % len(after)
        duo.kv_append_circular(kp, vp, table, k_tok, v_tok, before[j], lens_tmp, mask, w.sink,
                               w.recent, w.ring_blocks)
        if ev is not None:
            duo.profile_next_launch(ev[0], ev[1])
        duo.duo_attn_decode(q, kp, vp, table, after[j], mask, w.sink, w.recent, w.ring_blocks,
                            w.scale, out, ws)

    for i in range(min(args.warmup, steps)):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / steps
    step_bytes = float(np.mean([decode_bytes(w, lens_seq[i % len(lens_seq)]) for i in range(steps)]))
    kern_all = sample_kernels(torch, step, steps, KERNEL_SAMPLES, args.flush)
    kern_s = float(np.mean(kern_all))
    # bytes of the sampled launches (the 1M context grows by one token per step)
    nbytes = float(np.mean([decode_bytes(w, lens_seq[(steps + i) % len(lens_seq)])
                            for i in range(KERNEL_SAMPLES)]))
    res = {"workload": w.name, "value": round(step_bytes / step_s / 1e9, 1), "unit": "GB/s",
           "us_per_step": round(step_s * 1e6, 2), "steps": steps, "layers_rotated": n_layers,
           "step": "kv_append_circular(1 token/seq) + duo_attn_decode",
           "algorithmic_bytes_per_launch": int(nbytes),
           "roofline": {"bound": "hbm", "achieved": round(nbytes / kern_s / 1e9, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(nbytes / kern_s / 1e9 / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(tag),
                        "kernel": f"duo::decode_kernel<{synth.DTYPE_NAMES[w.dtype]},{w.head_dim}>",
                        "kernel_us": round(kern_s * 1e6, 2), **spread_us(kern_all),
                        "cold": f"{FLUSH_BYTES >> 20} MiB read before each sampled launch"}}
    log(f"[{tag}] step {step_s * 1e6:.1f} us, kernel {kern_s * 1e6:.1f} us, "
        f"{nbytes / kern_s / 1e9:.0f} GB/s kernel ({nbytes / 1e6:.1f} MB per launch)")
    return res


def gemma_leg(args, torch, duo):
    """Gemma-2b static-cache decode: batch 16, MQA, D 256, fp16, valid lengths U[1024, 8192]."""
    w = synth.gemma_2b_static_decode()
    lens = synth.valid_lengths(w, 1024, 8192)
    return decode_shape_leg(args, torch, duo, w, [lens], 8, args.steps, "gemma")


def long_context_leg(args, torch, duo):
    """1M-token decode: batch 1, Llama-3-8B GQA shape; step k appends one token and attends over
    1,048,576 + k positions (k = 1..64)."""
    w = synth.long_context_decode()
    seq = [np.array([w.context + k]) for k in range(1, w.steps + 1)]
    return decode_shape_leg(args, torch, duo, w, seq, 2, w.steps, "1m")


def decode_quant_leg(args, torch, duo, dec, bits: int):
    """The decode workload over the int8 (bits = 8) or 4-bit (bits = 4) cache, on the bf16 leg's K/V
    bits (quantized by the library's own append; the 4-bit cache's per-channel scales are seeded
    stand-ins for calibrated ones)."""
    w = dec["w"]
    K, V = dec["K"], dec["V"]
    dev = torch.device("cuda:0")
    L = w.context
    tag = f"decode-int{bits}"
    log(f"[{tag}] filling the cache")
    table_h, nblocks = synth.block_table(w)
    table = torch.from_numpy(table_h).to(dev)
    mask = w.retrieval_mask
    if bits == 8:
        append, decode = duo.kv_append_circular_int8, duo.duo_attn_decode_int8
        ss = (nblocks, w.block_size)

        def new_pools():
            return (torch.empty((nblocks, w.block_size, w.head_dim), dtype=torch.int8, device=dev),
                    torch.empty((nblocks, w.head_dim, w.block_size), dtype=torch.int8, device=dev),
                    torch.empty(ss, dtype=torch.float32, device=dev),
                    torch.empty(ss, dtype=torch.float32, device=dev))
    else:
        append, decode = duo.kv_append_circular_int4, duo.duo_attn_decode_int4
        ks = torch.from_numpy(synth.channel_scales(w, synth.S_K)).to(dev)
        vs = torch.from_numpy(synth.channel_scales(w, synth.S_V)).to(dev)

        def new_pools():
            return (torch.empty((nblocks, w.block_size, w.head_dim // 2), dtype=torch.uint8, device=dev),
                    torch.empty((nblocks, w.head_dim, w.block_size // 2), dtype=torch.uint8, device=dev),
                    ks, vs)
    after = torch.empty(w.batch, dtype=torch.int32, device=dev)
    layers = []
    for li in range(args.layers):
        pools = new_pools()
        if li == 0:
            for s0 in range(0, L - 1, 8192):
                e = min(L - 1, s0 + 8192)
                kn = to_dev(torch, K[:, :, s0:e].transpose(0, 2, 1, 3), w.dtype, dev)
                vn = to_dev(torch, V[:, :, s0:e].transpose(0, 2, 1, 3), w.dtype, dev)
                lb = torch.full((w.batch,), s0, dtype=torch.int32, device=dev)
                append(*pools, table, kn, vn, lb, after, mask, w.sink, w.recent, w.ring_blocks)
        else:
            for dst, src in zip(pools[:2], layers[0][:2]):
                dst.copy_(src)
            if bits == 8:
                for dst, src in zip(pools[2:], layers[0][2:]):
                    dst.copy_(src)
        layers.append(pools)
    k_tok = to_dev(torch, K[:, :, L - 1:L].transpose(0, 2, 1, 3), w.dtype, dev)
    v_tok = to_dev(torch, V[:, :, L - 1:L].transpose(0, 2, 1, 3), w.dtype, dev)
    q = to_dev(torch, dec["q_bits"], w.dtype, dev)
    out = torch.empty_like(q)
    ws = duo.decode_workspace(q, table, w.block_size)
    lens_before = torch.full((w.batch,), L - 1, dtype=torch.int32, device=dev)
    lens = torch.empty_like(lens_before)
    torch.cuda.synchronize()

    def step(i, ev=None):
        pools = layers[i % len(layers)]
        append(*pools, table, k_tok, v_tok, lens_before, lens, mask, w.sink, w.recent,
               w.ring_blocks)
        if ev is not None:
            duo.profile_next_launch(ev[0], ev[1])
        decode(q, *pools, table, lens, mask, w.sink, w.recent, w.ring_blocks, w.scale, out, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    kern_all = sample_kernels(torch, step, args.warmup + args.steps, KERNEL_SAMPLES, args.flush)
    kern_s = float(np.mean(kern_all))
    nbytes = decode_bytes(w, np.full(w.batch, L), int8_cache=bits == 8, int4_cache=bits == 4)
    # the same step as one launch (duo_attn_append_decode_int8 / _int4), back to back
    fused_call = duo.duo_attn_append_decode_int8 if bits == 8 else duo.duo_attn_append_decode_int4
    lens_fused = torch.empty_like(lens_before)

    def fused_step(i):
        pools = layers[i % len(layers)]
        fused_call(q, k_tok, v_tok, *pools, table, lens_before, lens_fused, mask, w.sink, w.recent,
                   w.ring_blocks, w.scale, out, ws)

    for i in range(args.warmup):
        fused_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fused_step(args.warmup + i)
    torch.cuda.synchronize()
    fused_s = (time.perf_counter() - t0) / args.steps
    fused = {"call": f"duo_attn_append_decode_int{bits} (1 token/seq, one launch)",
             "us_per_step": round(fused_s * 1e6, 2), "GB/s": round(nbytes / fused_s / 1e9, 1)}
    res = {
        "workload": w.name + f"-int{bits}-kv", "value": round(nbytes / step_s / 1e9, 1),
        "unit": "GB/s", "ms_per_step": round(step_s * 1e3, 4),
        "step": f"kv_append_circular_int{bits}(1 token/seq) + duo_attn_decode_int{bits}",
        "algorithmic_bytes_per_step": nbytes,
        "step_speedup_vs_bf16": round(dec["ms_per_step"] / (step_s * 1e3), 3),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / kern_s / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / kern_s / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"decode_int{bits}"),
                     "kernel": f"duo::decode_int{bits}_kernel<bf16,128>",
                     "kernel_us": round(kern_s * 1e6, 2),
                     **spread_us(kern_all),
                     "cold": f"{FLUSH_BYTES >> 20} MiB read before each sampled launch",
                     "algorithmic_bytes_per_launch": nbytes},
    }
    res["fused_step"] = fused
    log(f"[{tag}] step {step_s * 1e6:.1f} us, kernel {kern_s * 1e6:.1f} us, "
        f"{res['value']:.0f} GB/s per step, {nbytes / kern_s / 1e9:.0f} GB/s kernel, "
        f"{res['step_speedup_vs_bf16']}x the bf16 step")
    return res


# ---- prefill leg -----------------------------------------------------------------------------
def prefill_leg(args, torch, duo):
    w = synth.llama2_7b_chunked_prefill()
    dev = torch.device("cuda:0")
    log(f"[prefill] generating {w.name}")
    L = w.context
    K = logical_bits(w, L, synth.S_K)
    V = logical_bits(w, L, synth.S_V)
    table_h, nblocks = synth.block_table(w)
    table = torch.from_numpy(table_h).to(dev)
    mask = w.retrieval_mask
    tdt = torch_dtype(torch, w.dtype)
    kp = torch.empty((nblocks, w.block_size, w.head_dim), dtype=tdt, device=dev)
    vp = torch.empty((nblocks, w.head_dim, w.block_size), dtype=tdt, device=dev)
    chunks = []
    for c in range(w.steps):
        s, e = c * w.q_len, (c + 1) * w.q_len
        kn = to_dev(torch, K[:, :, s:e].transpose(0, 2, 1, 3), w.dtype, dev)
        vn = to_dev(torch, V[:, :, s:e].transpose(0, 2, 1, 3), w.dtype, dev)
        q = to_dev(torch, synth.f32_to_storage(synth.queries(w, c), w.dtype), w.dtype, dev)
        lb = torch.full((w.batch,), s, dtype=torch.int32, device=dev)
        la = torch.full((w.batch,), e, dtype=torch.int32, device=dev)
        chunks.append((kn, vn, q, lb, la, torch.empty_like(q)))
    del K, V
    ws = duo.prefill_workspace(chunks[0][2], table, mask)
    torch.cuda.synchronize()

    def one_pass(evs=None):
        for c, (kn, vn, q, lb, la, out) in enumerate(chunks):
            duo.kv_append_circular(kp, vp, table, kn, vn, lb, la, mask, w.sink, w.recent,
                                   w.ring_blocks)
            if evs is not None:
                duo.profile_next_launch(evs[c][0], evs[c][1])
            duo.duo_attn_prefill(q, kp, vp, table, la, mask, w.sink, w.recent, w.ring_blocks,
                                 w.scale, out, ws)

    for _ in range(args.prefill_warmup):
        one_pass()
    torch.cuda.synchronize()
    all_evs = [[event_pair(torch)
                for _ in chunks] for _ in range(args.prefill_passes)]
    t0 = time.perf_counter()
    for p in range(args.prefill_passes):
        one_pass(all_evs[p])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pass_s = (t1 - t0) / args.prefill_passes
    per_chunk_flops = [prefill_flops(w, (c + 1) * w.q_len, w.q_len) for c in range(w.steps)]
    flops = sum(per_chunk_flops)
    kern = np.array([[a.elapsed_time(b) * 1e-3 for a, b in pe] for pe in all_evs]).mean(axis=0)
    kern_total = float(kern.sum())
    traffic = measured_traffic("prefill")
    res = {
        "workload": w.name, "value": round(flops / pass_s / 1e12, 2), "unit": "TFLOP/s",
        "ms_per_pass": round(pass_s * 1e3, 3), "flops_per_pass": flops,
        "chunk7_tflops": round(per_chunk_flops[-1] / kern[-1] / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(flops / kern_total / 1e12, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / kern_total / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": "duo::prefill_kernel<bf16,128>",
                     "kernel_us_per_chunk": [round(x * 1e6, 1) for x in kern]},
    }
    log(f"[prefill] pass {pass_s * 1e3:.3f} ms, kernels {kern_total * 1e3:.3f} ms, "
        f"{res['value']} TFLOP/s per pass, {res['roofline']['achieved']} TFLOP/s kernels")
    return res


def continuous_batching_leg(args, torch, duo):
    """A continuous-batching step (Llama-3-8B GQA shape, 32 sequences at 32768 tokens: one 4096-row
    prompt chunk and 31 single decode rows) as one duo_attn_prefill_varlen launch, against the same
    work as two calls (duo_attn_prefill on the chunk, duo_attn_decode on the 31 rows). The pools are
    filled on the device with N(0,1) values; parity at this shape is in the GPU tests."""
    w = synth.continuous_batching_step()
    rows_n = w.extra["rows"]
    dev = torch.device("cuda:0")
    B, L, n0 = w.batch, w.context, rows_n[0]
    log(f"[cb] {w.name}")
    table_h, nblocks = synth.block_table(w)
    table = torch.from_numpy(table_h).to(dev)
    mask = w.retrieval_mask
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    kp = torch.randn((nblocks, w.block_size, w.head_dim), generator=g, device=dev).to(torch.bfloat16)
    vp = torch.randn((nblocks, w.head_dim, w.block_size), generator=g, device=dev).to(torch.bfloat16)
    total_q = sum(rows_n)
    q = torch.randn((total_q, w.num_q_heads, w.head_dim), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    q_start = torch.from_numpy(np.concatenate([[0], np.cumsum(rows_n)]).astype(np.int32)).to(dev)
    ws_mix = duo.prefill_varlen_workspace(q, table, mask, n0, B, w.block_size)
    q_chunk = q[:n0].reshape(1, n0, w.num_q_heads, w.head_dim)
    out_chunk = torch.empty_like(q_chunk)
    ws_pre = duo.prefill_workspace(q_chunk, table[:1], mask)
    q_dec = q[n0:].contiguous()
    out_dec = torch.empty_like(q_dec)
    ws_dec = duo.decode_workspace(q_dec, table[1:], w.block_size)

    def mixed(ev=None):
        if ev is not None:
            duo.profile_next_launch(*ev)
        duo.duo_attn_prefill_varlen(q, kp, vp, table, lens, q_start, n0, mask, w.sink, w.recent,
                                    w.ring_blocks, w.scale, out, ws_mix)

    def separate(ev=None):
        if ev is not None:
            duo.profile_next_launch(*ev[0])
        duo.duo_attn_prefill(q_chunk, kp, vp, table[:1], lens[:1], mask, w.sink, w.recent,
                             w.ring_blocks, w.scale, out_chunk, ws_pre)
        if ev is not None:
            duo.profile_next_launch(*ev[1])
        duo.duo_attn_decode(q_dec, kp, vp, table[1:], lens[1:], mask, w.sink, w.recent,
                            w.ring_blocks, w.scale, out_dec, ws_dec)

    reps = max(4, args.prefill_passes * 2)
    for _ in range(2):
        mixed()
        separate()
    torch.cuda.synchronize()
    res_m, res_p, res_d, wall_m, wall_s = [], [], [], [], []
    for _ in range(reps):
        e = event_pair(torch)
        args.flush()
        t0 = time.perf_counter()
        mixed(e)
        torch.cuda.synchronize()
        wall_m.append(time.perf_counter() - t0)
        res_m.append(e[0].elapsed_time(e[1]) * 1e-3)
        e2 = (event_pair(torch), event_pair(torch))
        args.flush()
        t0 = time.perf_counter()
        separate(e2)
        torch.cuda.synchronize()
        wall_s.append(time.perf_counter() - t0)
        res_p.append(e2[0][0].elapsed_time(e2[0][1]) * 1e-3)
        res_d.append(e2[1][0].elapsed_time(e2[1][1]) * 1e-3)
    t_m = float(np.median(res_m))
    t_p, t_d = float(np.median(res_p)), float(np.median(res_d))
    w1 = synth.replace(w, batch=1)
    flops = prefill_flops(w1, L, n0)
    dbytes = decode_bytes(synth.replace(w, batch=B - 1), np.full(B - 1, L))
    ideal = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) + dbytes / (HBM_PEAK_GBS * 1e9)
    res = {"workload": w.name, "rows": f"1 x {n0} + {B - 1} x 1",
           "one_launch_us": round(t_m * 1e6, 1),
           "two_calls_us": {"prefill": round(t_p * 1e6, 1), "decode": round(t_d * 1e6, 1),
                            "sum": round((t_p + t_d) * 1e6, 1)},
           "one_launch_vs_two_calls": round((t_p + t_d) / t_m, 3),
           "wall_us": {"one_launch": round(float(np.median(wall_m)) * 1e6, 1),
                       "two_calls": round(float(np.median(wall_s)) * 1e6, 1)},
           "roofline": {"bound": "mfma+hbm", "chunk_flops": flops, "decode_bytes": dbytes,
                        "ideal_us": round(ideal * 1e6, 1),
                        "achieved": round(ideal / t_m, 4), "peak": 1.0,
                        "unit": "ideal time / kernel time",
                        "frac": round(ideal / t_m, 4), "traffic": measured_traffic("cb"),
                        "kernel": "duo::prefill_kernel<bf16,128,mixed>",
                        "note": "ideal = chunk FLOP at bf16 MFMA peak + decode-row bytes at HBM peak"},
           "kernel_samples": reps}
    log(f"[cb] one launch {t_m * 1e6:.1f} us; two calls {t_p * 1e6:.1f} + {t_d * 1e6:.1f} us; "
        f"ideal {ideal * 1e6:.1f} us")
    return res


def dca_flops(w: synth.Workload, L: int, q_len: int) -> int:
    """4 D FLOP per (query, key) pair; every head sees keys 0..p (Dual Chunk Attention changes which
    query vector meets a key, not how many keys)."""
    p = np.arange(L - q_len, L, dtype=np.int64)
    return int(4 * w.head_dim * w.num_q_heads * w.batch * (p + 1).sum())


def dca_leg(args, torch, duo):
    """Dual Chunk Attention prefill: the last 32768-row chunk of a 131072-token Qwen2-72B context
    (one GPU's share at tensor parallelism 4), timed with HIP events per launch."""
    w = synth.qwen2_72b_dca_prefill()
    dev = torch.device("cuda:0")
    C, L, n = w.extra["chunk_len"], w.context, w.q_len
    log(f"[dca] generating {w.name}")
    K = logical_bits(w, L, synth.S_K)
    V = logical_bits(w, L, synth.S_V)
    table_h, nblocks = synth.block_table(w)
    table = torch.from_numpy(table_h).to(dev)
    mask = w.retrieval_mask
    tdt = torch_dtype(torch, w.dtype)
    kp = torch.empty((nblocks, w.block_size, w.head_dim), dtype=tdt, device=dev)
    vp = torch.empty((nblocks, w.head_dim, w.block_size), dtype=tdt, device=dev)
    for s0 in range(0, L, n):
        kn = to_dev(torch, K[:, :, s0:s0 + n].transpose(0, 2, 1, 3), w.dtype, dev)
        vn = to_dev(torch, V[:, :, s0:s0 + n].transpose(0, 2, 1, 3), w.dtype, dev)
        lb = torch.full((w.batch,), s0, dtype=torch.int32, device=dev)
        la = torch.full((w.batch,), s0 + n, dtype=torch.int32, device=dev)
        duo.kv_append_circular(kp, vp, table, kn, vn, lb, la, mask, w.sink, w.recent,
                               w.ring_blocks)
    del K, V
    lens = torch.full((w.batch,), L, dtype=torch.int32, device=dev)
    qs = [to_dev(torch, synth.f32_to_storage(synth.queries(w, 3 * (w.steps - 1) + k), w.dtype),
                 w.dtype, dev) for k in range(3)]
    ms = torch.from_numpy(synth.row_scales(w, w.steps - 1, n)).to(dev)
    out = torch.empty_like(qs[0])
    ws = duo.dca_prefill_workspace(qs[0], table)
    torch.cuda.synchronize()
    # one call is ~28 ms of sustained MFMA work: an eighth of the prefill leg's passes (2 calls,
    # ~56 ms) is warm-up enough
    for _ in range(-(-args.prefill_warmup // 8)):
        duo.dca_attn_prefill(*qs, ms, C, kp, vp, table, lens, w.scale, out, ws)
    torch.cuda.synchronize()
    evs = [event_pair(torch)
           for _ in range(args.prefill_passes)]
    for a, b in evs:
        duo.profile_next_launch(a, b)
        duo.dca_attn_prefill(*qs, ms, C, kp, vp, table, lens, w.scale, out, ws)
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) * 1e-3 for a, b in evs]))
    flops = dca_flops(w, L, n)
    ach = flops / t / 1e12
    # the decode of the next token over the same cache (batch 1): every kv head's K/V is read once
    qd = [x[:, -1].contiguous() for x in qs]     # [batch][Hq][D]: the chunk's last row
    msd = ms[:, -1].contiguous()
    outd = torch.empty_like(qd[0])
    wsd = duo.decode_workspace(qd[0], table, w.block_size)
    for _ in range(10):
        duo.dca_attn_decode(*qd, msd, C, kp, vp, table, lens, w.scale, outd, wsd)
    torch.cuda.synchronize()
    devs = [event_pair(torch)
            for _ in range(50)]
    for a, b in devs:
        duo.profile_next_launch(a, b)
        duo.dca_attn_decode(*qd, msd, C, kp, vp, table, lens, w.scale, outd, wsd)
    torch.cuda.synchronize()
    td = float(np.median([a.elapsed_time(b) * 1e-3 for a, b in devs]))
    dbytes = (2 * w.num_kv_heads * L * w.head_dim * w.elem_bytes
              + 4 * w.num_kv_heads * (-(-L // w.block_size))
              + 4 * w.num_q_heads * w.head_dim * w.elem_bytes)    # K/V, tables, three q + out
    res = {"workload": w.name, "value": round(ach, 2), "unit": "TFLOP/s",
           "ms_per_call": round(t * 1e3, 3), "flops_per_call": flops, "chunk_len": C,
           "context": L, "q_len": n,
           "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": measured_traffic("dca"),
                        "kernel": "duo::prefill_kernel<bf16,128,dca>"},
           "decode": {"batch": w.batch, "us_per_call": round(td * 1e6, 2),
                      "algorithmic_bytes": dbytes, "GB/s": round(dbytes / td / 1e9, 1),
                      "frac_hbm": round(dbytes / td / 1e9 / HBM_PEAK_GBS, 4),
                      "kernel": "duo::decode_dca_kernel<bf16,128>",
                      "note": "batch 1 over 134 MB: too small to fill the chip; context only"}}
    log(f"[dca] prefill {t * 1e3:.3f} ms per call, {ach:.1f} TFLOP/s; decode {td * 1e6:.1f} us, "
        f"{dbytes / td / 1e9:.0f} GB/s")
    return res


# ---- CPU baseline: the oracle on a bounded sample ----------------------------------------------
def cpu_baseline(dec, budget_s: float):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    w, K, V, q_bits = dec["w"], dec["K"], dec["V"], dec["q_bits"]
    L = w.context
    done, spent, nbytes = 0, 0.0, 0
    per_seq = decode_bytes(synth.replace(w, batch=1), np.array([L]))
    # whole sequences of the workload, cycling through the batch until the time budget is spent
    while spent < budget_s or done == 0:
        b = done % w.batch
        t0 = time.perf_counter()
        oracle.attend(q_bits[b:b + 1, None], K[b:b + 1], V[b:b + 1], np.array([L]), w.retrieval_mask,
                      sink=w.sink, recent=w.recent, scale=w.scale, dtype=w.dtype)
        spent += time.perf_counter() - t0
        nbytes += per_seq
        done += 1
    return {"value": round(nbytes / spent / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} sequence-steps of the decode workload (batch {w.batch} cycled, all "
                      f"{w.num_q_heads} q heads, context {L}), {spent:.1f} s of fp64 NumPy"}


# ---- rocprofv3 counter bookkeeping -------------------------------------------------------------
COPY_KERNEL_HINT = "copy"   # the device-to-device copy (a runtime blit kernel) has "copy" in its name
CALIBRATION_REPS = 3


def calibrate_copy(torch, mib: int, reps: int = CALIBRATION_REPS):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE counters."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[calibrate] copied {mib} MiB x {reps}")


def _read_counter_csv(path):
    import csv
    rows = []
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            rows.append(r)
    return rows


def summarize_counters(fetch_csv: str, write_csv: str, copy_mib: int, out_path: str, command: str,
                       rename: dict | None = None):
    """Per-launch HBM bytes of the decode, prefill and Dual Chunk kernels from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), scaled by what the same counters read for a
    copy of copy_mib MiB in the same run. Merges the results into profiles/counters.json, keyed by
    leg, with the source hash. rename maps a kernel key to the leg it measured in this run (a run
    of the Gemma-2b leg alone: decode -> gemma), or to "-" to leave it out (a run of the
    continuous-batching leg alone also launches the plain prefill and decode kernels)."""
    def per_kernel(path, counter):
        acc, copies = {}, []
        for r in _read_counter_csv(path):
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            val = float(r["Counter_Value"]) * 1024.0          # counters are KiB per dispatch
            if "decode_int8_kernel" in name:
                acc.setdefault("decode_int8", []).append(val)
            elif "decode_int4_kernel" in name:
                acc.setdefault("decode_int4", []).append(val)
            elif "decode_kernel" in name:
                acc.setdefault("decode", []).append(val)
            elif "prefill_kernel" in name:
                # template arguments <T, D, DCA, MIX>: the Dual Chunk instantiation has DCA set, the
                # packed-batch launch with decode items (continuous batching) MIX
                if "Lb1ELb0E" in name or ", true, false>" in name:
                    acc.setdefault("dca", []).append(val)
                elif "Lb0ELb1E" in name or ", false, true>" in name:
                    acc.setdefault("cb", []).append(val)
                else:
                    acc.setdefault("prefill", []).append(val)
            elif COPY_KERNEL_HINT in name.lower():
                copies.append((int(r["Dispatch_Id"]), val))
        # the calibration copies are the last CALIBRATION_REPS copy dispatches of the run
        copies.sort()
        if copies:
            acc["copy"] = [v for _, v in copies[-CALIBRATION_REPS:]]
        return {k: float(np.mean(v)) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}
    fetch, nf = per_kernel(fetch_csv, "FETCH_SIZE")
    write, nw = per_kernel(write_csv, "WRITE_SIZE")
    known = float(copy_mib << 20)
    f_scale = known / fetch["copy"] if fetch.get("copy") else 1.0
    w_scale = known / write["copy"] if write.get("copy") else 1.0
    try:
        with open(out_path) as fh:
            out = json.load(fh)
    except (OSError, ValueError):
        out = {}
    out.pop("calibration", None)   # older layout: one calibration for the whole file
    calib = {"copy_bytes": known, "fetch_raw": fetch.get("copy"), "write_raw": write.get("copy"),
             "fetch_scale": f_scale, "write_scale": w_scale, "command": command}
    rename = rename or {}
    for k in ("decode", "decode_int8", "decode_int4", "prefill", "dca", "cb"):
        if k in fetch and k in write:
            leg = rename.get(k, k)
            if leg == "-":
                continue
            out[leg] = {"source_sha": source_sha(leg),
                        "fetch_bytes_per_launch": fetch[k] * f_scale,
                        "write_bytes_per_launch": write[k] * w_scale,
                        "hbm_bytes_per_launch": fetch[k] * f_scale + write[k] * w_scale,
                        "dispatches": [nf.get(k), nw.get(k)], "calibration": calib}
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=4, help="decode caches rotated across steps")
    ap.add_argument("--prefill-passes", type=int, default=5)
    # Untimed passes before the timed ones. Back to back, the prefill kernels speed up over their
    # first ~30 ms of sustained MFMA work (3.39 -> 2.78 ms per pass over the first ten passes, one
    # box) as the clocks settle; 16 passes (~50 ms) put the timed ones past that ramp.
    ap.add_argument("--prefill-warmup", type=int, default=16)
    ap.add_argument("--legs", default="decode,decode_int8,decode_int4,prefill,dca,gemma,1m,cb")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs into profiles/counters.json")
    ap.add_argument("--counters-command", default="", help="command recorded with the summary")
    ap.add_argument("--counters-as", default="", metavar="KERNEL=LEG,...",
                    help="record a kernel's counters under another leg (decode=gemma)")
    args = ap.parse_args()
    if args.summarize_counters:
        rename = dict(x.split("=", 1) for x in args.counters_as.split(",") if x)
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1],
                           args.calibrate_copy, COUNTERS, args.counters_command, rename)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU would run its "
              "own share of heads; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_sparsity_amd as duo
    duo.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    legs = set(args.legs.split(","))
    # No cyclic garbage collection while GPU work is timed: a collection pause on the host while
    # the GPU queue has drained would land between a launch's start and stop events.
    gc.collect()
    gc.disable()
    args.flush = Flusher(torch)
    dec = decode_leg(args, torch, duo) if legs & {"decode", "decode_int8", "decode_int4"} else None
    dq = decode_quant_leg(args, torch, duo, dec, 8) if "decode_int8" in legs else None
    d4 = decode_quant_leg(args, torch, duo, dec, 4) if "decode_int4" in legs else None
    pre = prefill_leg(args, torch, duo) if "prefill" in legs else None
    dca = dca_leg(args, torch, duo) if "dca" in legs else None
    gem = gemma_leg(args, torch, duo) if "gemma" in legs else None
    lng = long_context_leg(args, torch, duo) if "1m" in legs else None
    cbs = continuous_batching_leg(args, torch, duo) if "cb" in legs else None
    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy)
    gc.enable()
    cpu = None
    if dec is not None and not args.no_cpu_baseline:
        log("[cpu] timing the oracle")
        cpu = cpu_baseline(dec, args.cpu_budget)
    w = synth.llama3_8b_decode()
    line = {
        "metric": METRIC,
        "value": round(dec["value"], 1) if dec else None,
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 4) if dec else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) K/V/Q, random page placement)",
        "config": {"workload": w.name, "batch": w.batch, "context": w.context,
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "retrieval_kv_heads": list(w.retrieval), "sink": w.sink, "recent": w.recent,
                   "block_size": w.block_size, "layers_rotated": args.layers,
                   "step": "kv_append_circular(1 token/seq) + duo_attn_decode",
                   "algorithmic_bytes_per_step": dec["bytes"] if dec else None},
        "fused_step": dec["fused_step"] if dec else None,
        "roofline": dec["roofline"] if dec else None,
        "cpu_baseline": cpu,
        "prefill": pre,
        "decode_int8": dq,
        "decode_int4": d4,
        "dca_prefill": dca,
        "decode_gemma_2b_static": gem,
        "decode_1m_context": lng,
        "continuous_batching": cbs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
