"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

Workload (one step = the whole hot path over one batch): a Llama-8B-like
layer, 32 query / 8 KV heads, head_dim 128, 32768 cached tokens, batch 1.
Each step encodes all 32768 tokens' K (turbo4: 3-bit codebook + 1-bit QJL)
and V (4-bit codebook) and runs one decode-attention step (sparse V at
1e-6) over a packed cache.  Inputs are synthetic (seeded, see workloads.py)
and resident in HBM before the timed region.

The working set of one step (~170 MB) fits in the 256 MB Infinity Cache, so
the benchmark rotates over 8 copies of the inputs and packed caches (~1.4 GB),
and step i decodes the cache encoded at step i-4: every kernel reads data
that was last touched >600 MB of traffic earlier.

Prints one JSON line.  The oracle (float64 NumPy on the host cores) is timed
on a bounded slice of the same workload as `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn GB/s (% of HBM peak) over turbo KV; encode Mtokens/s"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak of the MI355X
N_COPIES = 8
LAG = 4
KERNEL_SOURCES = ["encode.hip", "attn.hip", "device_common.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-tokens", type=int, default=32768,
                    help="tokens of the workload the oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the tiny, min-max, 70B-like full-cache and batched needle measurements")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run plain 1 GiB device copies (counter calibration)")
    ap.add_argument("--only", choices=["tiny", "minmax", "decode_70b", "decode_needle", "decode_loop", "prefill",
                                       "quality"],
                    help="run only this extra measurement and print its JSON (for profiling)")
    return ap.parse_args()


def copy_calibration():
    """Plain device-to-device copies of a known size: under rocprofv3 --pmc
    their FETCH_SIZE / WRITE_SIZE per dispatch calibrate the counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "kv_cache_quantization_encode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_profile(kernel: str, section: str = "kernels"):
    """Per-launch figures from committed rocprofv3 --pmc summaries (HBM bytes
    under "kernels", MFMA utilisation under "mfma"), if they were taken on the
    current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic_llama8b.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    return t.get(section, {}).get(kernel)


def cpu_baseline(tokens: int):
    """Time the oracle on `tokens` positions of the same workload (all heads)."""
    from threadpoolctl import threadpool_info

    from kv_cache_quantization_encode_amd import workloads as W
    from oracle import turbokv_oracle as O

    case = W.llama8b(T=tokens)
    tab = O.Tables(128, seed=42)
    B, Hq, Hkv, T = case.shape
    k = case.k.reshape(-1, 128)
    v = case.v.reshape(-1, 128)
    t0 = time.perf_counter()
    ek = O.encode(k, 3, True, tab)
    ev = O.encode(v, 4, False, tab)
    kp = O.pack_tq(ek, "prod", 3, 128)
    vp = O.pack_tq(ev, "mse", 4, 128)
    t1 = time.perf_counter()
    n = k.shape[0]
    kh = O.dequant_packed(kp, "prod", 3, tab, n).reshape(B, Hkv, T, 128)
    vh = O.dequant_packed(vp, "mse", 4, tab, n).reshape(B, Hkv, T, 128)
    out, p = O.attention_decode(case.q.astype(np.float64), kh, vh, 1e-6)
    t2 = time.perf_counter()
    g = Hq // Hkv
    keep_rows = int(np.sum(np.any((p >= 1e-6).reshape(B, Hkv, g, T), axis=2)))
    attn_bytes = n * 68 + keep_rows * 64 + n * 2 + B * Hq * 128 * 6
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": attn_bytes / (t2 - t1) / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{tokens} of 32768 tokens, all 8 KV / 32 query heads: oracle encode+pack "
                  f"({t1 - t0:.1f} s, {tokens / (t1 - t0) / 1e6:.5f} Mtokens/s) then dense "
                  f"dequant + fp64 attention ({t2 - t1:.1f} s); value = decode-attn GB/s",
        "encode_mtok_s": tokens / (t1 - t0) / 1e6,
        "host_cpus": os.cpu_count(),
    }


def kept_v_rows(TK, ctx, q, kbuf, kf, B, Hq, Hkv, T, tau, dev):
    """Number of V rows the exact sparse-V rule keeps (some query head of the
    group has weight >= tau), from the library's own dequantisation of the
    packed K and a float32 softmax on the GPU.  Byte accounting only; it runs
    outside every timed region."""
    import torch
    n_vec = B * Hkv * T
    khat = torch.empty((n_vec, 128), dtype=torch.float16, device=dev)
    TK.tq_decode_kv(ctx, kbuf, kf, n_vec, khat)
    g = Hq // Hkv
    kh = khat.view(B * Hkv, T, 128).float()
    qq = q.view(B * Hkv, g, 128).float().transpose(1, 2).contiguous()
    scores = torch.bmm(kh, qq) / math.sqrt(128)  # [B*Hkv, T, g]
    p = torch.softmax(scores, dim=1)
    kept = int((p >= tau).any(dim=2).sum().item())
    del khat, kh, scores, p
    return kept


def v_bytes_read(TK, vf, n_vec, kept):
    """V bytes the decode reads: index rows of kept tokens only, plus every
    fp16 norm (codebook V: the norm scales each candidate's weight) or the
    block scales of kept rows (q8 V)."""
    if vf.kind == TK.KIND_Q8:
        return kept * (128 + 8)
    return kept * 16 * vf.bits + n_vec * 2


def outlier_normal_gpu(gen, shape, n_out, dev, scale=20.0):
    """N(0,1) fp16 tensor [..., T, 128] with n_out channels per leading index
    scaled by `scale` (the tiny/70B-like recipe), drawn on the GPU."""
    import torch
    x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    lead = x.view(-1, shape[-2], shape[-1])
    for i in range(lead.shape[0]):
        ch = torch.randperm(shape[-1], generator=gen, device=dev)[:n_out]
        lead[i][:, ch] *= scale
    return x.half()


def graph_time(fn, reps, warm, stream):
    """Mean time of one replay of a HIP graph that holds fn(), by HIP events
    on the replay stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager run before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    cur = torch.cuda.current_stream()
    for a, b in ev:
        a.record(cur)
        g.replay()
        b.record(cur)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3


def bench_70b(TK, ctx, dev, reps=10, warm=3):
    """70B-like full cache on one GPU: 80 layers x 8 KV heads x 131072 tokens,
    64 query heads; turbo3 K (2-bit codebook + QJL) + 2-bit V, layers 0, 1,
    78, 79 at q8 for K and V.  K/V of each layer are N(0,1) with 4 channels
    x20 (seed 404 + layer, drawn on the GPU), encoded once; one decode step =
    the 80 per-layer attention calls, replayed as one HIP graph."""
    import torch
    L, Hkv, Hq, T, B = 80, 8, 64, 131072, 1
    n_vec = B * Hkv * T
    tau = 1e-6
    boundary = (0, 1, 78, 79)
    layers = []
    moved = logical = 0
    for l in range(L):
        gen = torch.Generator(device=dev)
        gen.manual_seed(404 + l)
        if l in boundary:
            kf, vf = TK.Q8, TK.Q8
        else:
            kf, vf = TK.turbo_k(3), TK.mse(2)
        k = outlier_normal_gpu(gen, (Hkv, T, 128), 4, dev).view(-1, 128)
        v = outlier_normal_gpu(gen, (Hkv, T, 128), 4, dev).view(-1, 128)
        q = torch.randn((B, Hq, 128), generator=gen, device=dev).half()
        kp, vp = TK.alloc_packed(kf, n_vec), TK.alloc_packed(vf, n_vec)
        TK.tq_encode_kv(ctx, k, v, n_vec, kf, vf, kp.buf, vp.buf)
        del k, v
        kept = kept_v_rows(TK, ctx, q, kp.buf, kf, B, Hq, Hkv, T, tau, dev)
        kb = int(kp.layout.total_bytes)
        moved += kb + v_bytes_read(TK, vf, n_vec, kept) + B * Hq * 128 * (2 + 4)
        logical += kb + int(vp.layout.total_bytes) + B * Hq * 128 * (2 + 4)
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
        layers.append((q, kp, vp, kf, vf, out))
    ws, wsb = TK.alloc_workspace(B, Hq, Hkv, T, TK.turbo_k(3), TK.mse(2))

    def step():
        for q, kp, vp, kf, vf, out in layers:
            TK.tq_attn_decode(ctx, q, kp.buf, vp.buf, kf, vf, B, Hq, Hkv, T, None, tau, out, ws, wsb)

    t = graph_time(step, reps, warm, None)
    res = {"workload": "70B-like decode step: 80 layers x 8 KV / 64 q heads x 131072 tokens, batch 1; "
                       "turbo3 K + 2-bit V, layers 0,1,78,79 q8; one HIP graph of 80 calls",
           "step_ms": round(t * 1e3, 4), "moved_gb": round(moved / 1e9, 4), "logical_gb": round(logical / 1e9, 4),
           "moved_gbs": round(moved / t / 1e9, 1), "frac_hbm": round(moved / t / 1e9 / HBM_PEAK_GBS, 4),
           "logical_gbs": round(logical / t / 1e9, 1)}
    del layers, ws
    torch.cuda.empty_cache()
    return res


def bench_needle(TK, ctx, dev, reps=20, warm=5):
    """Batched needle decode: 64 sequences x 8192 tokens, 32 q / 8 KV heads;
    K N(0,1) with 8 channels x20 per KV head, V N(0,1); each query head points
    at one of 16 needle keys of its sequence (outlier channels removed, norm
    3 sqrt(128)), so each head's softmax is dominated by one token.  turbo4 K
    + 2-bit V, tau 1e-6.  Drawn on the GPU (seed 505)."""
    import torch
    B, T, Hq, Hkv = 64, 8192, 32, 8
    n_vec = B * Hkv * T
    tau = 1e-6
    gen = torch.Generator(device=dev)
    gen.manual_seed(505)
    k = torch.randn((B, Hkv, T, 128), generator=gen, device=dev)
    out_ch = torch.stack([torch.randperm(128, generator=gen, device=dev)[:8] for _ in range(Hkv)])
    for h in range(Hkv):
        k[:, h, :, out_ch[h]] *= 20.0
    k = k.half()
    v = torch.randn((B, Hkv, T, 128), generator=gen, device=dev).half()
    needles = torch.stack([torch.sort(torch.randperm(T, generator=gen, device=dev)[:16])[0] for _ in range(B)])
    g = Hq // Hkv
    q = torch.zeros((B, Hq, 128), device=dev)
    for h in range(Hq):
        kvh = h // g
        kn = k[torch.arange(B, device=dev), kvh, needles[:, h % 16]].float()  # [B, 128]
        kn[:, out_ch[kvh]] = 0.0
        q[:, h] = 3.0 * math.sqrt(128) * kn / kn.norm(dim=1, keepdim=True)
    q = q.half()
    kf, vf = TK.turbo_k(4), TK.mse(2)
    kp, vp = TK.alloc_packed(kf, n_vec), TK.alloc_packed(vf, n_vec)
    TK.tq_encode_kv(ctx, k.view(-1, 128), v.view(-1, 128), n_vec, kf, vf, kp.buf, vp.buf)
    del k, v
    kept = kept_v_rows(TK, ctx, q, kp.buf, kf, B, Hq, Hkv, T, tau, dev)
    ws, wsb = TK.alloc_workspace(B, Hq, Hkv, T, kf, vf)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)

    def call():
        TK.tq_attn_decode(ctx, q, kp.buf, vp.buf, kf, vf, B, Hq, Hkv, T, None, tau, out, ws, wsb)

    t = graph_time(call, reps, warm, None)
    kb = int(kp.layout.total_bytes)
    moved = kb + v_bytes_read(TK, vf, n_vec, kept) + B * Hq * 128 * 6
    logical = kb + int(vp.layout.total_bytes) + B * Hq * 128 * 6
    res = {"workload": "batched needle decode: 64 x 8192 tokens, 32 q / 8 KV heads; turbo4 K + 2-bit V, tau 1e-6",
           "us": round(t * 1e6, 2), "v_rows_kept": kept, "moved_gbs": round(moved / t / 1e9, 1),
           "frac_hbm": round(moved / t / 1e9 / HBM_PEAK_GBS, 4), "logical_gbs": round(logical / t / 1e9, 1)}
    del kp, vp, ws, out
    torch.cuda.empty_cache()
    return res


def bench_tiny(TK, ctx, dev, reps=50, warm=10):
    """Tiny case: 1 KV head x 1024 tokens, K/V N(0,1) with 4 channels x20,
    turbo3 K (2-bit codebook + QJL) + 2-bit V; latency of one encode of all
    tokens and of one decode-attention step (each a HIP graph replay)."""
    import torch
    T = 1024
    gen = torch.Generator(device=dev)
    gen.manual_seed(101)
    k = outlier_normal_gpu(gen, (T, 128), 4, dev)
    v = outlier_normal_gpu(gen, (T, 128), 4, dev)
    q = torch.randn((1, 1, 128), generator=gen, device=dev).half()
    kf, vf = TK.turbo_k(3), TK.mse(2)
    kp, vp = TK.alloc_packed(kf, T), TK.alloc_packed(vf, T)
    ws, wsb = TK.alloc_workspace(1, 1, 1, T, kf, vf)
    out = torch.empty((1, 1, 128), dtype=torch.float32, device=dev)
    t_enc = graph_time(lambda: TK.tq_encode_kv(ctx, k, v, T, kf, vf, kp.buf, vp.buf), reps, warm, None)
    t_att = graph_time(lambda: TK.tq_attn_decode(ctx, q, kp.buf, vp.buf, kf, vf, 1, 1, 1, T, None, 1e-6, out, ws,
                                                 wsb), reps, warm, None)
    return {"workload": "tiny: 1 KV head x 1024 tokens; turbo3 K + 2-bit V", "encode_us": round(t_enc * 1e6, 2),
            "decode_attn_us": round(t_att * 1e6, 2)}


def bench_decode_loop(TK, ctx, dev, reps=10, warm=3):
    """Decode loop on the llama8b-like layer (32 q / 8 KV heads, 32768-token
    cache capacity, turbo4 K + 4-bit V, tau 1e-6): one step appends the new
    token's K and V for the 8 KV heads at position 32767 (tq_append_kv) and
    then attends over all 32768 tokens.  Eight caches are rotated so that the
    packed bytes do not stay in the 256 MB MALL; one HIP graph holds eight
    steps.  K = lognormal(0, 0.5) per (head, channel) x Student-t(3), V and q
    N(0, 1), drawn on the GPU from a seeded generator."""
    import torch
    B, Hq, Hkv, T, copies = 1, 32, 8, 32768, 8
    n_vec = B * Hkv * T
    kf, vf, tau = TK.turbo_k(4), TK.mse(4), 1e-6
    gen = torch.Generator(device=dev)
    gen.manual_seed(606)

    def student_k(shape):
        z = torch.randn(shape, generator=gen, device=dev)
        chi = torch.randn((3,) + tuple(shape), generator=gen, device=dev).pow(2).sum(0)
        return z / torch.sqrt(chi / 3.0)

    scale = torch.exp(0.5 * torch.randn((Hkv, 1, 128), generator=gen, device=dev))
    kps, vps = [], []
    for _ in range(copies):
        k = (student_k((Hkv, T, 128)) * scale).half().reshape(-1, 128)
        v = torch.randn((n_vec, 128), generator=gen, device=dev).half()
        kp, vp = TK.alloc_packed(kf, n_vec), TK.alloc_packed(vf, n_vec)
        TK.tq_encode_kv(ctx, k, v, n_vec, kf, vf, kp.buf, vp.buf)
        kps.append(kp)
        vps.append(vp)
        del k, v
    k_new = (student_k((Hkv, 128)) * scale[:, 0]).half().reshape(B, Hkv, 128)
    v_new = torch.randn((B, Hkv, 128), generator=gen, device=dev).half()
    q = torch.randn((B, Hq, 128), generator=gen, device=dev).half()
    pos = torch.full((B,), T - 1, dtype=torch.int32, device=dev)
    lens = pos + 1
    ws, wsb = TK.alloc_workspace(B, Hq, Hkv, T, kf, vf)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def appends():
        for c in range(copies):
            TK.tq_append_kv(ctx, k_new, v_new, B, Hkv, T, pos, kf, vf, kps[c].buf, vps[c].buf)

    def steps():
        for c in range(copies):
            TK.tq_append_kv(ctx, k_new, v_new, B, Hkv, T, pos, kf, vf, kps[c].buf, vps[c].buf)
            TK.tq_attn_decode(ctx, q, kps[c].buf, vps[c].buf, kf, vf, B, Hq, Hkv, T, lens, tau, out, ws, wsb)

    t_app = graph_time(appends, reps, warm, None) / copies
    t_step = graph_time(steps, reps, warm, None) / copies
    return {"workload": "decode loop, llama8b-like layer: append 1 token (K+V, 8 KV heads) then attend over "
                        "32768 tokens; turbo4 K + 4-bit V, tau 1e-6",
            "append_us": round(t_app * 1e6, 2), "step_us": round(t_step * 1e6, 2)}


def bench_prefill(TK, ctx, dev, reps=10, warm=3, Tq=16):
    """Causal prefill attention on the llama8b-like layer (32 q / 8 KV heads,
    32768 tokens, turbo4 K + 4-bit V, tau 1e-6): the last Tq positions attend
    to their prefixes (tq_attn_prefill).  Eight rotating caches, one HIP graph
    of eight calls; inputs drawn on the GPU from a seeded generator (K
    lognormal(0, 0.5) per (head, channel) x Student-t(3), V and q N(0, 1))."""
    import torch
    B, Hq, Hkv, T, copies = 1, 32, 8, 32768, 8
    n_vec = B * Hkv * T
    kf, vf, tau = TK.turbo_k(4), TK.mse(4), 1e-6
    gen = torch.Generator(device=dev)
    gen.manual_seed(707)
    scale = torch.exp(0.5 * torch.randn((Hkv, 1, 128), generator=gen, device=dev))
    kps, vps = [], []
    for _ in range(copies):
        z = torch.randn((Hkv, T, 128), generator=gen, device=dev)
        chi = torch.randn((3, Hkv, T, 128), generator=gen, device=dev).pow(2).sum(0)
        k = (z / torch.sqrt(chi / 3.0) * scale).half().reshape(-1, 128)
        v = torch.randn((n_vec, 128), generator=gen, device=dev).half()
        kp, vp = TK.alloc_packed(kf, n_vec), TK.alloc_packed(vf, n_vec)
        TK.tq_encode_kv(ctx, k, v, n_vec, kf, vf, kp.buf, vp.buf)
        kps.append(kp)
        vps.append(vp)
        del k, v, z, chi
    q = torch.randn((B, Tq, Hq, 128), generator=gen, device=dev).half()
    wsb = TK.tq_attn_prefill_workspace_bytes(B, Hq, Hkv, T, Tq, kf, vf)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Tq, Hq, 128), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def calls():
        for c in range(copies):
            TK.tq_attn_prefill(ctx, q, kps[c].buf, vps[c].buf, kf, vf, B, Hq, Hkv, T, Tq, None, tau, out, ws, wsb)

    t = graph_time(calls, reps, warm, None) / copies
    k_bytes = n_vec * 68
    return {"workload": f"causal prefill attention, llama8b-like layer: last {Tq} of 32768 positions as queries, "
                        "32 q / 8 KV heads; turbo4 K + 4-bit V, tau 1e-6",
            "us": round(t * 1e6, 2), "queries_per_s": round(Tq / t, 1),
            "k_read_gbs_per_query": round(k_bytes * Tq / t / 1e9, 1)}


def bench_minmax(TK, dev, reps=10, warm=3):
    """Per-group asymmetric min-max baseline: K and V tensors of 32 layers x
    8 KV heads x 4096 tokens x 128 (2 x 134M fp16 elements), N(0,1) times a
    per-64-group scale log-uniform in [1e-3, 8] (drawn on the GPU, seed 303);
    group 64 at 2/3/4 bits.  Quantise and dequantise GB/s (bytes read +
    written), MSE and cosine (flattened and mean per 128-vector)."""
    import torch
    n = 32 * 8 * 4096 * 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(303)
    res = {"workload": "min-max: 2 x 32 layers x 8 KV heads x 4096 tokens x 128, group 64"}
    xs = []
    for _ in range(2):
        x = torch.randn((n // 64, 64), generator=gen, device=dev)
        sc = torch.exp(torch.empty((n // 64, 1), device=dev).uniform_(math.log(1e-3), math.log(8.0), generator=gen))
        xs.append((x * sc).half().view(-1))
        del x, sc
    for bits in (2, 3, 4):
        codes = [torch.empty(n * bits // 8, dtype=torch.uint8, device=dev) for _ in xs]
        scale = [torch.empty(n // 64, dtype=torch.float16, device=dev) for _ in xs]
        zero = [torch.empty(n // 64, dtype=torch.float16, device=dev) for _ in xs]
        outs = [torch.empty(n, dtype=torch.float16, device=dev) for _ in xs]

        def quant():
            for i, x in enumerate(xs):
                TK.tq_minmax_quant(x, n, 64, bits, codes[i], scale[i], zero[i])

        def dequant():
            for i in range(len(xs)):
                TK.tq_minmax_dequant(codes[i], scale[i], zero[i], n, 64, bits, outs[i])

        tq_ = graph_time(quant, reps, warm, None)
        td_ = graph_time(dequant, reps, warm, None)
        per_elem = 2 + bits / 8 + 4 / 64
        mse = cos = cosv = 0.0
        for i, x in enumerate(xs):
            xf, yf = x.float(), outs[i].float()
            mse += float(((xf - yf) ** 2).mean()) / len(xs)
            cos += float(torch.dot(xf, yf) / (xf.norm() * yf.norm())) / len(xs)
            xv, yv = xf.view(-1, 128), yf.view(-1, 128)
            cosv += float((torch.sum(xv * yv, 1) / (xv.norm(dim=1) * yv.norm(dim=1)).clamp_min(1e-30)).mean()) / len(xs)
            del xf, yf, xv, yv
        res[f"b{bits}"] = {"quant_gbs": round(2 * n * per_elem / tq_ / 1e9, 1),
                           "dequant_gbs": round(2 * n * per_elem / td_ / 1e9, 1),
                           "quant_gelem_s": round(2 * n / tq_ / 1e9, 2), "mse": mse, "cosine": round(cos, 5),
                           "cosine_per_vector": round(cosv, 5)}
        del codes, scale, zero, outs
    del xs
    torch.cuda.empty_cache()
    return res


def bench_quality(TK, ctx, dev):
    """Reconstruction quality of the codecs (tq_encode_kv then tq_decode_kv)
    next to the min-max baseline at similar bits, on two inputs drawn on the
    GPU: (a) one tensor of the min-max workload (32 layers x 8 KV heads x 4096
    tokens x 128, N(0,1) times a per-64-group scale log-uniform in [1e-3, 8],
    seed 303) and (b) llama8b-like K (8 KV heads x 32768 tokens x 128,
    lognormal(0, 0.5) per (head, channel) x Student-t(3), seed 808), whose
    outlier channels the rotation spreads out.  Bits per element include the
    stored norms / scales; ratio = 16 / bits."""
    import torch
    res = {"workload": "reconstruction quality: turboN K (QJL), b-bit V, q8 and min-max (group 64) on the "
                       "min-max workload's K tensor and on llama8b-like K"}
    gen = torch.Generator(device=dev)
    gen.manual_seed(303)
    n_a = 32 * 8 * 4096 * 128
    x = torch.randn((n_a // 64, 64), generator=gen, device=dev)
    sc = torch.exp(torch.empty((n_a // 64, 1), device=dev).uniform_(math.log(1e-3), math.log(8.0), generator=gen))
    data_a = (x * sc).half().view(-1, 128)
    del x, sc
    gen.manual_seed(808)
    z = torch.randn((8, 32768, 128), generator=gen, device=dev)
    chi = torch.randn((3, 8, 32768, 128), generator=gen, device=dev).pow(2).sum(0)
    scale = torch.exp(0.5 * torch.randn((8, 1, 128), generator=gen, device=dev))
    data_b = (z / torch.sqrt(chi / 3.0) * scale).half().view(-1, 128)
    del z, chi

    def stats(xh, yh):
        xf, yf = xh.float(), yh.float()
        cos = float(torch.dot(xf.view(-1), yf.view(-1)) / (xf.norm() * yf.norm()))
        cv = float((torch.sum(xf * yf, 1) / (xf.norm(dim=1) * yf.norm(dim=1)).clamp_min(1e-30)).mean())
        return {"mse": float(((xf - yf) ** 2).mean()), "cosine": round(cos, 5), "cosine_per_vector": round(cv, 5)}

    fmts = [("turbo2_k", TK.turbo_k(2), 2.25), ("turbo3_k", TK.turbo_k(3), 3.25), ("turbo4_k", TK.turbo_k(4), 4.25),
            ("v2", TK.mse(2), 2.125), ("v3", TK.mse(3), 3.125), ("v4", TK.mse(4), 4.125), ("q8", TK.Q8, 8.5)]
    for name, data in (("minmax_data", data_a), ("llama8b_k", data_b)):
        n_vec = data.shape[0]
        out = {}
        y = torch.empty_like(data)
        for fname, f, bpe in fmts:
            pk = TK.alloc_packed(f, n_vec)
            TK.tq_encode_kv(ctx, data, None, n_vec, f, f, pk.buf, None)
            TK.tq_decode_kv(ctx, pk.buf, f, n_vec, y)
            torch.cuda.synchronize()
            out[fname] = {"bits_per_elem": bpe, "ratio": round(16 / bpe, 2), **stats(data, y)}
            del pk
        n = data.numel()
        for bits in (2, 3, 4):
            codes = torch.empty(n * bits // 8, dtype=torch.uint8, device=dev)
            sz = torch.empty(n // 64, dtype=torch.float16, device=dev)
            zz = torch.empty(n // 64, dtype=torch.float16, device=dev)
            TK.tq_minmax_quant(data.view(-1), n, 64, bits, codes, sz, zz)
            TK.tq_minmax_dequant(codes, sz, zz, n, 64, bits, y.view(-1))
            torch.cuda.synchronize()
            bpe = bits + 0.5
            out[f"minmax_b{bits}"] = {"bits_per_elem": bpe, "ratio": round(16 / bpe, 2), **stats(data, y)}
            del codes, sz, zz
        res[name] = out
        del y
    del data_a, data_b
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.copy_calib:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU sharding of the "
                                   "KV-cache path is described in the design notes but not built"}))
        sys.exit(2)
    import torch

    from kv_cache_quantization_encode_amd import turbokv as TK
    from kv_cache_quantization_encode_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    TK.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.only:
        if args.only == "minmax":
            r = bench_minmax(TK, dev)
        elif args.only == "quality":
            r = bench_quality(TK, TK.tq_codebook_init(128, 128, 42), dev)
        else:
            ctx1 = TK.tq_codebook_init(128, 128, 42)
            fn = {"tiny": bench_tiny, "decode_70b": bench_70b, "decode_needle": bench_needle,
                  "decode_loop": bench_decode_loop, "prefill": bench_prefill}[args.only]
            r = fn(TK, ctx1, dev, reps=5, warm=2)
        print(json.dumps({args.only: r}), flush=True)
        return

    case = W.llama8b()
    B, Hq, Hkv, T = case.shape
    n_vec = B * Hkv * T
    kf, vf, tau = TK.turbo_k(4), TK.mse(4), 1e-6

    k0 = torch.from_numpy(case.k.reshape(-1, 128)).to(dev)
    v0 = torch.from_numpy(case.v.reshape(-1, 128)).to(dev)
    q = torch.from_numpy(case.q).to(dev)
    ks = [k0] + [k0.clone() for _ in range(N_COPIES - 1)]
    vs = [v0] + [v0.clone() for _ in range(N_COPIES - 1)]
    kps = [TK.alloc_packed(kf, n_vec) for _ in range(N_COPIES)]
    vps = [TK.alloc_packed(vf, n_vec) for _ in range(N_COPIES)]
    ws, wsb = TK.alloc_workspace(B, Hq, Hkv, T, kf, vf)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    ctx = TK.tq_codebook_init(128, 128, 42)

    def step(i, ev=None):
        s = i % N_COPIES
        d = (i - LAG) % N_COPIES
        if ev is not None:
            ev[0].record(stream)
        TK.tq_encode_kv(ctx, ks[s], None, n_vec, kf, vf, kps[s].buf, None)
        if ev is not None:
            ev[1].record(stream)
        TK.tq_encode_kv(ctx, None, vs[s], n_vec, kf, vf, None, vps[s].buf)
        if ev is not None:
            ev[2].record(stream)
        TK.tq_attn_decode(ctx, q, kps[d].buf, vps[d].buf, kf, vf, B, Hq, Hkv, T, None, tau, out, ws, wsb)
        if ev is not None:
            ev[3].record(stream)

    for i in range(N_COPIES):  # every packed cache holds a valid encoding
        step(i)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    enc_k = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    enc_v = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    attn = np.array([e[2].elapsed_time(e[3]) for e in evs]) * 1e-3

    # sparse-V bookkeeping (byte accounting only, outside the timed region):
    # which V rows does the exact rule keep?  Scores from the library's own
    # dequantisation of the packed K, softmax in float64.
    d = (args.warmup + args.steps - 1 - LAG) % N_COPIES
    khat = torch.empty((n_vec, 128), dtype=torch.float16, device=dev)
    TK.tq_decode_kv(ctx, kps[d].buf, kf, n_vec, khat)
    kh = khat.view(B, Hkv, 1, T, 128).double()
    qq = q.view(B, Hkv, Hq // Hkv, 128, 1).double()
    scores = torch.matmul(kh, qq).squeeze(-1) / math.sqrt(128)  # [B, Hkv, g, T]
    p = torch.softmax(scores, dim=-1)
    keep = (p >= tau).any(dim=2)
    kept_rows = int(keep.sum().item())
    del khat, kh

    k_bytes = n_vec * 68
    v_row = 64
    attn_alg = k_bytes + kept_rows * v_row + n_vec * 2 + B * Hq * 128 * (2 + 4)
    attn_logical = k_bytes + n_vec * 66 + B * Hq * 128 * (2 + 4)
    enc_k_bytes = n_vec * (256 + 68)
    enc_v_bytes = n_vec * (256 + 66)
    t_attn, t_k, t_v = float(np.mean(attn)), float(np.mean(enc_k)), float(np.mean(enc_v))
    attn_gbs = attn_alg / t_attn / 1e9
    enc_mtok = T / (t_k + t_v) / 1e6

    kernels = {
        "encode_tq_kernel<3,true>": (t_k, enc_k_bytes),
        "encode_tq_kernel<4,false>": (t_v, enc_v_bytes),
        "attention (scores+values)": (t_attn, attn_alg),
    }
    dom = max(kernels, key=lambda n: kernels[n][0])

    def roof(name):
        t, by = kernels[name]
        ach = by / t / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": load_profile(name), "kernel": name,
             "avg_us": round(t * 1e6, 2), "alg_bytes_per_launch": by}
        mf = load_profile(name, "mfma")
        if mf and mf.get("flops_per_launch"):
            # matrix-core side of the same kernel: busy share from the counters,
            # fp16 MFMA rate from the counted flops and the live duration
            r["mfma"] = {"util": round(mf["util_pct"] / 100.0, 3),
                         "achieved_tflops": round(mf["flops_per_launch"] / t / 1e12, 1),
                         "peak_tflops": MFMA_F16_PEAK_TFLOPS}
        return r

    res = {
        "metric": METRIC,
        "value": round(attn_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "llama8b-like layer: 32 q / 8 kv heads, head_dim 128, 32768 tokens, batch 1; "
                               "turbo4 K (3-bit codebook + QJL) + 4-bit V, sparse V tau 1e-6",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "decode_attn_us": round(t_attn * 1e6, 2),
        "decode_attn_frac_hbm": round(attn_gbs / HBM_PEAK_GBS, 4),
        "decode_attn_logical_gbs": round(attn_logical / t_attn / 1e9, 1),
        "v_rows_read_frac": round(kept_rows / n_vec, 4),
        "encode_mtok_s": round(enc_mtok, 2),
        "encode_gbs": round((enc_k_bytes + enc_v_bytes) / (t_k + t_v) / 1e9, 1),
        "encode_frac_hbm": round((enc_k_bytes + enc_v_bytes) / (t_k + t_v) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roof(dom),
        "roofline_attn": roof("attention (scores+values)"),
        "roofline_encode_k": roof("encode_tq_kernel<3,true>"),
        "source_hash": source_hash(),
    }
    del kps, vps, ks, vs, ws
    torch.cuda.empty_cache()
    if not args.no_extra:
        res["tiny"] = bench_tiny(TK, ctx, dev)
        res["minmax"] = bench_minmax(TK, dev)
        res["decode_70b"] = bench_70b(TK, ctx, dev)
        res["decode_needle"] = bench_needle(TK, ctx, dev)
        res["decode_loop"] = bench_decode_loop(TK, ctx, dev)
        res["prefill"] = bench_prefill(TK, ctx, dev)
        res["quality"] = bench_quality(TK, ctx, dev)
    TK.tq_ctx_destroy(ctx)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
