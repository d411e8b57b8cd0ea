#!/usr/bin/env python3
"""Decode-step benchmark of the ParisKV retrieval + sparse-attention path on one MI355X.

One step = one decode token of one layer for a batch of 4 sequences at 128K
context (8 KV heads, 32 query heads, head dim 128, bf16): append the new
token (every 256 steps of a layer this evicts 256 local tokens into the
retrieval zone and encodes them), rotate the queries and build the vote
table, collision-vote scan of every retrieval-zone key, coarse top 5 %,
RSQ-IP rerank, top-2048, and GQA attention over sink + local + buffer +
retrieved keys.  Steps cycle over 4 layer replicas so that one step's
~136 MB working set is not served from the 256 MB last-level cache.

Prints one JSON line.  Inputs are synthetic (seeded), resident in HBM before
the timed region.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode retrieval+sparse-attn steps/s and HBM GB/s % peak at 128K ctx"
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--context", type=int, default=131072)
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--buf-tokens", type=int, default=256)
    ap.add_argument("--profile-steps", type=int, default=40)
    ap.add_argument("--warm-steps", type=int, default=256,
                    help="steps timed on one layer replica only (its working set can stay in "
                         "the last-level cache), reported beside the graded cycled figure")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=4)
    ap.add_argument("--no-sub-configs", action="store_true",
                    help="default run only: skip the compact 1M host-store and drift records")
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--sweep", choices=("capacity", "variants"), default=None,
                    help="capacity: sparse decode step vs dense attention at 128K..1M tokens, "
                         "batch 4; variants: probe count, vote weights and coarse fraction at "
                         "128K, batch 4 (time, bytes and recall per setting); one JSON line each")
    ap.add_argument("--sweep-steps", type=int, default=256)
    ap.add_argument("--centroids", choices=("analytic", "learned"), default="analytic",
                    help="--config 5 only: the page's analytic centroids, or the comparison "
                         "stage with centroids fitted by k-means to the prefill keys")
    ap.add_argument("--kmeans-iters", type=int, default=10)
    ap.add_argument("--drift-sigma", type=float, default=2.0,
                    help="--config 5 only: drift of the key/query mean over the decode steps")
    ap.add_argument("--config", type=int, default=3, choices=(3, 4, 5),
                    help="3: 128K context, batch 4 (default); 4: 1M context, K/V store in pinned "
                         "host memory; 5: 16384 drifting decode steps after a 32K prefill")
    return ap.parse_args()


def stream_reference(torch, scan_bytes=None):
    """Plain streaming kernels on this GPU over 1 GiB: the library's streaming-read
    reference kernel (pk_stream_read) and a torch device copy (read + write bytes).
    With scan_bytes, also the streaming read of exactly that many bytes (the scan's
    algorithmic bytes per launch), timed cold: a 1 GiB read of another buffer
    before each timed read evicts the last-level cache.  That read is timed by
    events attached to its dispatch, as the step's stages are."""
    import ctypes
    import kv_cache_top_amd._native as nat
    x = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").normal_()
    y = torch.empty_like(x)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def read():
        nat.check(nat.lib.pk_stream_read(ctypes.c_void_p(x.data_ptr()), 1 << 30,
                                         ctypes.c_void_p(sink.data_ptr()), None,
                                         ctypes.c_void_p(st)),
                  "pk_stream_read")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for name, fn, nbytes in (("read_GBps", read, 1 << 30), ("copy_GBps", lambda: y.copy_(x), 2 << 30)):
        for _ in range(3):
            fn()
        a.record()
        for _ in range(10):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[name] = nbytes * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    if scan_bytes:
        nb = int(scan_bytes) // 16 * 16
        part = y.view(torch.uint8)[:nb]
        kus = ctypes.c_float(0.0)
        times = []
        for i in range(9):
            read()                                   # evicts: 1 GiB of x
            nat.check(nat.lib.pk_stream_read(ctypes.c_void_p(part.data_ptr()), nb,
                                             ctypes.c_void_p(sink.data_ptr()), ctypes.byref(kus),
                                             ctypes.c_void_p(st)),
                      "pk_stream_read")
            if i > 0:
                times.append(kus.value)
        us = float(np.mean(times))
        out["read_scan_bytes"] = {"bytes": nb, "us": us, "GBps": nb / (us * 1e-6) / 1e9,
                                  "timing": "dispatch events, cold (mean of 8)"}
    del x, y
    torch.cuda.empty_cache()
    return out


def gather_reference(torch, layer, reps=8):
    """Plain random gathers on this GPU with the library's gather-read reference
    kernel (pk_gather_read), in the access patterns of the step's gather stages
    on this layer's window: the rerank's records (C random retrieval-zone
    positions per unit, ascending, 128-byte records over an array the size of
    the records) and the attention's rows (2 k random positions per unit,
    256-byte rows over an array the size of the K store).  A 1 GiB streaming
    read before each timed gather evicts the last-level cache; the gather alone
    is timed by events attached to its dispatch, as the step's stages are."""
    import ctypes
    import kv_cache_top_amd._native as nat
    wl, p = layer.wl, layer.wl.params
    units, cap = wl.n_units, layer.cap
    n, sink_end, r_end, _ = layer.ctx.window()
    n_r = r_end - sink_end
    C = min(n_r, max(p.top_k, (p.coarse_permille * n_r + 999) // 1000))
    k = min(p.top_k, C)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    base = (torch.arange(units, device="cuda", dtype=torch.int64) * cap + sink_end)[:, None]
    out = {}
    for name, rec_bytes, per_unit in (("records_128B", 128, C), ("rows_256B", 256, 2 * k)):
        arr = torch.empty(units * cap * rec_bytes, dtype=torch.uint8, device="cuda")
        sets = []
        for _ in range(reps):
            pos = torch.rand(units, n_r, device="cuda", generator=gen).argsort(dim=1)[:, :per_unit]
            sets.append((pos.sort(dim=1).values + base).to(torch.int32).contiguous())
        kus = ctypes.c_float(0.0)
        times = []
        for i in range(reps + 1):
            nat.check(nat.lib.pk_stream_read(ctypes.c_void_p(flush.data_ptr()), 1 << 30,
                                             ctypes.c_void_p(sink.data_ptr()), None, st),
                      "pk_stream_read")
            nat.check(nat.lib.pk_gather_read(ctypes.c_void_p(arr.data_ptr()), units * cap, rec_bytes,
                                             ctypes.c_void_p(sets[i % reps].data_ptr()),
                                             units * per_unit, ctypes.c_void_p(sink.data_ptr()),
                                             ctypes.byref(kus), st),
                      "pk_gather_read")
            if i > 0:
                times.append(kus.value)
        torch.cuda.synchronize()
        us = float(np.mean(times))
        nbytes = units * per_unit * rec_bytes
        out[name] = {"bytes": nbytes, "us": us, "GBps": nbytes / (us * 1e-6) / 1e9}
        del arr, sets
    del flush
    torch.cuda.empty_cache()
    return out


def stage_times(ctx_list, steps_fn, n_steps, torch, nat):
    """Per-stage kernel durations (dispatch-attached HIP events) over n_steps."""
    for c in ctx_list:
        c.profile(True)
    steps_fn(n_steps)
    torch.cuda.synchronize()
    ms = {k: 0.0 for k in nat.STAGES}
    cnt = {k: 0 for k in nat.STAGES}
    for c in ctx_list:
        for k, (m, n) in c.profile_read().items():
            ms[k] += m
            cnt[k] += n
        c.profile(False)
    return {k: {"launches": cnt[k], "avg_us": 1e3 * ms[k] / cnt[k]} for k in nat.STAGES if cnt[k]}


def run_config4(args):
    print(json.dumps(config4_record(args, args.steps, args.warmup)), flush=True)


def config4_record(args, n_steps, n_warmup):
    """1M-token context, batch 1 x 8 kv heads (G = 4), bf16, the K/V store in pinned host
    memory: ids and records in HBM, sink/local/buffer rows in a device ring, the
    retrieved rows read by the attention kernel over the host link."""
    import torch
    import kv_cache_top_amd._native as nat
    from kv_cache_top_amd import ParisKV
    from synth import workloads as W
    N = 1 << 20
    t0 = time.time()
    wl = W.gqa_bf16(N=N, batch=1, n_local=1024, buf_tokens=args.buf_tokens, threads=args.threads,
                    name="gqa_1m_b1_host_store_bf16")
    p = wl.params
    dt = torch.bfloat16
    ctx = ParisKV(batch=1, n_kv=8, n_q=32, capacity=N + n_steps + n_warmup + 96, dtype=dt,
                  host_mapped=True, rho=p.rho, vote_weights=p.vote_weights,
                  coarse_permille=p.coarse_permille, top_k=p.top_k, n_sink=p.n_sink,
                  n_local=p.n_local, buf_tokens=p.buf_tokens,
                  sign_bits=tuple(int(x) for x in wl.sign_bits))
    ctx.K[:, :, :N].copy_(torch.from_numpy(wl.K).to(dt))
    ctx.V[:, :, :N].copy_(torch.from_numpy(wl.V).to(dt))
    log(f"1M context generated and stored in host memory in {time.time() - t0:.1f}s")
    ctx.profile(True)
    ctx.encode_keys(N)
    enc_ms = ctx.profile_read()["encode"][0]
    ctx.profile(False)
    pool = 16
    q = torch.from_numpy(W.query_pool(wl, pool)).to(dt).cuda()
    kn, vn, _ = W.decode_stream(wl, pool, drift_sigma=0.0)
    kn, vn = torch.from_numpy(kn).to(dt).cuda(), torch.from_numpy(vn).to(dt).cuda()
    sel = torch.empty((1, 8, p.top_k), dtype=torch.int32, device="cuda")
    sel_n = torch.empty((1, 8), dtype=torch.int32, device="cuda")
    out = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    state = {"t": 0}

    def steps(n):
        for _ in range(n):
            i = state["t"] % pool
            state["t"] += 1
            ctx.decode_step_raw(kn[i].data_ptr(), vn[i].data_ptr(), q[i].data_ptr(), sel.data_ptr(),
                                sel_n.data_ptr(), out.data_ptr(), stream)

    steps(n_warmup)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    steps(n_steps)
    b.record()
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / n_steps
    stages = stage_times([ctx], steps, min(args.profile_steps, 32), torch, nat)
    n, sink_end, r_end, _ = ctx.window()
    # recall@k of the last step's selection against the exact top-k of the
    # retrieval zone (appended and evicted tokens included, read from the store)
    torch.cuda.synchronize()
    q_last = q[(state["t"] - 1) % pool].float().cpu().numpy()
    sel_h, sel_nh = sel.cpu().numpy().reshape(8, -1), sel_n.cpu().numpy().reshape(-1)
    pos = np.arange(sink_end, r_end)
    rec = [recall_at_k(sel_h[h][:sel_nh[h]],
                       exact_topk(ctx.K[0, h, :r_end].float().numpy(), q_last[0, 4 * h:4 * h + 4],
                                  pos, p.top_k))
           for h in range(8)]
    n_r = r_end - sink_end
    C = min(n_r, max(p.top_k, (p.coarse_permille * n_r + 999) // 1000))
    scan_b, rerank_b = 16 * n_r * 8, 128 * C * 8
    host_b = 512 * min(p.top_k, C) * 8              # retrieved K and V rows over the host link
    ring_b = 512 * (sink_end + n - r_end) * 8       # hot rows from the device ring
    st = lambda k: stages[k]["avg_us"] * 1e-6
    result = {
        "metric": "decode retrieval+sparse-attn steps/s at 1M ctx, K/V store in host memory",
        "value": 1e3 / ms_step, "unit": "steps/s", "n_gpus": 1, "steps": n_steps,
        "warmup": n_warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": 1, "kv_heads": 8, "q_heads": 32, "head_dim": 128,
                   "context": N, "kv_store": "pinned host memory", "top_k": p.top_k,
                   "coarse_permille": p.coarse_permille, "sink": p.n_sink, "local": p.n_local,
                   "update_buffer": p.buf_tokens},
        "hbm": {"scan_GBps": scan_b / st("scan") / 1e9, "rerank_GBps": rerank_b / st("rerank") / 1e9,
                "scan_bytes": scan_b, "rerank_bytes": rerank_b},
        "host_link": {"retrieved_bytes_per_step": host_b, "ring_bytes_per_step": ring_b,
                      "attend_us": stages["attend"]["avg_us"],
                      "retrieved_GBps": host_b / st("attend") / 1e9},
        "stages": stages,
        "encode": {"keys": 8 * n_r, "ms": enc_ms, "host_read_GBps": 8 * n_r * 256 / (enc_ms * 1e-3) / 1e9},
        "recall_at_k": float(np.mean(rec)),
        "wall_s": round(time.time() - t0, 1),
    }
    ctx.close()
    del ctx, wl
    torch.cuda.empty_cache()
    return result


def run_config5(args):
    print(json.dumps(config5_record(args)), flush=True)


def config5_record(args):
    """Drifting decode: 32768-token prefill (batch 1 x 8 kv heads, G = 4, bf16), then
    16384 decode steps whose key/query mean drifts by two standard deviations; U = 256,
    k = 1024.  Timed in 16 segments of 1024 steps; recall@k of every unit against the
    exact top-k of its retrieval zone after each segment (untimed)."""
    import torch
    from kv_cache_top_amd import ParisKV
    from synth import workloads as W
    N0, T, seg = 32768, 16384, 1024
    t_wall = time.time()
    wl = W.gqa_bf16(N=N0, top_k=1024, buf_tokens=256, threads=args.threads,
                    name="gqa_32k_drift16k_bf16")
    p = wl.params
    Kn, Vn, Qn = W.decode_stream(wl, T, drift_sigma=args.drift_sigma)
    dt = torch.bfloat16
    ctx = ParisKV(batch=1, n_kv=8, n_q=32, capacity=N0 + T, dtype=dt, rho=p.rho,
                  vote_weights=p.vote_weights, coarse_permille=p.coarse_permille, top_k=p.top_k,
                  n_sink=p.n_sink, n_local=p.n_local, buf_tokens=p.buf_tokens,
                  sign_bits=tuple(int(x) for x in wl.sign_bits))
    ctx.K[:, :, :N0].copy_(torch.from_numpy(wl.K).to(dt))
    ctx.V[:, :, :N0].copy_(torch.from_numpy(wl.V).to(dt))
    fit_ms = None
    if args.centroids == "learned":
        init = torch.from_numpy(W.kmeans_init_positions(8, N0)).cuda()
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        ctx.fit_centroids(N0, init, args.kmeans_iters)
        f1.record()
        torch.cuda.synchronize()
        fit_ms = f0.elapsed_time(f1)
        log(f"k-means fit ({args.kmeans_iters} iterations, {8 * N0} keys): {fit_ms:.2f} ms")
    ctx.encode_keys(N0)
    Kd, Vd, Qd = (torch.from_numpy(x).to(dt).cuda() for x in (Kn, Vn, Qn))
    Kall = np.concatenate([wl.K, np.moveaxis(Kn, 0, 2)], axis=2)
    sel = torch.empty((1, 8, p.top_k), dtype=torch.int32, device="cuda")
    sel_n = torch.empty((1, 8), dtype=torch.int32, device="cuda")
    out = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total_ms, curve = 0.0, []
    for s0 in range(0, T, seg):
        a.record()
        for t in range(s0, s0 + seg):
            ctx.decode_step_raw(Kd[t].data_ptr(), Vd[t].data_ptr(), Qd[t].data_ptr(), sel.data_ptr(),
                                sel_n.data_ptr(), out.data_ptr(), stream)
        b.record()
        torch.cuda.synchronize()
        total_ms += a.elapsed_time(b)
        n, sink_end, r_end, _ = ctx.window()
        s_h, n_h = sel.cpu().numpy().reshape(8, -1), sel_n.cpu().numpy()[0]
        pos = np.arange(sink_end, r_end)
        rec = [recall_at_k(s_h[u][:n_h[u]], exact_topk(Kall[0, u], Qn[s0 + seg - 1, 0, 4 * u:4 * u + 4],
                                                       pos, p.top_k)) for u in range(8)]
        curve.append(round(float(np.mean(rec)), 4))
        log(f"steps {s0 + seg}: window {ctx.window()}, recall@k {curve[-1]:.3f}")
    result = {
        "metric": "drifting decode steps/s over 16384 steps after a 32K prefill, recall@k per 1K steps",
        "value": T / (total_ms * 1e-3), "unit": "steps/s", "n_gpus": 1, "steps": T, "warmup": 0,
        "ms_per_step": total_ms / T, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": 1, "kv_heads": 8, "q_heads": 32, "head_dim": 128,
                   "prefill": N0, "decode_steps": T, "drift_sigma": args.drift_sigma, "top_k": p.top_k,
                   "coarse_permille": p.coarse_permille, "sink": p.n_sink, "local": p.n_local,
                   "update_buffer": p.buf_tokens, "centroids": args.centroids},
        "recall_at_k_per_1k_steps": curve,
    }
    if fit_ms is not None:
        result["kmeans_fit"] = {"iterations": args.kmeans_iters, "keys": 8 * N0, "ms": fit_ms}
    result["wall_s"] = round(time.time() - t_wall, 1)
    ctx.close()
    del ctx, Kd, Vd, Qd
    torch.cuda.empty_cache()
    return result


def calibrate_copy():
    """A plain device-to-device copy of a known size, 8 times; under
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE its per-dispatch readings give the
    counters' scale (expected: 1 GiB read and 1 GiB written per dispatch)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "dispatches": 8}), flush=True)


class Layer:
    """One layer replica: its ParisKV context, query and token pools, outputs.
    `wl` reuses an already drawn workload; `override` replaces method parameters
    (rho, vote_weights, coarse_permille)."""

    def __init__(self, args, layer, pool=8, wl=None, **override):
        import dataclasses
        import torch
        from kv_cache_top_amd import ParisKV
        from synth import workloads as W
        t0 = time.time()
        if wl is None:
            wl = W.gqa_bf16(N=args.context, batch=args.batch, layer=layer, n_plant=64,
                            buf_tokens=args.buf_tokens, threads=args.threads,
                            name=f"gqa_{args.context // 1024}k_b{args.batch}_planted_bf16")
        if override:
            wl = dataclasses.replace(wl, params=dataclasses.replace(wl.params, **override))
        self.wl = wl
        p = wl.params
        steps_here = (args.warmup + args.steps + args.profile_steps) // args.layers + 2 + \
            (args.warm_steps + 16 if layer == 0 else 0)
        self.cap = args.context + steps_here + 8
        dt = torch.bfloat16
        self.ctx = ParisKV(batch=wl.batch, n_kv=wl.n_kv, n_q=wl.n_kv * wl.group, capacity=self.cap,
                           dtype=dt, rho=p.rho, vote_weights=p.vote_weights,
                           coarse_permille=p.coarse_permille, top_k=p.top_k, n_sink=p.n_sink,
                           n_local=p.n_local, buf_tokens=p.buf_tokens,
                           sign_bits=tuple(int(x) for x in wl.sign_bits),
                           codebook=0 if p.codebook == "lloyd_max" else 1, n_sub=p.n_sub,
                           sub_dim=p.sub_dim)
        N = wl.n_tokens
        self.ctx.K[:, :, :N].copy_(torch.from_numpy(wl.K).to(dt))
        self.ctx.V[:, :, :N].copy_(torch.from_numpy(wl.V).to(dt))
        qp = W.query_pool(wl, pool)
        kn, vn, _ = W.decode_stream(wl, pool, drift_sigma=0.0, layer=layer)
        self.q_host, self.kn_host = qp, kn       # host copies (the recall reference reads them)
        self.q = torch.from_numpy(qp).to(dt).cuda()
        self.kn = torch.from_numpy(kn).to(dt).cuda()
        self.vn = torch.from_numpy(vn).to(dt).cuda()
        self.sel = torch.empty((wl.batch, wl.n_kv, p.top_k), dtype=torch.int32, device="cuda")
        self.sel_n = torch.empty((wl.batch, wl.n_kv), dtype=torch.int32, device="cuda")
        self.out = torch.empty((wl.batch, wl.n_kv * wl.group, 128), dtype=torch.float32, device="cuda")
        self.pool = pool
        self.t = 0
        log(f"layer {layer}: generated and uploaded in {time.time() - t0:.1f}s")

        # per-step buffers validated once; the timed loop passes raw addresses
        for t in (self.q, self.kn, self.vn):
            assert t.is_contiguous()
        self._args = [(self.kn[i].data_ptr(), self.vn[i].data_ptr(), self.q[i].data_ptr(),
                       self.sel.data_ptr(), self.sel_n.data_ptr(), self.out.data_ptr())
                      for i in range(pool)]
        self._stream = torch.cuda.current_stream().cuda_stream

    def step(self):
        i = self.t % self.pool
        self.t += 1
        self.ctx.decode_step_raw(*self._args[i], self._stream)


KERNEL_SOURCES = ("kv_cache_top_amd/csrc/pk_scan.hip", "kv_cache_top_amd/csrc/pk_device.hpp")
TRAFFIC_PROFILE = "profiles/scan_kernel_gqa128k_b4_hbm_traffic.txt"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per scan launch from the committed counter summary (rocprofv3
    FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's readings), or None when
    the summary is missing or the scan kernel's sources changed since."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def counts(layer):
    """Algorithmic HBM bytes of one step's scan / rerank / attention on this layer at
    its current window: scan 16 B per retrieval-zone key, rerank one record per
    candidate (64 B of codes + 4 B per subspace: 128 B for m = 8), attention one bf16 K row and one V row (512 B) per attended key.  The
    hot-zone rows (sink, local, buffer) are gathered by the fine-selection launch
    (bf16 device stores, G <= 4, at most 16384 candidates), the selected rows by
    the attention launch."""
    p = layer.wl.params
    n, sink_end, r_end, buf = layer.ctx.window()
    units = layer.wl.n_units
    n_r = r_end - sink_end
    C = min(n_r, max(p.top_k, (p.coarse_permille * n_r + 999) // 1000))
    k_eff = min(p.top_k, C)
    hot = sink_end + (n - r_end)
    fused = layer.wl.dtype == "bf16" and layer.wl.group <= 4 and C <= 16384 and \
        not getattr(layer, "host_mapped", False)
    return dict(scan=16 * n_r * units, rerank=(64 + 4 * p.n_sub) * C * units,
                attend=512 * (k_eff + (0 if fused else hot)) * units,
                fine=512 * hot * units if fused else 0, keys=n_r * units)


def dense_reference(torch, layer, ms_step, reps=20):
    """Full attention over every stored token of the layer (pk_dense_attend, same
    split kernel and merge), the decode attention the retrieval path replaces:
    its time per call, its rate over the K/V bytes it reads, and the whole sparse
    decode step's speedup over it."""
    ctx = layer.ctx
    q = layer.q[0] if layer.q.dim() == 4 else layer.q
    out = torch.empty((ctx.batch, ctx.n_q, 128), dtype=torch.float32, device="cuda")
    for _ in range(3):
        ctx.dense_attend(q, out)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        ctx.dense_attend(q, out)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    n = ctx.window()[0]
    nbytes = 512 * n * layer.wl.n_units
    return {"us_per_call": us, "bytes_per_call": nbytes, "GBps": nbytes / (us * 1e-6) / 1e9,
            "sparse_step_speedup": us / (ms_step * 1e3)}


def cpu_baseline(args, layer, budget_s=10.0):
    """The oracle (plain numpy, single thread) on a bounded sample: decode steps of
    `cpu_units` of the (batch, kv-head) units of one layer (their keys encoded
    first, untimed), repeated over the layer's query pool for about `budget_s`
    seconds, scaled to steps/s of the whole batch."""
    from threadpoolctl import threadpool_limits
    from oracle import pariskv as ok
    from oracle.codebook import spec_tables
    wl = layer.wl
    p = wl.params
    levels, sq_t = spec_tables()
    s = wl.signs()
    N = wl.n_tokens
    win = ok.Window(N, p.n_sink, p.n_local, p.buf_tokens)
    units = list(range(min(args.cpu_units, wl.n_units)))
    qpool = layer.q.float().cpu().numpy()
    with threadpool_limits(limits=1):
        metas = []
        for u in units:
            b, h = divmod(u, wl.n_kv)
            metas.append(ok.encode_keys(wl.K[b, h], s, levels, sq_t))
        n = 0
        t0 = time.perf_counter()
        while True:
            for u, (ids, nib, w) in zip(units, metas):
                b, h = divmod(u, wl.n_kv)
                Qg = qpool[n % len(qpool), b, 4 * h:4 * h + 4]
                ok.decode_step(wl.K[b, h], wl.V[b, h], Qg, ids, nib, w, win, s, levels, rho=p.rho,
                               weights=p.vote_weights, permille=p.coarse_permille, top_k=p.top_k)
            n += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s or n >= 200:
                break
    per_unit = dt / (n * len(units))
    return {"value": 1.0 / (per_unit * wl.n_units), "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{n * len(units)} oracle unit-steps (query prep, vote scan, coarse, RSQ-IP "
                      f"rerank, top-k, attention) on {len(units)} of the {wl.n_units} (batch, kv-head) "
                      f"units of one layer at {N} tokens, {dt:.1f}s single-threaded, scaled to a "
                      f"whole-batch step"}


def exact_topk(K, Qg, positions, k):
    """Quality reference for recall@k (not part of the method): the k positions with the
    largest summed raw score sum_g <q_g, k_i> in float64, ties to the lower position."""
    s = np.asarray(K, np.float64)[positions] @ np.atleast_2d(np.asarray(Qg, np.float64)).sum(0)
    order = np.lexsort((positions, -s))
    return positions[order[:min(k, positions.size)]]


def recall_at_k(selected, reference):
    return len(np.intersect1d(selected, reference)) / len(reference) if len(reference) else 1.0


def recall(layer):
    wl = layer.wl
    n, sink_end, r_end, _ = layer.ctx.window()
    sel = layer.sel.cpu().numpy().reshape(wl.n_units, -1)
    sel_n = layer.sel_n.cpu().numpy().reshape(-1)
    q = layer.q[(layer.t - 1) % layer.pool].float().cpu().numpy()
    rec, pl = [], []
    for u in range(0, wl.n_units, 4):
        b, h = divmod(u, wl.n_kv)
        K = wl.K[b, h]
        pos = np.arange(sink_end, min(r_end, wl.n_tokens))
        ref = exact_topk(K, q[b, 4 * h:4 * h + 4], pos, wl.params.top_k)
        got = sel[u][:sel_n[u]]
        rec.append(recall_at_k(got, ref))
        pl.append(float(np.isin(wl.planted[b, h], got).mean()))
    return float(np.mean(rec)), float(np.mean(pl))


def recall_all(layers, per_layer=2, threads=16):
    """recall@k and planted recall of every unit over `per_layer` further decode steps
    of each layer replica.  The exact top-k ranks the unit's whole retrieval zone at
    that step (prefill keys and the decode tokens evicted into it: the token appended
    at a layer's step t is its pool entry t mod pool) by sum_g <q_g, k_i> in float64,
    ties to the lower position.  Returns (recall@k, planted recall, unit-steps)."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    recs, plants = [], []
    for L in layers:
        wl = L.wl
        N, G = wl.n_tokens, wl.group
        snaps = []
        for _ in range(per_layer):
            L.step()
            torch.cuda.synchronize()
            snaps.append((L.ctx.window(), L.sel.cpu().numpy().reshape(wl.n_units, -1).copy(),
                          L.sel_n.cpu().numpy().reshape(-1).copy(), L.q_host[(L.t - 1) % L.pool]))
        r_max = max(w[2] for w, _, _, _ in snaps)

        def unit(u):
            b, h = divmod(u, wl.n_kv)
            K = wl.K[b, h, :min(r_max, N)].astype(np.float64)
            if r_max > N:
                K = np.concatenate([K, L.kn_host[np.arange(r_max - N) % L.pool, b, h].astype(np.float64)])
            out = []
            for (n, sink_end, r_end, _), sel, sel_n, q in snaps:
                pos = np.arange(sink_end, r_end)
                sc = K[sink_end:r_end] @ q[b, G * h:G * h + G].astype(np.float64).sum(0)
                ref = pos[np.lexsort((pos, -sc))[:min(wl.params.top_k, pos.size)]]
                got = sel[u][:sel_n[u]]
                out.append((recall_at_k(got, ref), float(np.isin(wl.planted[b, h], got).mean())))
            return out
        with ThreadPoolExecutor(threads) as ex:
            for res in ex.map(unit, range(wl.n_units)):
                for r, p_ in res:
                    recs.append(r)
                    plants.append(p_)
    return float(np.mean(recs)), float(np.mean(plants)), len(recs)


def cpu_threads():
    """Host threads for the oracle's all-cores run: the process's CPU share, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline_all_cores(args, layer, budget_s=10.0):
    """The oracle on every (batch, kv-head) unit of one layer, the units split over
    the host's threads (one numpy thread each): every unit encoded first (untimed),
    then whole-batch decode steps over the layer's query pool for about `budget_s`
    seconds."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import pariskv as ok
    from oracle.codebook import spec_tables
    wl = layer.wl
    p = wl.params
    levels, sq_t = spec_tables()
    s = wl.signs()
    N = wl.n_tokens
    win = ok.Window(N, p.n_sink, p.n_local, p.buf_tokens)
    qpool = layer.q.float().cpu().numpy()
    n_thr = cpu_threads()
    G = wl.group

    def enc(u):
        b, h = divmod(u, wl.n_kv)
        return ok.encode_keys(wl.K[b, h], s, levels, sq_t)

    def step(args_):
        u, i = args_
        b, h = divmod(u, wl.n_kv)
        ids, nib, w = metas[u]
        ok.decode_step(wl.K[b, h], wl.V[b, h], qpool[i % len(qpool), b, G * h:G * h + G], ids, nib, w,
                       win, s, levels, rho=p.rho, weights=p.vote_weights,
                       permille=p.coarse_permille, top_k=p.top_k)
    with threadpool_limits(limits=1), ThreadPoolExecutor(n_thr) as ex:
        metas = list(ex.map(enc, range(wl.n_units)))
        n = 0
        t0 = time.perf_counter()
        while True:
            list(ex.map(step, [(u, n) for u in range(wl.n_units)]))
            n += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s or n >= 200:
                break
    return {"value": n / dt, "unit": "steps/s", "cores": n_thr, "kind": "oracle",
            "sample": f"{n} whole-batch oracle decode steps (query prep, vote scan, coarse, RSQ-IP "
                      f"rerank, top-k, attention of all {wl.n_units} (batch, kv-head) units of one "
                      f"layer at {N} tokens, the units split over {n_thr} threads), {dt:.1f}s"}


def graph_replay_timing(torch, layer, reps=200):
    """Static retrieval + sparse attention (no append: the window does not move) on
    one layer replica, issued eagerly and as replays of a HIP graph capturing the same
    two calls: microseconds per call pair, and whether the replays' outputs equal the
    eager ones."""
    ctx, q = layer.ctx, layer.q[0]
    sel, sel_n, out = layer.sel, layer.sel_n, layer.out

    def eager():
        ctx.retrieve(q, sel, sel_n)
        ctx.sparse_attend(q, sel, sel_n, out)
    for _ in range(8):
        eager()
    torch.cuda.synchronize()
    ref = (sel.clone(), out.clone())
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        eager()
    b.record()
    torch.cuda.synchronize()
    us_eager = a.elapsed_time(b) / reps * 1e3
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        ctx.retrieve(q, sel, sel_n, stream=st)
        ctx.sparse_attend(q, sel, sel_n, out, stream=st)
    for _ in range(4):
        g.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us_graph = a.elapsed_time(b) / reps * 1e3
    same = bool(torch.equal(sel, ref[0]) and torch.equal(out, ref[1]))
    del g
    return {"us_eager": us_eager, "us_graph_replay": us_graph, "replay_equals_eager": same,
            "calls": "pk_retrieve + pk_sparse_attend, static context (one layer replica)"}


class DeviceLayer:
    """A layer replica for the capacity sweep: the gqa_bf16 recipe (no planted set)
    drawn on the GPU at any context length, with the same step interface as Layer."""

    def __init__(self, N, batch, layer, steps_here, buf_tokens, pool=8):
        import types
        import torch
        from kv_cache_top_amd import ParisKV
        from synth import workloads as W
        p = W.Params(buf_tokens=buf_tokens)
        self.wl = types.SimpleNamespace(params=p, n_units=batch * 8, dtype="bf16", group=4,
                                        batch=batch, n_kv=8)
        dt = torch.bfloat16
        self.ctx = ParisKV(batch=batch, n_kv=8, n_q=32, capacity=N + steps_here + 8, dtype=dt,
                           rho=p.rho, vote_weights=p.vote_weights,
                           coarse_permille=p.coarse_permille, top_k=p.top_k, n_sink=p.n_sink,
                           n_local=p.n_local, buf_tokens=p.buf_tokens,
                           sign_bits=tuple(int(x) for x in W.sign_bits(0, layer)))
        qp, kp, vp = W.fill_gqa_device(self.ctx.K, self.ctx.V, N, seed=0, layer=layer, pool=pool)
        self.q = torch.from_numpy(qp).to(dt).cuda()
        self.kn = torch.from_numpy(kp).to(dt).cuda()
        self.vn = torch.from_numpy(vp).to(dt).cuda()
        self.sel = torch.empty((batch, 8, p.top_k), dtype=torch.int32, device="cuda")
        self.sel_n = torch.empty((batch, 8), dtype=torch.int32, device="cuda")
        self.out = torch.empty((batch, 32, 128), dtype=torch.float32, device="cuda")
        self.pool, self.t = pool, 0
        self.ctx.encode_keys(N)
        self._stream = torch.cuda.current_stream().cuda_stream

    def step(self):
        i = self.t % self.pool
        self.t += 1
        self.ctx.decode_step_raw(self.kn[i].data_ptr(), self.vn[i].data_ptr(), self.q[i].data_ptr(),
                                 self.sel.data_ptr(), self.sel_n.data_ptr(), self.out.data_ptr(),
                                 self._stream)


def time_steps(torch, layers, warmup, steps):
    """ms per decode step over `steps` steps cycling the layers (after `warmup`)."""
    nl = len(layers)
    for i in range(warmup):
        layers[i % nl].step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        layers[(warmup + i) % nl].step()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def profiled_stages(torch, nat, layers, n):
    """Average per-stage kernel durations (us) over n more steps."""
    for L in layers:
        L.ctx.profile(True)
    for i in range(n):
        layers[i % len(layers)].step()
    torch.cuda.synchronize()
    ms, cnt = {k: 0.0 for k in nat.STAGES}, {k: 0 for k in nat.STAGES}
    for L in layers:
        for k, (m, c) in L.ctx.profile_read().items():
            ms[k] += m
            cnt[k] += c
        L.ctx.profile(False)
    return {k: round(1e3 * ms[k] / cnt[k], 2) for k in nat.STAGES if cnt[k]}


def run_capacity_sweep(args):
    """Sparse decode step against dense attention over every stored token, at 128K,
    256K, 384K and 1M tokens, batch 4 x 8 kv heads (G = 4, bf16, top-k 2048, coarse
    5 %), K/V drawn on the GPU; layer replicas are cycled while one step's working
    set is below twice the 256 MB last-level cache.  Also the batch that 288 GB-class
    HBM holds at each context, from the bytes each design keeps per token: dense
    attention K/V only (512 B), the retrieval path with the store in HBM (K/V + 16 B
    ids + 128 B records), and with the store in host memory (ids + records)."""
    import torch
    import kv_cache_top_amd._native as nat
    free, total = torch.cuda.mem_get_info()
    B = args.batch
    units = 8 * B
    for N in (131072, 262144, 393216, 1 << 20):
        t0 = time.time()
        ws = units * (16 * N + 128 * max(2048, N // 20) + 512 * (2048 + 516))
        nl = max(1, min(4, -(-(512 << 20) // ws)))
        steps_here = (16 + args.sweep_steps + 32) // nl + 2
        layers = [DeviceLayer(N, B, l, steps_here, args.buf_tokens) for l in range(nl)]
        torch.cuda.synchronize()
        ms = time_steps(torch, layers, 16, args.sweep_steps)
        st = profiled_stages(torch, nat, layers, 32)
        c = counts(layers[0])
        dense = dense_reference(torch, layers[0], ms, reps=5)
        per_tok = {"dense_kv": 512, "paris_store_in_hbm": 512 + 144, "paris_store_in_host": 144}
        max_batch = {k: int(total // (8 * N * v)) for k, v in per_tok.items()}
        print(json.dumps({
            "sweep": "capacity", "context": N, "batch": B, "layers_cycled": nl,
            "sparse_us_per_step": round(1e3 * ms, 2), "sparse_steps_per_s": round(1e3 / ms, 1),
            "stages_us": st,
            "sparse_alg_bytes_per_step": int(c["scan"] + c["rerank"] + c["attend"] + c["fine"]),
            "dense_us_per_call": round(dense["us_per_call"], 1),
            "dense_bytes_per_call": dense["bytes_per_call"], "dense_GBps": round(dense["GBps"], 1),
            "sparse_step_speedup_over_dense": round(dense["sparse_step_speedup"], 2),
            "max_batch_by_hbm_bytes": max_batch, "hbm_total_bytes": int(total),
            "wall_s": round(time.time() - t0, 1)}), flush=True)
        for L in layers:
            L.ctx.close()
        del layers
        torch.cuda.empty_cache()


def estimate_error(layer):
    """RMS error of the last step's RSQ-IP estimates against the exact summed inner
    products sum_g <k_i, q_g> of the candidates, relative to the RMS of the exact
    values (every fourth unit); a quality measure of the codes, not part of the path."""
    wl = layer.wl
    cand, est, meta = (layer.ctx.debug(i) for i in (4, 5, 6))
    q = layer.q[(layer.t - 1) % layer.pool].float().cpu().numpy()
    num = den = 0.0
    for u in range(0, wl.n_units, 4):
        b, h = divmod(u, wl.n_kv)
        C = int(meta[u][2])
        pos = cand[u][:C]
        exact = wl.K[b, h][pos].astype(np.float64) @ q[b, 4 * h:4 * h + 4].astype(np.float64).sum(0)
        num += float(np.sum((est[u][:C].astype(np.float64) - exact) ** 2))
        den += float(np.sum(exact ** 2))
    return math.sqrt(num / den) if den else None


def run_variant_sweep(args):
    """The knobs the page leaves open (probe count rho, the hierarchical vote weights,
    the coarse fraction, the codebook, the subspace width m) at 128K, batch 4, planted workload: step time, per-stage
    durations, algorithmic bytes and recall@k / planted recall (mean over one step
    per layer replica, every fourth unit) per setting."""
    import copy
    import torch
    import kv_cache_top_amd._native as nat
    from synth import workloads as W
    a = copy.copy(args)
    a.steps, a.warmup, a.profile_steps = args.sweep_steps, 16, 32
    wls = [W.gqa_bf16(N=a.context, batch=a.batch, layer=l, n_plant=64, buf_tokens=a.buf_tokens,
                      threads=a.threads, name=f"gqa_{a.context // 1024}k_b{a.batch}_planted_bf16")
           for l in range(a.layers)]
    variants = [dict(rho=4, vote_weights=(4, 3, 2, 1), coarse_permille=50),
                dict(rho=1, vote_weights=(1,), coarse_permille=50),
                dict(rho=2, vote_weights=(2, 1), coarse_permille=50),
                dict(rho=8, vote_weights=(8, 7, 6, 5, 4, 3, 2, 1), coarse_permille=50),
                dict(rho=4, vote_weights=(8, 4, 2, 1), coarse_permille=50),
                dict(rho=4, vote_weights=(4, 3, 2, 1), coarse_permille=100),
                dict(rho=4, vote_weights=(4, 3, 2, 1), coarse_permille=50, codebook="quantile"),
                dict(rho=4, vote_weights=(4, 3, 2, 1), coarse_permille=50, n_sub=32, sub_dim=4),
                dict(rho=4, vote_weights=(4, 3, 2, 1), coarse_permille=50, n_sub=8, sub_dim=16)]
    for v in variants:
        layers = [Layer(a, l, wl=wls[l], **v) for l in range(a.layers)]
        for L in layers:
            L.ctx.encode_keys(L.wl.n_tokens)
        torch.cuda.synchronize()
        ms = time_steps(torch, layers, a.warmup, a.steps)
        st = profiled_stages(torch, nat, layers, a.profile_steps)
        c = counts(layers[0])
        rec, pl, ee = [], [], []
        for L in layers:
            L.step()
            torch.cuda.synchronize()
            r, p_ = recall(L)
            rec.append(r)
            pl.append(p_)
            ee.append(estimate_error(L))
        print(json.dumps({
            "sweep": "variants", "context": a.context, "batch": a.batch,
            "rho": v["rho"], "vote_weights": list(v["vote_weights"]),
            "coarse_permille": v["coarse_permille"], "codebook": v.get("codebook", "lloyd_max"),
            "subspaces": v.get("n_sub", 16), "sub_dim": v.get("sub_dim", 8),
            "us_per_step": round(1e3 * ms, 2), "steps_per_s": round(1e3 / ms, 1), "stages_us": st,
            "alg_bytes_per_step": int(c["scan"] + c["rerank"] + c["attend"] + c["fine"]),
            "recall_at_k": round(float(np.mean(rec)), 4),
            "planted_recall": round(float(np.mean(pl)), 4),
            "estimate_rel_rms_error": round(float(np.mean(ee)), 5)}), flush=True)
        for L in layers:
            L.ctx.close()
        del layers
        torch.cuda.empty_cache()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus} GPUs, WORLD_SIZE={world}); "
              "the ParisKV path shards by (batch, kv-head) unit with no exchange, so there is no "
              "multi-GPU figure to take here.", flush=True)
        sys.exit(2)
    import torch
    import kv_cache_top_amd._native as nat
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.init()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.sweep == "capacity":
        return run_capacity_sweep(args)
    if args.sweep == "variants":
        return run_variant_sweep(args)
    if args.config == 4:
        return run_config4(args)
    if args.config == 5:
        return run_config5(args)

    layers = [Layer(args, l) for l in range(args.layers)]
    # prefill encode of every layer (timed per layer, reported separately)
    enc_ms = []
    for L in layers:
        L.ctx.profile(True)
        L.ctx.encode_keys(L.wl.n_tokens)
        enc_ms.append(L.ctx.profile_read()["encode"][0])
        L.ctx.profile(False)
    torch.cuda.synchronize()

    nl = len(layers)
    for i in range(args.warmup):
        layers[i % nl].step()
    torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    before = [counts(L) for L in layers]
    t_host = time.perf_counter()
    start.record()
    for i in range(args.steps):
        layers[(args.warmup + i) % nl].step()
    end.record()
    host_s = time.perf_counter() - t_host       # submission only (no wait)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    after = [counts(L) for L in layers]
    keys_per_step = np.mean([0.5 * (a["keys"] + b["keys"]) for a, b in zip(after, before)])

    # profiled pass: per-stage kernel durations from HIP events on the launch stream
    for L in layers:
        L.ctx.profile(True)
    sums = {k: 0.0 for k in ("scan", "rerank", "fine", "attend")}
    base = args.warmup + args.steps
    for i in range(args.profile_steps):
        L = layers[(base + i) % nl]
        c = counts(L)
        for k in sums:
            sums[k] += c[k]
        L.step()
    torch.cuda.synchronize()
    stage_ms = {k: 0.0 for k in nat.STAGES}
    stage_n = {k: 0 for k in nat.STAGES}
    for L in layers:
        for k, (ms, n) in L.ctx.profile_read().items():
            stage_ms[k] += ms
            stage_n[k] += n
        L.ctx.profile(False)
    stages = {}
    for name in nat.STAGES:
        if stage_n[name]:
            stages[name] = {"launches": stage_n[name], "avg_us": 1e3 * stage_ms[name] / stage_n[name]}
    n_prof = max(1, args.profile_steps)

    def gbs(name):
        if name not in stages:
            return None
        return (sums[name] / n_prof) / (stages[name]["avg_us"] * 1e-6) / 1e9

    scan_gbs = gbs("scan")
    comb_bytes = sum(sums.values()) / n_prof
    # the hot rows are gathered inside the fine-selection launch: its whole time counts
    comb_us = sum(stages[k]["avg_us"] for k in ("scan", "rerank", "attend") if k in stages)
    if sums["fine"] and "fine" in stages:
        comb_us += stages["fine"]["avg_us"]
    comb_gbs = comb_bytes / (comb_us * 1e-6) / 1e9 if comb_us else None
    for k in ("scan", "rerank", "attend") + (("fine",) if sums["fine"] else ()):
        if k in stages:
            stages[k]["alg_bytes"] = int(sums[k] / n_prof)
            stages[k]["GBps"] = gbs(k)

    dense = dense_reference(torch, layers[0], ms_step)
    warm = None
    if args.warm_steps > 0:
        ms_warm = time_steps(torch, [layers[0]], 16, args.warm_steps)
        warm = {"steps": args.warm_steps, "us_per_step": 1e3 * ms_warm, "steps_per_s": 1e3 / ms_warm}
    sref = stream_reference(torch, scan_bytes=stages.get("scan", {}).get("alg_bytes"))
    gref = gather_reference(torch, layers[0])
    if stages.get("scan", {}).get("GBps") and "read_scan_bytes" in sref:
        stages["scan"]["frac_of_same_size_read"] = stages["scan"]["GBps"] / sref["read_scan_bytes"]["GBps"]
    for k, ref in (("rerank", "records_128B"), ("attend", "rows_256B")):
        if stages.get(k, {}).get("GBps"):
            stages[k]["frac_of_gather_reference"] = stages[k]["GBps"] / gref[ref]["GBps"]
    graph = graph_replay_timing(torch, layers[0])
    log("recall over every unit ...")
    rec, planted, rec_n = recall_all(layers, threads=cpu_threads())
    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (all cores, then one core) on a bounded sample ...")
        cpu = cpu_baseline_all_cores(args, layers[0])
        cpu1 = cpu_baseline(args, layers[0])

    wl = layers[0].wl
    sub_cfg = {}
    if not args.no_sub_configs:
        for L in layers:
            L.ctx.close()
        del layers
        torch.cuda.empty_cache()
        log("1M-token host-store record ...")
        c4 = config4_record(args, 64, 8)
        sub_cfg["config_1m_host_store"] = {
            "workload": c4["config"]["workload"], "steps_per_s": c4["value"],
            "us_per_step": 1e3 * c4["ms_per_step"], "steps": c4["steps"],
            "stages_us": {k: round(v["avg_us"], 2) for k, v in c4["stages"].items()},
            "hbm": c4["hbm"], "host_link": c4["host_link"], "recall_at_k": c4["recall_at_k"],
            "wall_s": c4["wall_s"]}
        log("drift record ...")
        c5 = config5_record(args)
        sub_cfg["config_drift_32k_16k_steps"] = {
            "workload": c5["config"]["workload"], "steps_per_s": c5["value"],
            "us_per_step": 1e3 * c5["ms_per_step"], "steps": c5["steps"],
            "drift_sigma": c5["config"]["drift_sigma"],
            "recall_at_k_per_1k_steps": c5["recall_at_k_per_1k_steps"], "wall_s": c5["wall_s"]}
    enc_keys = wl.n_units * (wl.n_tokens - wl.params.n_sink - wl.params.n_local)
    result = {
        "metric": METRIC,
        "value": 1e3 / ms_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch": wl.batch, "kv_heads": wl.n_kv, "q_heads": wl.n_kv * wl.group, "head_dim": 128,
            "context": wl.n_tokens, "kv_dtype": "bf16", "top_k": wl.params.top_k,
            "coarse_permille": wl.params.coarse_permille, "rho": wl.params.rho,
            "subspaces": wl.params.n_sub, "sub_dim": wl.params.sub_dim,
            "sink": wl.params.n_sink, "local": wl.params.n_local,
            "update_buffer": wl.params.buf_tokens, "layers_cycled": nl,
        },
        "roofline": {
            "kernel": "scan (collision-vote scan)",
            "bound": "hbm",
            "achieved": scan_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": (scan_gbs / HBM_PEAK_GBS) if scan_gbs else None,
            "traffic": measured_traffic(),
            # a plain cold streaming read of the same bytes on this GPU
            "same_size_read_GBps": sref.get("read_scan_bytes", {}).get("GBps"),
            "frac_of_same_size_read": stages.get("scan", {}).get("frac_of_same_size_read"),
        },
        "retrieval_hbm": {"scan_rerank_gather_GBps": comb_gbs,
                          "frac": comb_gbs / HBM_PEAK_GBS if comb_gbs else None,
                          "frac_of_stream_read": comb_gbs / sref["read_GBps"] if comb_gbs else None,
                          "bytes_per_step": int(comb_bytes), "kernel_us_per_step": comb_us},
        "stream_reference": sref,
        "gather_reference": gref,
        "dense_attention": dense,
        "warm_single_layer": warm,
        "stages": stages,
        "keys_scanned_per_s": keys_per_step * 1e3 / ms_step,
        "host_submit_ms_per_step": 1e3 * host_s / args.steps,
        "encode": {"keys": enc_keys, "avg_ms": float(np.mean(enc_ms)),
                   "GBps": enc_keys * 400 / (np.mean(enc_ms) * 1e-3) / 1e9},
        "recall_at_k": rec,
        "planted_recall": planted,
        "recall_sample": f"{rec_n} unit-steps: every unit of every layer replica, 2 decode steps each",
        "graph_replay": graph,
        "cpu_baseline": cpu,
        "cpu_baseline_one_core": cpu1,
        **sub_cfg,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
