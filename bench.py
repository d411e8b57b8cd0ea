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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=4)
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


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
    """One layer replica: its ParisKV context, query and token pools, outputs."""

    def __init__(self, args, layer, pool=8):
        import torch
        from kv_cache_top_amd import ParisKV
        from synth import workloads as W
        t0 = time.time()
        wl = W.gqa_bf16(N=args.context, batch=args.batch, layer=layer, n_plant=64,
                        buf_tokens=args.buf_tokens, threads=args.threads,
                        name=f"gqa_{args.context // 1024}k_b{args.batch}_planted_bf16")
        self.wl = wl
        p = wl.params
        steps_here = (args.warmup + args.steps + args.profile_steps) // args.layers + 2
        self.cap = args.context + steps_here + 8
        dt = torch.bfloat16
        self.ctx = ParisKV(batch=wl.batch, n_kv=wl.n_kv, n_q=wl.n_kv * wl.group, capacity=self.cap,
                           dtype=dt, rho=p.rho, vote_weights=p.vote_weights,
                           coarse_permille=p.coarse_permille, top_k=p.top_k, n_sink=p.n_sink,
                           n_local=p.n_local, buf_tokens=p.buf_tokens,
                           sign_bits=tuple(int(x) for x in wl.sign_bits))
        N = wl.n_tokens
        self.ctx.K[:, :, :N].copy_(torch.from_numpy(wl.K).to(dt))
        self.ctx.V[:, :, :N].copy_(torch.from_numpy(wl.V).to(dt))
        qp = W.query_pool(wl, pool)
        kn, vn, _ = W.decode_stream(wl, pool, drift_sigma=0.0, layer=layer)
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


KERNEL_SOURCES = ("kv_cache_top_amd/csrc/pk_retrieve.hip", "kv_cache_top_amd/csrc/pk_device.hpp")
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
    its current window: scan 16 B per retrieval-zone key, rerank 128 B per
    candidate, attention one bf16 K row and one V row (512 B) per attended key."""
    p = layer.wl.params
    n, sink_end, r_end, buf = layer.ctx.window()
    units = layer.wl.n_units
    n_r = r_end - sink_end
    C = min(n_r, max(p.top_k, (p.coarse_permille * n_r + 999) // 1000))
    k_eff = min(p.top_k, C)
    hot = sink_end + (n - r_end)
    return dict(scan=16 * n_r * units, rerank=128 * C * units, attend=512 * (hot + k_eff) * units,
                keys=n_r * units)


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


def recall(layer):
    from oracle import pariskv as ok
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
        ref = ok.exact_topk(K, q[b, 4 * h:4 * h + 4], pos, wl.params.top_k)
        got = sel[u][:sel_n[u]]
        rec.append(ok.recall(got, ref))
        pl.append(float(np.isin(wl.planted[b, h], got).mean()))
    return float(np.mean(rec)), float(np.mean(pl))


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
    sums = {k: 0.0 for k in ("scan", "rerank", "attend")}
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
    comb_us = sum(stages[k]["avg_us"] for k in ("scan", "rerank", "attend") if k in stages)
    comb_gbs = comb_bytes / (comb_us * 1e-6) / 1e9 if comb_us else None
    for k in ("scan", "rerank", "attend"):
        if k in stages:
            stages[k]["alg_bytes"] = int(sums[k] / n_prof)
            stages[k]["GBps"] = gbs(k)

    rec, planted = recall(layers[(base + args.profile_steps - 1) % nl])
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(args, layers[0])

    wl = layers[0].wl
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
        },
        "retrieval_hbm": {"scan_rerank_gather_GBps": comb_gbs,
                          "frac": comb_gbs / HBM_PEAK_GBS if comb_gbs else None,
                          "bytes_per_step": int(comb_bytes), "kernel_us_per_step": comb_us},
        "stages": stages,
        "keys_scanned_per_s": keys_per_step * 1e3 / ms_step,
        "host_submit_ms_per_step": 1e3 * host_s / args.steps,
        "encode": {"keys": enc_keys, "avg_ms": float(np.mean(enc_ms)),
                   "GBps": enc_keys * 400 / (np.mean(enc_ms) * 1e-3) / 1e9},
        "recall_at_k": rec,
        "planted_recall": planted,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
