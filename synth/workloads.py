"""Seeded synthetic decode workloads for the ParisKV retrieval path.

This module only draws random inputs (keys, values, queries, the SRHT sign
diagonal); it holds none of the method's arithmetic.  Both the CPU oracle
(through the tests) and the HIP library (through the tests and the bench) are
fed from here.

Every random stream is a numpy PCG64 generator seeded with
``SeedSequence(entropy=seed, spawn_key=(layer, unit, stream_id))`` so that the
draws do not depend on thread count or on which units are materialised.  A
*unit* is one (batch, kv-head) sequence.

Shapes follow an 8B-class GQA decoder layer (32 query heads, 8 KV heads,
head dim 128), the attention shape of the models the ParisKV page evaluates
(ParisKV page, "Experimental results").  Values stand in for real activations:
per-channel lognormal scales, a few outlier channels, and (for the recall
workload) a planted relevant set.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # bf16 rounding (round-to-nearest-even) is done with torch on the CPU
    import torch
except ImportError:  # pragma: no cover - torch is part of the image
    torch = None

# stream ids inside one unit
_S_SCALE, _S_KEYS, _S_VALS, _S_QUERY, _S_PLANT, _S_DECODE = range(6)
_S_SIGNS = 99


@dataclasses.dataclass
class Params:
    """Method parameters of one workload (ParisKV page: analytic centroids,
    coarse candidate generation, RSQ-IP reranking, sliding window)."""
    head_dim: int = 128
    n_sub: int = 16          # B
    sub_dim: int = 8         # m
    rho: int = 4
    vote_weights: tuple = (4, 3, 2, 1)
    coarse_permille: int = 50
    top_k: int = 2048
    n_sink: int = 4
    n_local: int = 512
    buf_tokens: int = 0      # U (update buffer); 0 = static context
    codebook: str = "lloyd_max"   # magnitude codebook reading: "lloyd_max" or "quantile"


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    n_kv: int
    group: int               # G = query heads per kv head
    n_tokens: int            # prefill length N0
    dtype: str               # "f32" or "bf16"
    params: Params
    sign_bits: np.ndarray    # uint64[2]; bit j set -> D_jj = -1
    K: np.ndarray            # float32 [batch, n_kv, N0, d] (bf16-representable when dtype == bf16)
    V: np.ndarray
    Q: np.ndarray            # float32 [batch, n_kv*group, d]
    planted: np.ndarray | None = None   # int64 [batch, n_kv, n_plant] positions
    planted_dir: np.ndarray | None = None  # float64 [batch, n_kv, d] unit directions
    seed: int = 0
    layer: int = 0

    @property
    def n_units(self) -> int:
        return self.batch * self.n_kv

    def signs(self) -> np.ndarray:
        """The +-1 diagonal as float32 [d] (a view of ``sign_bits``)."""
        d = self.params.head_dim
        bits = np.array([(int(self.sign_bits[j // 64]) >> (j % 64)) & 1 for j in range(d)])
        return np.where(bits == 1, -1.0, 1.0).astype(np.float32)


def _rng(seed: int, layer: int, unit: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=seed, spawn_key=(layer, unit, stream))))


def sign_bits(seed: int, layer: int = 0) -> np.ndarray:
    """128 Rademacher signs packed in two uint64 words (shared by all heads)."""
    return _rng(seed, layer, 0, _S_SIGNS).integers(0, 2**64, size=2, dtype=np.uint64)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even), returned as float32."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _channel_scales(r: np.random.Generator, d: int, n_outlier: int) -> np.ndarray:
    s = r.lognormal(0.0, 0.5, size=d).astype(np.float32)
    if n_outlier:
        ch = r.choice(d, size=n_outlier, replace=False)
        s[ch] *= np.float32(20.0)
    return s


def _unit_draw(seed, layer, unit, N, d, n_outlier, group, gqa_values_std_normal):
    """Keys, values and the query group of one unit."""
    rs = _rng(seed, layer, unit, _S_SCALE)
    s_k = _channel_scales(rs, d, n_outlier)
    if gqa_values_std_normal:
        s_v = np.ones(d, np.float32)
    else:
        s_v = rs.lognormal(0.0, 0.5, size=d).astype(np.float32)
    K = _rng(seed, layer, unit, _S_KEYS).standard_normal((N, d), dtype=np.float32) * s_k
    V = _rng(seed, layer, unit, _S_VALS).standard_normal((N, d), dtype=np.float32) * s_v
    Q = _rng(seed, layer, unit, _S_QUERY).standard_normal((group, d), dtype=np.float32) * s_k
    return s_k, K, V, Q


def _build(name, batch, n_kv, group, N, dtype, params, seed, layer, n_outlier,
           gqa_values_std_normal, n_plant=0, plant_cos=0.3, threads=8):
    d = params.head_dim
    units = batch * n_kv
    K = np.empty((batch, n_kv, N, d), np.float32)
    V = np.empty((batch, n_kv, N, d), np.float32)
    Q = np.empty((batch, n_kv * group, d), np.float32)
    planted = np.empty((batch, n_kv, n_plant), np.int64) if n_plant else None
    pdir = np.empty((batch, n_kv, d), np.float64) if n_plant else None

    def one(u):
        b, h = divmod(u, n_kv)
        _, k, v, q = _unit_draw(seed, layer, u, N, d, n_outlier, group, gqa_values_std_normal)
        if n_plant:
            # a known-relevant set: n_plant retrieval-zone keys turned towards a
            # shared random direction, and queries that are noisy copies of it
            rp = _rng(seed, layer, u, _S_PLANT)
            lo, hi = params.n_sink, N - params.n_local
            pos = np.sort(rp.choice(np.arange(lo, hi), size=n_plant, replace=False))
            uhat = rp.standard_normal(d)
            uhat /= np.linalg.norm(uhat)
            k64 = k.astype(np.float64)
            for p in pos:
                k64[p] = np.linalg.norm(k64[p]) * uhat
            k = k64.astype(np.float32)
            q64 = q.astype(np.float64)
            for g in range(group):
                e = rp.standard_normal(d)
                e -= (e @ uhat) * uhat
                e /= np.linalg.norm(e)
                q64[g] = np.linalg.norm(q64[g]) * (plant_cos * uhat + math.sqrt(1 - plant_cos**2) * e)
            q = q64.astype(np.float32)
            planted[b, h] = pos
            pdir[b, h] = uhat
        if dtype == "bf16":
            k, v, q = round_bf16(k), round_bf16(v), round_bf16(q)
        K[b, h] = k
        V[b, h] = v
        Q[b, h * group:(h + 1) * group] = q

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(units)))
    return Workload(name, batch, n_kv, group, N, dtype, params, sign_bits(seed, layer),
                    K, V, Q, planted, pdir, seed, layer)


# ---------------------------------------------------------------------------
# the five workloads (sizes can be shrunk for the oracle-sized parity cases)
# ---------------------------------------------------------------------------

def single_head_f32(N=4096, seed=0, layer=0, top_k=128, threads=8) -> Workload:
    """One KV head, fp32, i.i.d. N(0,1) keys/values with per-channel lognormal(0, 0.5)
    scales, one query; B=16, m=8, rho=4, keep 10%, top-k 128, sink 4 + local 64."""
    p = Params(coarse_permille=100, top_k=top_k, n_sink=4, n_local=64)
    return _build("single_head_4k_f32", 1, 1, 1, N, "f32", p, seed, layer,
                  n_outlier=0, gqa_values_std_normal=False, threads=threads)


def gqa_bf16(N=32768, batch=1, seed=0, layer=0, top_k=2048, permille=50,
             n_sink=4, n_local=512, buf_tokens=0, n_plant=0, threads=8,
             name=None, group=4, dtype="bf16") -> Workload:
    """8B-class GQA layer: 8 KV heads, 4 query heads each (`group`), bf16 (or
    `dtype` "f32"); keys with 4 outlier channels (x20) on top of lognormal
    channel scales, values N(0,1), queries drawn like the keys of their head
    (or planted noisy copies)."""
    p = Params(coarse_permille=permille, top_k=top_k, n_sink=n_sink, n_local=n_local,
               buf_tokens=buf_tokens)
    nm = name or f"gqa_{N // 1024}k_b{batch}_{dtype}" + ("" if group == 4 else f"_g{group}")
    return _build(nm, batch, 8, group, N, dtype, p, seed, layer, n_outlier=4,
                  gqa_values_std_normal=True, n_plant=n_plant, threads=threads)


def gqa_128k_planted(N=131072, batch=4, seed=0, layer=0, threads=8) -> Workload:
    """The 128K-context recall workload: batch 4 x 8 KV heads, 64 planted keys per
    unit, queries at cosine 0.3 to the planted direction; keep 5%, top-k 2048."""
    return gqa_bf16(N=N, batch=batch, seed=seed, layer=layer, n_plant=64, threads=threads,
                    name=f"gqa_{N // 1024}k_b{batch}_planted_bf16")


def decode_stream(w: Workload, n_steps: int, drift_sigma: float = 2.0, seed: int = 0,
                  layer: int = 0):
    """Per-step keys, values and queries for a decode run whose key mean drifts
    linearly to ``drift_sigma`` standard deviations along a random direction.

    Returns float32 arrays K_new [T, batch, n_kv, d], V_new [T, batch, n_kv, d],
    Q_new [T, batch, n_kv*G, d] (bf16-representable when the workload is bf16).
    """
    d = w.params.head_dim
    T = n_steps
    Kn = np.empty((T, w.batch, w.n_kv, d), np.float32)
    Vn = np.empty_like(Kn)
    Qn = np.empty((T, w.batch, w.n_kv * w.group, d), np.float32)
    for u in range(w.n_units):
        b, h = divmod(u, w.n_kv)
        s_k = _channel_scales(_rng(seed, layer, u, _S_SCALE), d, 4 if w.dtype == "bf16" else 0)
        r = _rng(seed, layer, u, _S_DECODE)
        rhat = r.standard_normal(d)
        rhat /= np.linalg.norm(rhat)
        sigma_r = math.sqrt(float(np.sum(rhat**2 * s_k.astype(np.float64)**2)))
        frac = (np.arange(T, dtype=np.float64) + 1.0) / T
        mu = (drift_sigma * frac * sigma_r)[:, None] * rhat[None, :]
        k = r.standard_normal((T, d)) * s_k + mu
        q = r.standard_normal((T, w.group, d)) * s_k + mu[:, None, :]
        v = r.standard_normal((T, d))
        if w.dtype == "bf16":
            k, v, q = round_bf16(k), round_bf16(v), round_bf16(q)
        Kn[:, b, h] = k
        Vn[:, b, h] = v
        Qn[:, b, h * w.group:(h + 1) * w.group] = q
    return Kn, Vn, Qn


def kmeans_init_positions(n_units: int, n_tokens: int, seed: int = 0, layer: int = 0,
                          k: int = 256) -> np.ndarray:
    """k distinct token positions in [0, n_tokens) per unit, uniformly drawn: the
    initial centroids of the learned-centroid comparator.  int32 [n_units, k]."""
    out = np.empty((n_units, k), np.int32)
    for u in range(n_units):
        r = _rng(seed, layer, u, 2000)
        out[u] = np.sort(r.choice(n_tokens, size=k, replace=False))
    return out


def fill_gqa_device(K, V, n_tokens: int, seed: int = 0, layer: int = 0, pool: int = 8):
    """The gqa_bf16 recipe drawn on the GPU, for contexts whose host-side draw would
    take minutes (capacity sweeps).  K, V: device tensors [batch, n_kv, cap, d]
    (bf16 or fp32) whose first n_tokens rows are filled: keys s * z with the unit's
    channel scales s (drawn exactly as gqa_bf16 draws them: lognormal(0, 0.5), 4
    outlier channels x20), values z, z ~ N(0, 1) from torch's generator on the
    device seeded per (seed, layer, unit).  Returns host float32 pools of `pool`
    query sets [pool, batch, n_kv*4, d] drawn like the keys, and of `pool` new
    tokens' keys and values [pool, batch, n_kv, d] (rounded to K's dtype)."""
    batch, n_kv, _, d = K.shape
    group = 4
    qp = np.empty((pool, batch, n_kv * group, d), np.float32)
    kp = np.empty((pool, batch, n_kv, d), np.float32)
    vp = np.empty((pool, batch, n_kv, d), np.float32)
    g = torch.Generator(device=K.device)
    for u in range(batch * n_kv):
        b, h = divmod(u, n_kv)
        s_k = _channel_scales(_rng(seed, layer, u, _S_SCALE), d, 4)
        g.manual_seed(int(np.random.SeedSequence(entropy=seed, spawn_key=(layer, u, 7)).generate_state(1)[0]))
        st = torch.from_numpy(s_k).to(K.device)
        for lo in range(0, n_tokens, 1 << 18):
            hi = min(n_tokens, lo + (1 << 18))
            z = torch.randn((hi - lo, d), generator=g, device=K.device)
            K[b, h, lo:hi].copy_(z * st)
            V[b, h, lo:hi].copy_(torch.randn((hi - lo, d), generator=g, device=K.device))
        r = _rng(seed, layer, u, 1000 + _S_QUERY)
        qp[:, b, h * group:(h + 1) * group] = r.standard_normal((pool, group, d)) * s_k
        kp[:, b, h] = r.standard_normal((pool, d)) * s_k
        vp[:, b, h] = r.standard_normal((pool, d))
    if K.dtype == torch.bfloat16:
        qp, kp, vp = round_bf16(qp), round_bf16(kp), round_bf16(vp)
    return qp, kp, vp


def query_pool(w: Workload, n: int, plant_cos: float = 0.3) -> np.ndarray:
    """n further query sets drawn with the workload's recipe (new draws, same
    channel scales; planted workloads: new noisy copies of the planted
    direction).  float32 [n, batch, n_kv*G, d]."""
    d = w.params.head_dim
    out = np.empty((n, w.batch, w.n_kv * w.group, d), np.float32)
    for u in range(w.n_units):
        b, h = divmod(u, w.n_kv)
        s_k = _channel_scales(_rng(w.seed, w.layer, u, _S_SCALE), d, 4 if w.dtype == "bf16" else 0)
        r = _rng(w.seed, w.layer, u, 1000 + _S_QUERY)
        q = r.standard_normal((n, w.group, d)) * s_k
        if w.planted_dir is not None:
            uhat = w.planted_dir[b, h]
            for i in range(n):
                for g in range(w.group):
                    e = r.standard_normal(d)
                    e -= (e @ uhat) * uhat
                    e /= np.linalg.norm(e)
                    q[i, g] = np.linalg.norm(q[i, g]) * (plant_cos * uhat +
                                                         math.sqrt(1 - plant_cos**2) * e)
        if w.dtype == "bf16":
            q = round_bf16(q)
        out[:, b, h * w.group:(h + 1) * w.group] = q
    return out
