"""GPU parity over seeded random small configurations.

Each case draws a context length, batch, query-group size, dtype, subspace
width, probe count and weights, top-k, coarse fraction, sink / local / update
buffer sizes from a fixed seed, then checks the static retrieval and attention
stage by stage against the oracle (same bars as tests/test_gpu_parity.py) and,
when the case has an update buffer, runs fused decode steps through two
evictions and checks the last step.  The point is combinations the hand-made
cases do not reach (zone sizes against chunk boundaries, thresholds against
the prefetched suffix-count range, odd top-k against the candidate count).
"""
import dataclasses

import numpy as np
import pytest
import torch

from synth import workloads as W
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import kv_cache_top_amd  # noqa: F401  (fails loudly when the library is missing)
    yield
    torch.cuda.synchronize()


def _draw_cases(n_cases=14, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        m = int(rng.choice([8, 8, 8, 4, 16]))
        group = int(rng.choice([1, 2, 4, 8]))
        rho = int(rng.integers(1, 9))
        w = np.sort(rng.integers(1, 9, size=rho))[::-1]
        # a vote-table byte holds G * max weight (twice that for m = 4)
        wmax_ok = 255 // (group * (2 if m == 4 else 1))
        w = np.minimum(w, wmax_ok)
        n_local = int(rng.choice([0, 64, 512]))
        buf = int(rng.choice([0, 16])) if n_local >= 16 else 0
        cases.append(dict(
            idx=i,
            N=int(rng.integers(300, 16001)),
            batch=int(rng.choice([1, 2])),
            group=group,
            dtype="f32" if rng.random() < 0.2 else "bf16",
            m=m,
            rho=rho,
            weights=tuple(int(x) for x in w),
            top_k=int(rng.choice([16, 100, 512, 1024, 2048, 3000])),
            permille=int(rng.choice([10, 50, 100, 300, 1000])),
            n_sink=int(rng.choice([0, 4, 16])),
            n_local=n_local,
            buf=buf,
        ))
    return cases


CASES = _draw_cases()


def _tag(c):
    return (f"r{c['idx']}-N{c['N']}-b{c['batch']}-g{c['group']}-{c['dtype']}-m{c['m']}-rho{c['rho']}"
            f"-k{c['top_k']}-p{c['permille']}-s{c['n_sink']}-l{c['n_local']}-u{c['buf']}")


@pytest.mark.parametrize("case", CASES, ids=[_tag(c) for c in CASES])
def test_random_config(case):
    c = case
    wl = W.gqa_bf16(N=c["N"], batch=c["batch"], seed=100 + c["idx"], top_k=c["top_k"],
                    permille=c["permille"], n_sink=c["n_sink"], n_local=c["n_local"],
                    buf_tokens=c["buf"], group=c["group"], dtype=c["dtype"])
    wl.params = dataclasses.replace(wl.params, n_sub=128 // c["m"], sub_dim=c["m"], rho=c["rho"],
                                    vote_weights=c["weights"])
    units = sorted({0, wl.n_units - 1})
    steps = 2 * c["buf"] + 3 if c["buf"] else 0
    gc.log(f"[random {_tag(c)}] units {units}, {steps} decode steps")
    pkv = gc.make_ctx(wl, capacity=wl.n_tokens + steps)
    pkv.encode_keys(wl.n_tokens)
    q = gc.queries(wl)
    sel, sel_n = pkv.retrieve(q)
    out = pkv.sparse_attend(q, sel, sel_n)
    torch.cuda.synchronize()
    enc = gc.check_encode(wl, pkv, units)
    gc.check_retrieval(wl, pkv, units, sel, sel_n, enc)
    gc.check_attention(wl, pkv, units, sel, sel_n, out)
    if not steps:
        return
    dt = gc.torch_dtype(wl)
    Kn, Vn, Qn = W.decode_stream(wl, steps)
    for t in range(steps):
        out, sel, sel_n = pkv.decode_step(torch.from_numpy(Kn[t]).to(dt).cuda(),
                                          torch.from_numpy(Vn[t]).to(dt).cuda(),
                                          torch.from_numpy(Qn[t]).to(dt).cuda())
    torch.cuda.synchronize()
    n = pkv.window()[0]
    assert n == wl.n_tokens + steps
    full = W.Workload(wl.name, wl.batch, wl.n_kv, wl.group, n, wl.dtype, wl.params, wl.sign_bits,
                      np.concatenate([wl.K, np.moveaxis(Kn, 0, 2)], axis=2),
                      np.concatenate([wl.V, np.moveaxis(Vn, 0, 2)], axis=2), Qn[-1])
    enc = gc.check_encode(full, pkv, units)
    gc.check_retrieval(full, pkv, units, sel, sel_n, enc)
    gc.check_attention(full, pkv, units, sel, sel_n, out)
