"""Helpers for the GPU parity tests: run the HIP path through the C ABI on a
synthetic workload and compare every stage with the oracle (per unit)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import pariskv as ok
from oracle.codebook import spec_tables

LEVELS, SQ_T = spec_tables()


def tables(wl):
    """(levels, squared thresholds) of the workload's codebook reading and subspace width."""
    return spec_tables(m=wl.params.sub_dim, kind=getattr(wl.params, "codebook", "lloyd_max"))


def sub_shape(wl):
    return wl.params.n_sub, wl.params.sub_dim


def pack_ids(ids: np.ndarray, m: int) -> np.ndarray:
    """The library's 16 id bytes per key: one id per byte for m = 8; for m = 4
    subspace 2i in the low half of byte i and 2i + 1 in the high half; for
    m = 16 the 16-bit id of subspace b little-endian at bytes 2b, 2b + 1."""
    if m == 16:
        ids = np.ascontiguousarray(np.asarray(ids, np.uint16).astype("<u2"))
        return ids.view(np.uint8).reshape(ids.shape[0], 16)
    ids = np.asarray(ids, np.uint8)
    if m == 8:
        return ids
    return (ids[:, 0::2] | (ids[:, 1::2] << 4)).astype(np.uint8)


def _hash16(c: int) -> int:
    return ((c * 40503) & 0xFFFF) >> 8


def check_hashed_votes(table_bytes: np.ndarray, L: np.ndarray, u: int) -> None:
    """m = 16: the 8 hash tables of a unit hold exactly the oracle's nonzero
    votes (entry = vote << 16 | centroid, 0 = empty), each centroid once, and
    each entry is reachable by linear probing from its home slot (no empty slot
    on the way), so the scan's probe finds it."""
    tab = np.ascontiguousarray(table_bytes).view(np.uint32).reshape(8, 256)
    for b in range(8):
        got = {}
        for slot in np.flatnonzero(tab[b]):
            e = int(tab[b, slot])
            c, vote = e & 0xFFFF, e >> 16
            assert c not in got, f"unit {u}, subspace {b}: centroid {c} twice"
            got[c] = vote
            h = _hash16(c)
            k = h
            while k != slot:
                assert tab[b, k] != 0, f"unit {u}, subspace {b}: {c} unreachable from slot {h}"
                k = (k + 1) & 255
        want = {int(c): int(L[b, c]) for c in np.flatnonzero(L[b])}
        assert got == want, f"unit {u}, subspace {b}: votes {got} != {want}"


def byte_vote_table(L: np.ndarray, m: int) -> np.ndarray:
    """The table the scan reads, [16][256]: the vote table itself for m = 8;
    for m = 4, entry c of row i = L[2i][c & 15] + L[2i + 1][c >> 4]."""
    L = np.asarray(L, np.int64)
    if m == 8:
        return L
    c = np.arange(256)
    return L[0::2][:, c & 15] + L[1::2][:, c >> 4]

# acceptance bars
W_RTOL = 1e-6          # calibration scale (fp32 on both sides; derivation in the design notes)
EST_RTOL = 1e-4        # RSQ-IP estimate, relative to the sum of the absolute terms
ATT_TOL = {"bf16": 2e-2, "f32": 1e-5}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def make_ctx(wl, capacity=None, host_mapped=False, **override):
    from kv_cache_top_amd import ParisKV
    p = wl.params
    kw = dict(rho=p.rho, vote_weights=p.vote_weights, coarse_permille=p.coarse_permille,
              top_k=p.top_k, n_sink=p.n_sink, n_local=p.n_local, buf_tokens=p.buf_tokens,
              sign_bits=tuple(int(x) for x in wl.sign_bits),
              codebook=0 if p.codebook == "lloyd_max" else 1, n_sub=p.n_sub, sub_dim=p.sub_dim)
    kw.update(override)
    cap = capacity or wl.n_tokens
    dt = torch_dtype(wl)
    pkv = ParisKV(batch=wl.batch, n_kv=wl.n_kv, n_q=wl.n_kv * wl.group, capacity=cap, dtype=dt,
                  host_mapped=host_mapped, **kw)
    N = wl.n_tokens
    pkv.K[:, :, :N].copy_(torch.from_numpy(wl.K).to(dt))
    pkv.V[:, :, :N].copy_(torch.from_numpy(wl.V).to(dt))
    return pkv


def queries(wl, Q=None):
    Q = wl.Q if Q is None else Q
    return torch.from_numpy(np.ascontiguousarray(Q)).to(torch_dtype(wl)).cuda()


def unit_view(wl, u):
    b, h = divmod(u, wl.n_kv)
    return wl.K[b, h], wl.V[b, h], wl.Q[b, h * wl.group:(h + 1) * wl.group]


def est_scale(nib, w, Qg, signs, levels=LEVELS, n_sub=16, m=8):
    """sum_g sum_b |w_b <v_b, (R q_g)_b>|: the magnitude the estimate error is measured against."""
    v = ok.dequantize(ok.unpack_nibbles(nib, n_sub, m), levels)
    R = ok.srht_matrix(signs)
    w = np.asarray(w, np.float64)
    s = np.zeros(v.shape[0])
    for q in np.atleast_2d(np.asarray(Qg, np.float64)):
        y = (R @ q).reshape(n_sub, m)
        s += np.sum(np.abs(w * np.einsum("nbj,bj->nb", v, y)), axis=1)
    return s


class UnitReport:
    def __init__(self):
        self.lines = []

    def add(self, s):
        self.lines.append(s)


def check_encode(wl, pkv, units, ids_all=None, rec_all=None, ids_fn=None):
    """ids and nibbles bit-exact, w within W_RTOL, for the retrieval zone of `units`.
    ids_fn(u, keys) gives the expected ids when they are not the analytic ones
    (the learned-centroid comparison stage)."""
    n, sink_end, r_end, _ = pkv.window()
    ids_all = pkv.debug(0) if ids_all is None else ids_all
    rec_all = pkv.debug(1) if rec_all is None else rec_all
    s = wl.signs()
    n_sub, m = sub_shape(wl)
    out = {}
    for u in units:
        K, _, _ = unit_view(wl, u)
        pos = np.arange(sink_end, r_end)
        i_o, n_o, w_o = ok.encode_keys(K[pos], s, *tables(wl), n_sub=n_sub, m=m)
        if ids_fn is not None:
            i_o = ids_fn(u, K[pos])
        ids_g = ids_all[u].reshape(-1, 16)[pos]
        rec_g = rec_all[u].reshape(-1, 64 + 4 * n_sub)[pos]
        nib_g = rec_g[:, :64]
        w_g = rec_g[:, 64:].copy().view(np.float32)
        i_p = pack_ids(i_o, m)
        assert np.array_equal(ids_g, i_p), f"unit {u}: bucket ids differ at {np.argwhere(ids_g != i_p)[:5]}"
        assert np.array_equal(nib_g, n_o), f"unit {u}: nibbles differ at {np.argwhere(nib_g != n_o)[:5]}"
        rel = np.abs(w_g.astype(np.float64) - w_o) / np.maximum(np.abs(w_o), 1e-30)
        assert np.all(rel <= W_RTOL), f"unit {u}: w rel err {rel.max():.3g}"
        out[u] = (i_o, n_o, w_o)
    return out


def check_retrieval(wl, pkv, units, sel, sel_n, enc, vote_fn=None):
    """LUT, scores, candidates bit-exact; estimates within EST_RTOL; fine sets by the tie rule.
    vote_fn(u, Qg) gives the expected vote table when it is not the analytic one.
    Returns per-unit oracle results."""
    n, sink_end, r_end, _ = pkv.window()
    lut = pkv.debug(2)
    scores = pkv.debug(3)
    cand = pkv.debug(4)
    est = pkv.debug(5)
    meta = pkv.debug(6)
    sel = sel.cpu().numpy().reshape(wl.n_units, -1)
    sel_n = sel_n.cpu().numpy().reshape(-1)
    s = wl.signs()
    p = wl.params
    n_sub, m = sub_shape(wl)
    res = {}
    for u in units:
        K, V, Qg = unit_view(wl, u)
        i_o, n_o, w_o = enc[u]
        pos = np.arange(sink_end, r_end)
        N_r = pos.size
        L = (ok.vote_table(Qg, s, p.rho, p.vote_weights, n_sub, m)[0] if vote_fn is None
             else vote_fn(u, Qg))
        if m == 16:
            check_hashed_votes(lut[u], L, u)
        else:
            assert np.array_equal(lut[u].reshape(16, 256).astype(np.int64), byte_vote_table(L, m)), \
                f"unit {u}: vote table differs"
        sc_o = ok.coarse_scores(i_o, L) if N_r else np.zeros(0, np.int64)
        # scores are stored saturated at 255 (the threshold logic rescores saturated keys)
        assert np.array_equal(scores[u][:N_r].astype(np.int64), np.minimum(sc_o, 255)), \
            f"unit {u}: coarse scores differ"
        C = ok.coarse_count(N_r, p.coarse_permille, p.top_k)
        assert meta[u][2] == C, f"unit {u}: C {meta[u][2]} != {C}"
        cand_o = ok.top_by_key(sc_o, pos, C)
        assert np.array_equal(cand[u][:C], cand_o), f"unit {u}: coarse candidate set differs"
        rel = cand_o - sink_end
        e_o = ok.rsq_ip(n_o[rel], w_o[rel], Qg, s, tables(wl)[0], n_sub, m) if C else np.zeros(0)
        scale = (est_scale(n_o[rel], w_o[rel], Qg, s, tables(wl)[0], n_sub, m) if C
                 else np.zeros(0))
        err = np.abs(est[u][:C].astype(np.float64) - e_o)
        assert np.all(err <= EST_RTOL * np.maximum(scale, 1e-30)), \
            f"unit {u}: est rel err {np.max(err / np.maximum(scale, 1e-30)):.3g}"
        k_eff = min(p.top_k, C)
        assert sel_n[u] == k_eff, f"unit {u}: sel_n {sel_n[u]} != {k_eff}"
        sel_g = sel[u][:k_eff]
        assert np.all(np.diff(sel_g) > 0), f"unit {u}: sel not strictly ascending"
        sel_o = ok.top_by_key(e_o, cand_o, k_eff)
        diff = np.setxor1d(sel_g, sel_o)
        if diff.size:
            kth = np.sort(e_o)[::-1][k_eff - 1]
            idx = np.searchsorted(cand_o, diff)
            assert np.all(np.isin(diff, cand_o)), f"unit {u}: selected a non-candidate"
            near = np.abs(e_o[idx] - kth) <= EST_RTOL * np.maximum(scale[idx], 1e-30)
            assert np.all(near), f"unit {u}: fine sets differ beyond ties: {diff[~near][:5]}"
        res[u] = dict(sel_o=sel_o, sel_g=sel_g, cand=cand_o, est=e_o, n_diff=int(diff.size))
    return res


def check_attention(wl, pkv, units, sel, sel_n, out, tol=None):
    """GPU output vs the oracle's attention over hot + the GPU's own selection."""
    n, sink_end, r_end, _ = pkv.window()
    sel = sel.cpu().numpy().reshape(wl.n_units, -1)
    sel_n = sel_n.cpu().numpy().reshape(-1)
    out = out.cpu().numpy().reshape(wl.n_units, wl.group, 128)
    tol = ATT_TOL[wl.dtype] if tol is None else tol
    worst = 0.0
    for u in units:
        K, V, Qg = unit_view(wl, u)
        hot = np.concatenate([np.arange(0, sink_end), np.arange(r_end, n)])
        A = np.concatenate([hot, sel[u][:sel_n[u]]])
        ref = ok.sparse_attention(Qg, K[:n], V[:n], A)
        e = float(np.max(np.abs(out[u] - ref)))
        worst = max(worst, e)
        assert e <= tol, f"unit {u}: attention max-abs err {e:.3g} > {tol}"
    return worst


def recall_report(wl, pkv, units, sel, sel_n):
    n, sink_end, r_end, _ = pkv.window()
    sel = sel.cpu().numpy().reshape(wl.n_units, -1)
    sel_n = sel_n.cpu().numpy().reshape(-1)
    rec, planted = [], []
    for u in units:
        K, _, Qg = unit_view(wl, u)
        pos = np.arange(sink_end, r_end)
        ref = ok.exact_topk(K, Qg, pos, wl.params.top_k)
        rec.append(ok.recall(sel[u][:sel_n[u]], ref))
        if wl.planted is not None:
            b, h = divmod(u, wl.n_kv)
            pl = wl.planted[b, h]
            planted.append(np.isin(pl, sel[u][:sel_n[u]]).mean())
    return float(np.mean(rec)), (float(np.mean(planted)) if planted else None)
