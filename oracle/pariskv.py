"""Oracle (test infrastructure): a plain, slow CPU implementation of one ParisKV
decode step for one unit, i.e. one (batch, kv-head) sequence.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  It shares no code with the HIP library and imports nothing from
it.  Integer-valued results (bucket ids, 4-bit codes, votes, candidate and
selected sets) are decided in the same fp32 arithmetic the spec fixes for both
sides; float results (the scale w, RSQ-IP estimates, attention) are computed
in float64.

Source: the ParisKV page ("ParisKV: Fast and Drift-Robust KV-Cache Retrieval
for Long-Context LLMs").  Each function names the part of the page it follows.

Readings where the page is silent (every one is also listed in the design notes):
  * rotation = one SRHT round R = H D / sqrt(d) (Sylvester Hadamard H, Rademacher
    D), shared by keys, queries and all heads; no subsampling;
  * ids and codes are scale invariant, so the l2 normalisation is folded into
    w and into ||q||; both are evaluated on x = H D k in fp32 with the
    butterfly stages in ascending order;
  * subspace b = rotated coordinates [m b, m b + m); a centroid index c has
    coordinate j equal to -1/sqrt(m) when bit j of c is set, else +1/sqrt(m);
  * "hierarchical" vote weights = a weight per rank (default rho - r + 1);
    with grouped-query attention the votes of all query heads of a kv head are
    summed, and so are their RSQ-IP estimates;
  * coarse keeps C = min(N_r, max(k, ceil(p N_r / 1000))) retrieval-zone keys;
  * every tie goes to the lower centroid index / lower token position.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# rotation (page: "Drift-robust analytic centroids > Normalization and rotation")
# ---------------------------------------------------------------------------


def sylvester_hadamard(n: int) -> np.ndarray:
    """H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]] (float64)."""
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == n, "n must be a power of two"
    return H


def srht_matrix(signs: np.ndarray) -> np.ndarray:
    """The shared random orthogonal rotation R = H D / sqrt(d), float64."""
    d = signs.shape[0]
    return sylvester_hadamard(d) * signs.astype(np.float64)[None, :] / math.sqrt(d)


def fwht_spec(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of the last axis in fp32.

    Stages h = 1, 2, 4, ... in that order; at each stage every pair (j, j+h)
    with bit h of j clear becomes (x_j + x_{j+h}, x_j - x_{j+h}), one IEEE fp32
    add or subtract each.  The result equals H x up to rounding.
    """
    x = np.array(x, dtype=np.float32, copy=True)
    d = x.shape[-1]
    lead = x.shape[:-1]
    h = 1
    while h < d:
        y = x.reshape(lead + (d // (2 * h), 2, h))
        lo = y[..., 0, :].copy()
        hi = y[..., 1, :].copy()
        y[..., 0, :] = lo + hi
        y[..., 1, :] = lo - hi
        h *= 2
    return x


def rotate_spec(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """x -> H D x in fp32 spec arithmetic (= sqrt(d) R x up to rounding)."""
    return fwht_spec(np.asarray(x, dtype=np.float32) * signs.astype(np.float32))


# ---------------------------------------------------------------------------
# analytic centroids and bucket ids
# (page: "Analytic centroids"; "Coarse candidate generation (collision based)")
# ---------------------------------------------------------------------------


def centroid(c: int, m: int) -> np.ndarray:
    """Sign-pattern centroid number c on the unit sphere of R^m."""
    bits = (c >> np.arange(m)) & 1
    return np.where(bits == 1, -1.0, 1.0) / math.sqrt(m)


def bucket_ids(x: np.ndarray, n_sub: int, m: int) -> np.ndarray:
    """Nearest analytic centroid of every subspace direction of rotated keys x.

    The nearest sign-pattern centroid of a direction is its own sign pattern:
    bit j of the id is set when coordinate j is negative (a zero coordinate
    gives bit 0, the lower of the two tied centroids).  Returns uint8/uint16
    [n, n_sub].
    """
    xb = np.asarray(x, np.float32).reshape(-1, n_sub, m)
    bits = (xb < 0).astype(np.int64)
    ids = np.sum(bits << np.arange(m)[None, None, :], axis=-1)
    return ids.astype(np.uint8 if m <= 8 else np.uint16)


# ---------------------------------------------------------------------------
# 4-bit codes and the calibration scale
# (page: "Candidate reranking (RSQ-IP) > Quantization, Calibration")
# ---------------------------------------------------------------------------


def _tree8(t: np.ndarray) -> np.ndarray:
    """((t0+t1)+(t2+t3)) + ((t4+t5)+(t6+t7)) over the last axis, fp32."""
    t = np.asarray(t, np.float32)
    return ((t[..., 0] + t[..., 1]) + (t[..., 2] + t[..., 3])) + \
           ((t[..., 4] + t[..., 5]) + (t[..., 6] + t[..., 7]))


def _tree(t: np.ndarray) -> np.ndarray:
    """The spec's pairwise fp32 sum over the last axis, terms paired in index
    order at every level (m = 8: _tree8; m = 4: (t0+t1)+(t2+t3); m = 16: the
    m = 8 tree of t0..t7 plus the m = 8 tree of t8..t15)."""
    t = np.asarray(t, np.float32)
    m = t.shape[-1]
    if m == 8:
        return _tree8(t)
    if m == 16:
        return _tree8(t[..., :8]) + _tree8(t[..., 8:])
    assert m == 4, "spec trees exist for m = 4, 8 and 16"
    return (t[..., 0] + t[..., 1]) + (t[..., 2] + t[..., 3])


def quantize_codes(x: np.ndarray, sq_thresholds: np.ndarray, n_sub: int, m: int):
    """Sign + 3-bit magnitude code of every coordinate of every subspace direction.

    For u = x_b / ||x_b||, the magnitude code of u_j is the number of thresholds
    t_l with |u_j| >= t_l, evaluated without sqrt or division as
    x_j^2 >= fl(T_l * ss_b), where ss_b is the fp32 pairwise sum of the squares
    and T_l = fp32(t_l^2).  nibble = (sign << 3) | magnitude.  A subspace whose
    ss_b is zero gets all-zero nibbles.  Returns uint8 [n, n_sub, m] and the
    fp32 ss [n, n_sub].
    """
    assert m in (4, 8, 16), "spec trees exist for m = 4, 8 and 16"
    xb = np.asarray(x, np.float32).reshape(-1, n_sub, m)
    sq = xb * xb
    ss = _tree(sq)
    T = np.asarray(sq_thresholds, np.float32)
    mag = np.zeros(xb.shape, np.int64)
    for l in range(T.shape[0]):
        bound = (T[l] * ss).astype(np.float32)           # one fp32 product
        mag += (sq >= bound[..., None]).astype(np.int64)
    sign = (xb < 0).astype(np.int64)
    nib = (sign << 3) | mag
    nib[ss == 0] = 0
    return nib.astype(np.uint8), ss


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """[n, B, m] nibbles -> [n, B*m/2] bytes: coordinate 2i in the low half of byte i."""
    flat = nib.reshape(nib.shape[0], -1).astype(np.uint8)
    return (flat[:, 0::2] | (flat[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, n_sub: int, m: int) -> np.ndarray:
    p = np.asarray(packed, np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out.reshape(-1, n_sub, m)


def dequantize(nib: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Dequantised direction v: coordinate = (sign ? -1 : +1) * level[magnitude], float64."""
    lv = np.asarray(levels, np.float32).astype(np.float64)
    mag = nib & 7
    sgn = np.where((nib >> 3) & 1, -1.0, 1.0)
    return sgn * lv[mag]


def calibrate_w(x: np.ndarray, v: np.ndarray, ss32: np.ndarray, n_sub: int, m: int):
    """Calibration scale w_b = ||(R k)_b|| / <v_b, u_b> with u_b = x_b / ||x_b||.

    x is sqrt(d) R k, so ||(R k)_b|| = ||x_b|| / sqrt(d).  Then
    ||q|| * w_b <v_b, q~_b> is exact when v_b = u_b, and w absorbs both the
    key norm and the alignment loss of the quantised direction.  float64; the
    encoder passes the same fp32 rotated coordinates that define the codes.
    Zero where the fp32 ss_b is zero.
    """
    d = n_sub * m
    xb = np.asarray(x, np.float64).reshape(-1, n_sub, m)
    norm = np.sqrt(np.sum(xb * xb, axis=-1))
    ok = np.asarray(ss32) != 0
    w = np.zeros(norm.shape)
    u = np.zeros_like(xb)
    u[ok] = xb[ok] / norm[ok][:, None]
    align = np.sum(np.asarray(v, np.float64) * u, axis=-1)
    w[ok] = (norm[ok] / math.sqrt(d)) / align[ok]
    return w


def encode_keys(K: np.ndarray, signs: np.ndarray, levels: np.ndarray,
                sq_thresholds: np.ndarray, n_sub: int = 16, m: int = 8):
    """Per-key metadata: bucket ids [n, B], packed nibbles [n, B*m/2], w fp32 [n, B].

    (page: coarse candidate generation for the ids; quantization and
    calibration for nibbles and w, computed once when a key enters the
    retrieval zone.)
    """
    x = rotate_spec(K, signs)
    ids = bucket_ids(x, n_sub, m)
    nib, ss = quantize_codes(x, sq_thresholds, n_sub, m)
    w = calibrate_w(x.astype(np.float64), dequantize(nib, levels), ss, n_sub, m)
    return ids, pack_nibbles(nib), w.astype(np.float32)


# ---------------------------------------------------------------------------
# query side: top-rho centroids and the collision votes
# (page: "Coarse candidate generation (collision based)")
# ---------------------------------------------------------------------------


def centroid_scores(y_b: np.ndarray) -> np.ndarray:
    """fp32 similarity of a rotated query subspace y_b (m = 4, 8 or 16) to all 2^m centroids.

    Score(c) = pairwise fp32 sum of t_j, t_j = -y_j if bit j of c is set else
    y_j.  This is sqrt(m) times the inner product with centroid c; the dropped
    positive factors do not change the ranking.
    """
    y = np.asarray(y_b, np.float32)
    m = y.shape[0]
    bits = ((np.arange(1 << m)[:, None] >> np.arange(m)[None, :]) & 1).astype(bool)
    t = np.where(bits, -y[None, :], y[None, :]).astype(np.float32)
    return _tree(t)


def top_rho(scores: np.ndarray, rho: int) -> np.ndarray:
    """The rho best centroids: higher score first, lower index on ties."""
    order = np.lexsort((np.arange(scores.shape[0]), -scores.astype(np.float64)))
    return order[:rho]


def vote_table(Qg: np.ndarray, signs: np.ndarray, rho: int, weights, n_sub=16, m=8):
    """Vote table L[b][c] = sum over the query heads of the group of the weight of
    the rank centroid c holds among that head's top-rho in subspace b (0 when
    not selected).  Returns (L uint16 [B, 256], picks int [G, B, rho])."""
    Qg = np.atleast_2d(np.asarray(Qg, np.float32))
    y = rotate_spec(Qg, signs)
    G = Qg.shape[0]
    L = np.zeros((n_sub, 1 << m), np.int64)
    picks = np.zeros((G, n_sub, rho), np.int64)
    for g in range(G):
        for b in range(n_sub):
            top = top_rho(centroid_scores(y[g, b * m:(b + 1) * m]), rho)
            picks[g, b] = top
            for r, c in enumerate(top):
                L[b, c] += int(weights[r])
    return L.astype(np.uint16), picks


def coarse_scores(ids: np.ndarray, L: np.ndarray) -> np.ndarray:
    """Integer coarse score of each key: its votes summed over the subspaces."""
    ids = np.asarray(ids, np.int64)
    n_sub = ids.shape[1]
    return np.sum(L[np.arange(n_sub)[None, :], ids].astype(np.int64), axis=1)


def coarse_count(n_retrieval: int, permille: int, top_k: int) -> int:
    """C = min(N_r, max(k, ceil(p N_r / 1000))) (integer arithmetic)."""
    return min(n_retrieval, max(top_k, (permille * n_retrieval + 999) // 1000))


def top_by_key(values: np.ndarray, positions: np.ndarray, count: int) -> np.ndarray:
    """Positions of the `count` entries with the largest value, ties -> lower
    position, returned in ascending position order."""
    order = np.lexsort((positions, -np.asarray(values, np.float64)))
    return np.sort(positions[order[:count]])


# ---------------------------------------------------------------------------
# RSQ-IP rerank (page: "Candidate reranking (RSQ-IP) > Estimation")
# ---------------------------------------------------------------------------


def rsq_ip_directions(v: np.ndarray, w: np.ndarray, Qg: np.ndarray,
                      signs: np.ndarray) -> np.ndarray:
    """The RSQ-IP estimate from directions v [n, B, m] and scales w [n, B]:
    sum over the query heads of the group of  ||q||_2 * sum_b w_b <v_b, q~_b>,
    with q~ = R q / ||q|| the rotated, normalised query.  float64."""
    v = np.asarray(v, np.float64)
    n, n_sub, m = v.shape
    w = np.asarray(w, np.float64)
    R = srht_matrix(signs)
    est = np.zeros(n)
    for q in np.atleast_2d(np.asarray(Qg, np.float64)):
        qn = np.linalg.norm(q)
        if qn == 0.0:
            continue
        qt = (R @ q / qn).reshape(n_sub, m)
        est += qn * np.sum(w * np.einsum("nbj,bj->nb", v, qt), axis=1)
    return est


def rsq_ip(nib: np.ndarray, w: np.ndarray, Qg: np.ndarray, signs: np.ndarray,
           levels: np.ndarray, n_sub: int = 16, m: int = 8) -> np.ndarray:
    """RSQ-IP estimate of keys from their packed 4-bit codes and fp32 scales."""
    v = dequantize(unpack_nibbles(nib, n_sub, m), levels)
    return rsq_ip_directions(v, np.asarray(w, np.float32), Qg, signs)


# ---------------------------------------------------------------------------
# sparse attention (page: "Problem definition" - attend only to a top-k subset)
# ---------------------------------------------------------------------------


def sparse_attention(Qg: np.ndarray, K: np.ndarray, V: np.ndarray,
                     attended: np.ndarray) -> np.ndarray:
    """o_g = sum_{i in A} softmax_i(<q_g, k_i> / sqrt(d)) v_i, float64 [G, d]."""
    Qg = np.atleast_2d(np.asarray(Qg, np.float64))
    Ka = np.asarray(K, np.float64)[attended]
    Va = np.asarray(V, np.float64)[attended]
    s = Qg @ Ka.T / math.sqrt(Qg.shape[1])
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ Va


# ---------------------------------------------------------------------------
# zones (page: "System-level innovations > 2. Sliding-window update mechanism")
# ---------------------------------------------------------------------------


class Window:
    """Zone bounds of one unit: sink [0, sink_end), retrieval [sink_end, r_end),
    local [r_end, n - buf), update buffer [n - buf, n).

    After a prefill of n0 tokens the last n_local tokens are local and the
    buffer is empty.  Each decode token enters the buffer; after the step in
    which the buffer reaches U tokens, the oldest local tokens move to the
    retrieval zone (just enough that local + buffer fits in n_local) and the
    buffer becomes part of the local zone.
    """

    def __init__(self, n0: int, n_sink: int, n_local: int, buf_tokens: int):
        self.n_sink, self.n_local, self.U = n_sink, n_local, buf_tokens
        self.n = n0
        self.sink_end = min(n_sink, n0)
        self.r_end = max(self.sink_end, n0 - n_local)
        self.buf = 0

    def append(self) -> None:
        self.n += 1
        self.buf += 1

    def end_step(self):
        """Returns the [start, end) range of positions evicted into retrieval."""
        if self.U and self.buf >= self.U:
            local = self.n - self.buf - self.r_end
            move = max(0, local + self.buf - self.n_local)
            lo = self.r_end
            self.r_end += move
            self.buf = 0
            return lo, self.r_end
        return self.r_end, self.r_end

    def retrieval(self) -> np.ndarray:
        return np.arange(self.sink_end, self.r_end)

    def hot(self) -> np.ndarray:
        """Sink, local and buffer positions, attended every step."""
        return np.concatenate([np.arange(0, self.sink_end), np.arange(self.r_end, self.n)])


# ---------------------------------------------------------------------------
# one decode step of one unit
# ---------------------------------------------------------------------------


def decode_step(K, V, Qg, ids, nib, w, win: Window, signs, levels, *, rho=4,
                weights=(4, 3, 2, 1), permille=50, top_k=2048, n_sub=16, m=8):
    """Coarse-to-fine retrieval followed by sparse attention, for one unit.

    ids / nib / w are the per-key metadata of positions [0, n) (only the
    retrieval zone's are read).  Returns a dict with every intermediate.
    """
    L, picks = vote_table(Qg, signs, rho, weights, n_sub, m)
    pos = win.retrieval()
    scores = coarse_scores(ids[pos], L) if pos.size else np.zeros(0, np.int64)
    C = coarse_count(pos.size, permille, top_k)
    cand = top_by_key(scores, pos, C)
    est = rsq_ip(nib[cand], w[cand], Qg, signs, levels, n_sub, m) if C else np.zeros(0)
    k_eff = min(top_k, C)
    sel = top_by_key(est, cand, k_eff)
    attended = np.concatenate([win.hot(), sel])
    out = sparse_attention(Qg, K[:win.n], V[:win.n], attended)
    return dict(lut=L, picks=picks, scores=scores, n_cand=C, cand=cand, est=est,
                sel=sel, attended=attended, out=out)


def exact_topk(K, Qg, positions, k):
    """Reference for recall: the k positions with the largest sum over the group
    of <q_g, k_i> (float64), ties -> lower position."""
    s = np.asarray(K, np.float64)[positions] @ np.atleast_2d(np.asarray(Qg, np.float64)).sum(0)
    return top_by_key(s, positions, min(k, positions.size))


def recall(selected, reference) -> float:
    if len(reference) == 0:
        return 1.0
    return len(np.intersect1d(selected, reference)) / len(reference)
