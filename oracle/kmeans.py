"""Oracle (test infrastructure) for the comparison coarse stage: centroids learned
from the prefill keys by k-means, in place of ParisKV's analytic sign-pattern
centroids.

The ParisKV page ("Problem definition"; "Drift-robust analytic centroids")
contrasts its data-independent centroids with centroids fitted to the keys
seen at prefill, whose buckets stop matching the keys once the key
distribution drifts during decoding.  The page does not define that fitting;
this module fixes one plain reading so that the GPU comparator can be checked
bit for bit:

  * data: the rotated keys x = H D k (the same fp32 rotation as the ParisKV
    path) of every stored token of the unit at fitting time, split into the
    same 16 subspaces of 8 coordinates;
  * similarity of centroid c and a subspace vector x_b: the fp32 pairwise tree
    ((t0+t1)+(t2+t3))+((t4+t5)+(t6+t7)) of t_j = fl32(c_j x_j); a key's bucket
    is the most similar of the 256 centroids, ties to the lower index;
  * initial centroids: the normalised subspace vectors of 256 given key
    positions per unit (a seeded sample drawn outside the method);
  * Lloyd iterations: assign every key, then centroid c = S_c / ||S_c|| where
    S_c is the exact sum of the assigned keys' subspace vectors in fixed point
    (every coordinate rounded to a multiple of 2^-20, summed as integers, so
    the order of the sum does not matter); the norm and the quotient in
    float64, the result rounded to fp32; a centroid whose sum is zero keeps
    its previous value;
  * queries: centroid scores with the same fp32 tree on the rotated query,
    top-rho by (score desc, index asc), votes exactly as on the ParisKV path.

The similarity is the cosine up to the positive factor ||x_b||, so this is
spherical k-means with each key weighted by its subspace norm.  Only the
tests, the smoke check and the bench's CPU baseline may import this package.
"""
from __future__ import annotations

import numpy as np

from oracle.pariskv import rotate_spec, top_rho

N_SUB, M, N_CENT = 16, 8, 256
FIX_BITS = 20


def fixed_point(x: np.ndarray) -> np.ndarray:
    """fp32 coordinates to int64 multiples of 2^-20, rounded to nearest (ties
    to even).  Exact for |x| < 2^43."""
    return np.rint(np.asarray(x, np.float32).astype(np.float64) * float(1 << FIX_BITS)).astype(np.int64)


def similarity(cents_b: np.ndarray, x_b: np.ndarray) -> np.ndarray:
    """fp32 similarity of subspace vectors x_b [n, 8] to centroids cents_b
    [256, 8]: the pairwise tree of the fp32 products.  Returns [n, 256]."""
    t = (np.asarray(x_b, np.float32)[:, None, :] * np.asarray(cents_b, np.float32)[None, :, :])
    t = t.astype(np.float32)
    return ((t[..., 0] + t[..., 1]) + (t[..., 2] + t[..., 3])) + \
           ((t[..., 4] + t[..., 5]) + (t[..., 6] + t[..., 7]))


def assign(cents: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Bucket of every subspace of rotated keys x [n, 128] under centroids
    cents [16, 256, 8]: the most similar centroid, the lower index on ties
    (argmax returns the first maximum).  Returns int64 [n, 16]."""
    xb = np.asarray(x, np.float32).reshape(-1, N_SUB, M)
    out = np.empty((xb.shape[0], N_SUB), np.int64)
    for b in range(N_SUB):
        out[:, b] = np.argmax(similarity(cents[b], xb[:, b]), axis=1)
    return out


def normalise(S: np.ndarray, old: np.ndarray | None = None) -> np.ndarray:
    """Centroids from integer sums S [..., 8]: S / ||S|| in float64 with the
    squares summed in coordinate order, rounded to fp32; where S is all zero
    the centroid is `old` (zero when none is given)."""
    S = np.asarray(S, np.int64)
    s = S.astype(np.float64)
    ss = np.zeros(S.shape[:-1], np.float64)
    for j in range(M):
        ss = ss + s[..., j] * s[..., j]
    nz = ss > 0
    nrm = np.sqrt(np.where(nz, ss, 1.0))
    c = (s / nrm[..., None]).astype(np.float32)
    base = np.zeros(S.shape, np.float32) if old is None else np.asarray(old, np.float32)
    return np.where(nz[..., None], c, base)


def fit(K: np.ndarray, signs: np.ndarray, init_pos: np.ndarray, iters: int):
    """k-means centroids of one unit from its keys K [n, 128] (fp32 values).
    Returns (cents fp32 [16, 256, 8], ids of the keys under them int64 [n, 16])."""
    x = rotate_spec(K, signs)
    F = fixed_point(x).reshape(-1, N_SUB, M)
    init = np.asarray(init_pos, np.int64)
    assert init.shape == (N_CENT,)
    cents = normalise(np.transpose(F[init], (1, 0, 2)))          # [16, 256, 8]
    for _ in range(iters):
        ids = assign(cents, x)
        S = np.zeros((N_SUB, N_CENT, M), np.int64)
        for b in range(N_SUB):
            np.add.at(S[b], ids[:, b], F[:, b])
        cents = normalise(S, old=cents)
    return cents, assign(cents, x)


def encode_ids(K: np.ndarray, signs: np.ndarray, cents: np.ndarray) -> np.ndarray:
    """Bucket ids (uint8 [n, 16]) of keys under fixed learned centroids (the
    comparator's ids for keys stored after fitting, e.g. evicted decode keys)."""
    return assign(cents, rotate_spec(K, signs)).astype(np.uint8)


def vote_table(Qg: np.ndarray, signs: np.ndarray, cents: np.ndarray, rho: int, weights):
    """Vote table [16, 256] of the query heads Qg [G, 128] under learned centroids:
    per head and subspace the top-rho centroids by similarity to the rotated
    query, each adding the weight of its rank."""
    Qg = np.atleast_2d(np.asarray(Qg, np.float32))
    y = rotate_spec(Qg, signs).reshape(-1, N_SUB, M)
    L = np.zeros((N_SUB, N_CENT), np.int64)
    for g in range(Qg.shape[0]):
        for b in range(N_SUB):
            s = similarity(cents[b], y[g, b][None, :])[0]
            for r, c in enumerate(top_rho(s, rho)):
                L[b, c] += int(weights[r])
    return L.astype(np.uint16)
