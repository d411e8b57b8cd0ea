"""Pins for the comparison coarse stage with learned (k-means) centroids: brute
force, closed forms, invariants and a recovery case, each written as a check of
the oracle callable so that a planted mistake can be shown to fail it (the
mutation tests at the end)."""
import math

import numpy as np

from oracle import kmeans as km
from oracle import pariskv as pk

D = 128


def _signs(seed):
    r = np.random.default_rng(seed)
    return np.where(r.integers(0, 2, D) == 1, -1.0, 1.0).astype(np.float32)


def _unit_rows(r, n, m=8):
    v = r.standard_normal((n, m))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def analytic_table():
    """The 256 sign-pattern centroids of every subspace as a learned table (fp32)."""
    c = np.stack([pk.centroid(i, 8) for i in range(256)]).astype(np.float32)
    return np.broadcast_to(c, (16, 256, 8)).copy()


# ------------------------------------------------------------------- checks

def check_fixed_point(fixed_point):
    """Round to the nearest multiple of 2^-20, ties to even, exact multiples kept."""
    s = 2.0 ** -20
    x = np.array([0.5 * s, 1.5 * s, 2.5 * s, -0.5 * s, -1.5 * s, 3 * s, -7 * s, 1000.0], np.float32)
    want = np.array([0, 2, 2, 0, -2, 3, -7, 1000 << 20], np.int64)
    return np.array_equal(fixed_point(x), want)


def check_normalise(normalise):
    """Unit norm (to fp32 rounding); exact invariance to doubling the sum; a zero
    sum keeps the old centroid."""
    r = np.random.default_rng(3)
    S = r.integers(-2**40, 2**40, size=(500, 8), dtype=np.int64)
    c = normalise(S).astype(np.float64)
    if not np.all(np.abs(np.linalg.norm(c, axis=1) - 1.0) < 1e-6):
        return False
    if not np.array_equal(normalise(2 * S), normalise(S)):
        return False
    # direction agrees with the exact quotient
    ref = S / np.linalg.norm(S.astype(np.float64), axis=1, keepdims=True)
    if not np.all(np.abs(c - ref) < 1e-7):
        return False
    old = r.standard_normal((3, 8)).astype(np.float32)
    Z = np.zeros((3, 8), np.int64)
    return np.array_equal(normalise(Z, old=old), old)


def check_assign_brute_force(assign):
    """Against a float64 brute force over all 256 centroids, wherever the best
    beats the runner-up clearly; duplicated centroids go to the lower index."""
    r = np.random.default_rng(5)
    cents = _unit_rows(r, 16 * 256).reshape(16, 256, 8).astype(np.float32)
    cents[:, 200] = cents[:, 17]                         # duplicates: 17 must win
    x = r.standard_normal((400, D)).astype(np.float32)
    xb = x.reshape(-1, 16, 8).astype(np.float64)
    x[:50].reshape(-1, 16, 8)[:] = cents[:, 17][None] * 3.0   # exactly on centroid 17
    xb[:50] = cents[:, 17][None].astype(np.float64) * 3.0
    got = assign(cents, x)
    dots = np.einsum("nbj,bcj->nbc", xb, cents.astype(np.float64))
    srt = np.sort(dots, axis=2)
    clear = (srt[..., -1] - srt[..., -2]) > 1e-4 * np.linalg.norm(xb, axis=2)
    best = np.argmax(dots, axis=2)
    if not np.array_equal(got[clear], best[clear]):
        return False
    return bool(np.all(got[:50] == 17))


def check_assign_analytic(assign):
    """With the sign-pattern table the best centroid of a subspace vector is its
    own sign pattern (the ParisKV bucket id), wherever no coordinate is so small
    that it is lost in rounding."""
    r = np.random.default_rng(6)
    x = pk.rotate_spec(r.standard_normal((300, D)).astype(np.float32), _signs(6))
    got = assign(analytic_table(), x)
    want = pk.bucket_ids(x, 16, 8).astype(np.int64)
    xb = np.abs(x.reshape(-1, 16, 8))
    ok = np.min(xb, axis=2) > 1e-3 * np.max(xb, axis=2)
    return bool(ok.mean() > 0.5) and np.array_equal(got[ok], want[ok])


def check_fit_recovers_directions(fit):
    """Keys whose rotated subspace vectors are positive multiples of four fixed
    directions per subspace: every fitted centroid is a unit vector, and every
    key ends up with a centroid along its own direction."""
    r = np.random.default_rng(7)
    s = _signs(7)
    n = 1200
    dirs = _unit_rows(r, 16 * 4).reshape(16, 4, 8)
    lab = r.integers(0, 4, size=(n, 16))
    scale = r.uniform(0.5, 2.0, size=(n, 16, 1))
    x = (dirs[np.arange(16)[None, :], lab] * scale).reshape(n, D)
    H = pk.sylvester_hadamard(D).astype(np.float64)
    K = ((x @ H) * s.astype(np.float64) / D).astype(np.float32)     # H D k = x
    init = r.choice(n, size=256, replace=False)
    cents, ids = fit(K, s, init, 4)
    c64 = cents.astype(np.float64)
    if not np.all(np.abs(np.linalg.norm(c64, axis=2) - 1.0) < 1e-6):
        return False
    got = c64[np.arange(16)[None, :], ids]                           # [n, 16, 8]
    cos = np.einsum("nbj,nbj->nb", got, dirs[np.arange(16)[None, :], lab])
    return bool(np.all(cos > 0.999))


def check_fit_objective_monotone(fit):
    """Lloyd's iterations never lower the objective sum_i max_c <c, x_ib> (each
    step maximises it over one of its two arguments)."""
    r = np.random.default_rng(8)
    s = _signs(8)
    K = r.standard_normal((1500, D)).astype(np.float32)
    init = r.choice(1500, size=256, replace=False)
    xb = pk.rotate_spec(K, s).reshape(-1, 16, 8).astype(np.float64)
    prev = -np.inf
    for it in range(4):
        cents, _ = fit(K, s, init, it)
        obj = np.einsum("nbc->", np.max(np.einsum("nbj,bcj->nbc", xb, cents.astype(np.float64)),
                                        axis=2)[..., None])
        if obj < prev - 1e-6 * abs(prev):
            return False
        prev = obj
    return True


def check_learned_vote_table(vote_table):
    """Votes against a float64 brute force of the top-rho centroids of every
    head and subspace (random unit centroids), where the ranking is clear."""
    r = np.random.default_rng(9)
    s = _signs(9)
    cents = _unit_rows(r, 16 * 256).reshape(16, 256, 8).astype(np.float32)
    weights = (4, 3, 2, 1)
    for trial in range(4):
        Qg = r.standard_normal((4, D)).astype(np.float32)
        L = vote_table(Qg, s, cents, 4, weights).astype(np.int64)
        y = pk.rotate_spec(Qg, s).reshape(4, 16, 8).astype(np.float64)
        want = np.zeros((16, 256), np.int64)
        clear = True
        for g in range(4):
            for b in range(16):
                d = cents[b].astype(np.float64) @ y[g, b]
                order = np.argsort(-d, kind="stable")
                gaps = -np.diff(d[order[:5]])
                if np.min(gaps) < 1e-4 * np.linalg.norm(y[g, b]):
                    clear = False
                for k in range(4):
                    want[b, order[k]] += weights[k]
        if clear and not np.array_equal(L, want):
            return False
    return True


# -------------------------------------------------------------------- pins

def test_fixed_point():
    assert check_fixed_point(km.fixed_point)


def test_normalise():
    assert check_normalise(km.normalise)


def test_assign_brute_force():
    assert check_assign_brute_force(km.assign)


def test_assign_analytic_table_gives_parsikv_ids():
    assert check_assign_analytic(km.assign)


def test_fit_recovers_directions():
    assert check_fit_recovers_directions(km.fit)


def test_fit_objective_monotone():
    assert check_fit_objective_monotone(km.fit)


def test_learned_vote_table():
    assert check_learned_vote_table(km.vote_table)


def test_encode_ids_are_fit_ids():
    r = np.random.default_rng(10)
    s = _signs(10)
    K = r.standard_normal((700, D)).astype(np.float32)
    cents, ids = km.fit(K, s, r.choice(700, 256, replace=False), 2)
    assert np.array_equal(km.encode_ids(K, s, cents).astype(np.int64), ids)


# ---------------------------------------------------------------- mutations

def test_mutation_rounding_toward_zero_is_caught():
    bad = lambda x: np.trunc(np.asarray(x, np.float32).astype(np.float64) * 2.0**20).astype(np.int64)
    assert not check_fixed_point(bad)


def test_mutation_zero_sum_not_kept_is_caught():
    def bad(S, old=None):
        return km.normalise(S, old=None)
    assert not check_normalise(bad)


def test_mutation_ties_to_higher_index_is_caught():
    def bad(cents, x):
        xb = np.asarray(x, np.float32).reshape(-1, 16, 8)
        out = np.empty((xb.shape[0], 16), np.int64)
        for b in range(16):
            s = km.similarity(cents[b], xb[:, b])[:, ::-1]
            out[:, b] = 255 - np.argmax(s, axis=1)
        return out
    assert not check_assign_brute_force(bad)


def test_mutation_dropped_term_is_caught():
    def bad(cents, x):
        xb = np.asarray(x, np.float32).reshape(-1, 16, 8).copy()
        xb[..., 7] = 0.0                                     # one coordinate ignored
        return km.assign(cents, xb.reshape(-1, D))
    assert not check_assign_brute_force(bad)


def test_mutation_unnormalised_centroids_is_caught():
    def bad(K, signs, init_pos, iters):
        x = pk.rotate_spec(K, signs)
        F = km.fixed_point(x).reshape(-1, 16, 8)
        cents = np.transpose(F[np.asarray(init_pos)], (1, 0, 2)).astype(np.float32)
        for _ in range(iters):
            ids = km.assign(cents, x)
            S = np.zeros((16, 256, 8), np.int64)
            for b in range(16):
                np.add.at(S[b], ids[:, b], F[:, b])
            cents = np.where((S != 0).any(axis=2, keepdims=True), S.astype(np.float32), cents)
        return cents, km.assign(cents, x)
    assert not check_fit_recovers_directions(bad)


def test_mutation_negated_query_is_caught():
    def bad(Qg, signs, cents, rho, weights):
        return km.vote_table(-np.asarray(Qg, np.float32), signs, cents, rho, weights)
    assert not check_learned_vote_table(bad)
