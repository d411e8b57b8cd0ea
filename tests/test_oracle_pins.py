"""Pins for the CPU oracle: closed forms, invariants, brute force and library
routines that fix what the oracle must compute, independently of the oracle's
own code.  Each check is a function of the oracle callable it checks, so
test_oracle_mutations.py can show that a planted mistake fails it.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import pariskv as pk
from oracle.codebook import spec_tables

D = 128
LEVELS, SQ_T = spec_tables()


def _signs(seed):
    r = np.random.default_rng(seed)
    return np.where(r.integers(0, 2, D) == 1, -1.0, 1.0).astype(np.float32)


# --------------------------------------------------------------------- rotation

def check_fwht_exact_on_integers(fwht):
    """On small integers every butterfly is exact in fp32, so the spec transform
    must equal the Hadamard product computed by scipy exactly."""
    r = np.random.default_rng(1)
    x = r.integers(-1000, 1000, size=(64, D)).astype(np.float32)
    H = scipy.linalg.hadamard(D).astype(np.float64)
    ref = x.astype(np.float64) @ H.T
    return np.array_equal(fwht(x).astype(np.float64), ref)


def test_sylvester_is_scipy_hadamard():
    for n in (1, 2, 8, 128):
        assert np.array_equal(pk.sylvester_hadamard(n), scipy.linalg.hadamard(n))


def test_fwht_exact_on_integers():
    assert check_fwht_exact_on_integers(pk.fwht_spec)


def test_fwht_close_to_dense_on_reals():
    r = np.random.default_rng(2)
    x = (r.standard_normal((256, D)) * r.lognormal(0, 0.5, D)).astype(np.float32)
    ref = x.astype(np.float64) @ scipy.linalg.hadamard(D).T
    bound = 7 * 2.0**-24 * np.abs(x.astype(np.float64)).sum(1, keepdims=True) * 2
    assert np.all(np.abs(pk.fwht_spec(x) - ref) <= bound)


def test_srht_orthogonal_and_norm_preserving():
    s = _signs(3)
    R = pk.srht_matrix(s)
    assert np.allclose(R @ R.T, np.eye(D), atol=1e-13)
    x = np.random.default_rng(4).standard_normal((32, D))
    assert np.allclose(np.linalg.norm(x @ R.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # the spec transform of D x is sqrt(d) R x
    y = pk.rotate_spec(x.astype(np.float32), s).astype(np.float64) / math.sqrt(D)
    assert np.allclose(y, x.astype(np.float32).astype(np.float64) @ R.T, atol=1e-5)


# ------------------------------------------------------------------ bucket ids

def check_bucket_ids_brute_force(bucket_ids):
    """Nearest analytic centroid by brute force over all 2^m sign patterns
    (largest inner product, lowest index on ties), with exact zeros present."""
    r = np.random.default_rng(5)
    x = r.standard_normal((40, D)).astype(np.float32)
    x[r.random(x.shape) < 0.1] = 0.0
    x[r.random(x.shape) < 0.05] = -0.0
    ids = bucket_ids(x, 16, 8)
    C = np.stack([pk.centroid(c, 8) for c in range(256)])        # [256, 8]
    for i in range(x.shape[0]):
        for b in range(16):
            dots = C @ x[i, 8 * b:8 * b + 8].astype(np.float64)
            best = max(range(256), key=lambda c: (dots[c], -c))
            if ids[i, b] != best:
                return False
    return True


def test_bucket_ids_brute_force():
    assert check_bucket_ids_brute_force(pk.bucket_ids)


def test_centroids_on_unit_sphere():
    for c in (0, 1, 77, 255):
        assert abs(np.linalg.norm(pk.centroid(c, 8)) - 1.0) < 1e-15


# ---------------------------------------------------------------- top-rho, LUT

def check_top_rho_brute_force(centroid_scores, top_rho):
    """On integer queries the fp32 tree is exact, so the spec scores equal the
    exact scaled inner products; ties are frequent and must go to the lower index."""
    r = np.random.default_rng(6)
    C = np.stack([pk.centroid(c, 8) for c in range(256)]) * math.sqrt(8)
    for _ in range(200):
        y = r.integers(-3, 4, size=8).astype(np.float32)
        sc = centroid_scores(y)
        if not np.array_equal(sc.astype(np.float64), C @ y.astype(np.float64)):
            return False
        ref = sorted(range(256), key=lambda c: (-float(C[c] @ y), c))[:4]
        if list(top_rho(sc, 4)) != ref:
            return False
    return True


def test_top_rho_brute_force():
    assert check_top_rho_brute_force(pk.centroid_scores, pk.top_rho)


def test_top_rho_structure_on_reals():
    """Rank 1 is the query's own sign pattern; rank 2 flips its smallest |y_j|."""
    r = np.random.default_rng(7)
    for _ in range(300):
        y = r.standard_normal(8).astype(np.float32)
        top = pk.top_rho(pk.centroid_scores(y), 4)
        own = int(np.sum((y < 0).astype(int) << np.arange(8)))
        assert top[0] == own
        assert top[1] == own ^ (1 << int(np.argmin(np.abs(y))))


def check_vote_table(vote_table):
    """Vote table by an explicit loop over (head, subspace, rank)."""
    r = np.random.default_rng(8)
    s = _signs(9)
    Qg = r.standard_normal((4, D)).astype(np.float32)
    w = (4, 3, 2, 1)
    L, picks = vote_table(Qg, s, 4, w)
    y = (Qg.astype(np.float64) * s) @ scipy.linalg.hadamard(D).T
    C = np.stack([pk.centroid(c, 8) for c in range(256)])
    ref = np.zeros((16, 256), np.int64)
    for g in range(4):
        for b in range(16):
            dots = C @ y[g, 8 * b:8 * b + 8]
            order = sorted(range(256), key=lambda c: (-dots[c], c))[:4]
            for rank, c in enumerate(order):
                ref[b, c] += w[rank]
    return np.array_equal(L.astype(np.int64), ref) and np.all(ref.sum(1) == 4 * sum(w))


def test_vote_table():
    assert check_vote_table(pk.vote_table)


def check_coarse_scores(coarse_scores):
    r = np.random.default_rng(10)
    ids = r.integers(0, 256, size=(500, 16)).astype(np.uint8)
    L = r.integers(0, 17, size=(16, 256)).astype(np.uint16)
    got = coarse_scores(ids, L)
    ref = [sum(int(L[b, ids[i, b]]) for b in range(16)) for i in range(500)]
    return list(got) == ref


def test_coarse_scores():
    assert check_coarse_scores(pk.coarse_scores)


def test_coarse_count():
    assert pk.coarse_count(4028, 100, 128) == 403
    assert pk.coarse_count(32252, 50, 2048) == 2048      # ceil(5%) = 1613 < k
    assert pk.coarse_count(130556, 50, 2048) == 6528
    assert pk.coarse_count(100, 50, 2048) == 100
    assert pk.coarse_count(0, 50, 2048) == 0
    assert pk.coarse_count(1000, 50, 10) == 50
    assert pk.coarse_count(1001, 50, 10) == 51           # ceiling


def check_top_by_key(top_by_key):
    r = np.random.default_rng(11)
    vals = r.integers(0, 6, size=300)                     # many ties
    pos = np.arange(1000, 1300)
    got = top_by_key(vals, pos, 37)
    ref = sorted(sorted(zip(vals, pos), key=lambda t: (-t[0], t[1]))[:37], key=lambda t: t[1])
    return list(got) == [p for _, p in ref]


def test_top_by_key():
    assert check_top_by_key(pk.top_by_key)


# ------------------------------------------------------------ codes, w, RSQ-IP

def test_codes_agree_with_real_number_rule():
    """The fp32 squared-threshold rule puts |u_j| in the Lloyd-Max bin given by
    the float64 thresholds, except within a few ulps of a threshold."""
    from oracle.codebook import lloyd_max
    _, t = lloyd_max()
    r = np.random.default_rng(12)
    x = pk.rotate_spec(r.standard_normal((4000, D)).astype(np.float32), _signs(13))
    nib, ss = pk.quantize_codes(x, SQ_T, 16, 8)
    xb = x.astype(np.float64).reshape(-1, 16, 8)
    u = np.abs(xb) / np.linalg.norm(xb, axis=-1, keepdims=True)
    mag_ref = np.searchsorted(t, u, side="right")
    mism = (nib & 7) != mag_ref
    near = np.min(np.abs(u[..., None] - t[None, None, None, :]), axis=-1) < 1e-6
    assert np.all(~mism | near)
    assert np.array_equal((nib >> 3) & 1, (xb < 0).astype(np.uint8))


def test_nibble_packing_roundtrip():
    r = np.random.default_rng(14)
    nib = r.integers(0, 16, size=(50, 16, 8)).astype(np.uint8)
    assert np.array_equal(pk.unpack_nibbles(pk.pack_nibbles(nib), 16, 8), nib)
    packed = pk.pack_nibbles(nib)
    assert packed[3, 0] == nib[3, 0, 0] | (nib[3, 0, 1] << 4)


def check_rsq_ip_identity(calibrate_w, rsq_ip_directions):
    """With identity quantisation (v = u) the estimator is the exact inner
    product sum_g <k, q_g> (float64)."""
    r = np.random.default_rng(15)
    s = _signs(16)
    R = pk.srht_matrix(s)
    K = r.standard_normal((64, D)) * r.lognormal(0, 0.5, D)
    Qg = r.standard_normal((4, D))
    x = K @ R.T * math.sqrt(D)                      # exact sqrt(d) R k
    xb = x.reshape(-1, 16, 8)
    u = xb / np.linalg.norm(xb, axis=-1, keepdims=True)
    w = calibrate_w(x, u, np.ones((64, 16)), 16, 8)
    est = rsq_ip_directions(u, w, Qg, s)
    ref = K @ Qg.sum(0)
    return np.allclose(est, ref, rtol=1e-12, atol=1e-12 * np.abs(K).sum())


def test_rsq_ip_identity_quantisation():
    assert check_rsq_ip_identity(pk.calibrate_w, pk.rsq_ip_directions)


def check_rsq_ip_parallel_query(calibrate_w, rsq_ip_directions, n_sub=16, m=8):
    """Real 4-bit codes, queries parallel to the key's own subspace directions.

    For a key with rotated subspaces x_b (x = sqrt(d) R k), u_b = x_b / ||x_b||
    and v_b its dequantised code, take the query whose rotated subspaces are
    alpha_b u_b (q = R^T y).  Then <k, q> = sum_b alpha_b ||x_b|| / sqrt(d), and
    the estimator gives sum_b w_b alpha_b <v_b, u_b>: with the calibration of
    the page ("Candidate reranking (RSQ-IP)", Calibration), w_b = ||(R k)_b|| /
    <v_b, u_b>, the two agree exactly although v_b != u_b.  Any other use of the
    alignment <v_b, u_b> (multiplying by it, or a least-squares scale
    <v_b, u_b> / ||v_b||^2) misses by the codes' alignment loss (~0.3 % per
    subspace), far outside the 1e-12 bar."""
    levels, sq_t = spec_tables(m=m)
    r = np.random.default_rng(31 + m)
    s = _signs(32 + m)
    R = pk.srht_matrix(s)
    n = 48
    K = r.standard_normal((n, D)) * r.lognormal(0, 0.5, D)
    x = K @ R.T * math.sqrt(D)                      # exact sqrt(d) R k (float64)
    nib, ss = pk.quantize_codes(x.astype(np.float32), sq_t, n_sub, m)
    v = pk.dequantize(nib, levels)
    assert np.all(ss != 0)
    xb = x.reshape(n, n_sub, m)
    u = xb / np.linalg.norm(xb, axis=-1, keepdims=True)
    assert np.min(np.abs(np.sum(v * u, axis=-1) - 1.0)) > 1e-6   # the codes are not exact
    w = calibrate_w(x, v, ss, n_sub, m)
    ok = True
    for i in range(n):
        alpha = r.uniform(-2.0, 2.0, n_sub)
        y = (alpha[:, None] * u[i]).reshape(D)
        q = R.T @ y                                  # rotated query = y
        est = rsq_ip_directions(v[i:i + 1], w[i:i + 1], q[None, :], s)[0]
        ref = float(K[i] @ q)
        ok &= abs(est - ref) <= 1e-12 * float(np.abs(K[i]) @ np.abs(q))
    return ok


@pytest.mark.parametrize("m", [8, 4, 16])
def test_rsq_ip_exact_for_parallel_queries(m):
    assert check_rsq_ip_parallel_query(pk.calibrate_w, pk.rsq_ip_directions, D // m, m)


def test_rsq_ip_estimates_inner_products():
    """With the 4-bit codes the estimate tracks <k, q> closely (the per-coordinate
    Lloyd-Max error is under 1e-3); a statistical sanity bound, not a pin."""
    r = np.random.default_rng(17)
    s = _signs(18)
    K = (r.standard_normal((2000, D)) * r.lognormal(0, 0.5, D)).astype(np.float32)
    q = r.standard_normal((1, D)).astype(np.float32)
    ids, nib, w = pk.encode_keys(K, s, LEVELS, SQ_T)
    est = pk.rsq_ip(nib, w, q, s, LEVELS)
    ref = K.astype(np.float64) @ q[0].astype(np.float64)
    err = np.abs(est - ref) / (np.linalg.norm(K, axis=1) * np.linalg.norm(q))
    assert np.mean(err) < 0.02 and np.corrcoef(est, ref)[0, 1] > 0.99


def test_zero_subspace_gives_zero_codes_and_w():
    s = _signs(19)
    K = np.zeros((2, D), np.float32)
    ids, nib, w = pk.encode_keys(K, s, LEVELS, SQ_T)
    assert not ids.any() and not nib.any() and not w.any()


# ------------------------------------------------------------------ attention

def _sdpa(Qg, K, V):
    q = torch.from_numpy(np.asarray(Qg, np.float64))[None, :, None, :]
    k = torch.from_numpy(np.asarray(K, np.float64))[None, None].expand(1, q.shape[1], -1, -1)
    v = torch.from_numpy(np.asarray(V, np.float64))[None, None].expand(1, q.shape[1], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(q, k, v)[0, :, 0].numpy()


def check_attention_full(sparse_attention):
    r = np.random.default_rng(20)
    K = r.standard_normal((300, D))
    V = r.standard_normal((300, D))
    Qg = r.standard_normal((4, D))
    got = sparse_attention(Qg, K, V, np.arange(300))
    return np.allclose(got, _sdpa(Qg, K, V), atol=1e-12)


def test_attention_all_keys_is_sdpa():
    assert check_attention_full(pk.sparse_attention)


def test_attention_single_key_returns_its_value():
    r = np.random.default_rng(21)
    K, V = r.standard_normal((10, D)), r.standard_normal((10, D))
    out = pk.sparse_attention(r.standard_normal((2, D)), K, V, np.array([7]))
    assert np.allclose(out, V[7][None, :].repeat(2, 0), atol=1e-15)


def test_decode_step_with_k_at_least_retrieval_is_full_attention():
    """k >= N_r with the whole retrieval zone kept reproduces full attention."""
    from synth.workloads import gqa_bf16
    wl = gqa_bf16(N=1024, top_k=4096, permille=1000, n_local=64)
    s = wl.signs()
    for h in (0, 5):
        K, V = wl.K[0, h], wl.V[0, h]
        Qg = wl.Q[0, 4 * h:4 * h + 4]
        ids, nib, w = pk.encode_keys(K, s, LEVELS, SQ_T)
        win = pk.Window(1024, 4, 64, 0)
        res = pk.decode_step(K, V, Qg, ids, nib, w, win, s, LEVELS, permille=1000, top_k=4096)
        assert np.array_equal(np.sort(res["attended"]), np.arange(1024))
        assert np.allclose(res["out"], _sdpa(Qg, K, V), atol=1e-12)


@pytest.mark.parametrize("m", [4, 16])
def test_decode_step_other_widths_keep_all_is_full_attention(m):
    """The whole oracle step at m = 4 and m = 16 (their codebooks, vote tables,
    scores and estimates) with every retrieval-zone key kept reproduces full
    attention, and the candidate set is the whole zone."""
    from oracle.codebook import spec_tables
    from synth.workloads import gqa_bf16
    wl = gqa_bf16(N=700, top_k=4096, permille=1000, n_local=64)
    s = wl.signs()
    lv, sq = spec_tables(m=m)
    K, V, Qg = wl.K[0, 2], wl.V[0, 2], wl.Q[0, 8:12]
    ids, nib, w = pk.encode_keys(K, s, lv, sq, n_sub=128 // m, m=m)
    res = pk.decode_step(K, V, Qg, ids, nib, w, pk.Window(700, 4, 64, 0), s, lv, permille=1000,
                         top_k=4096, n_sub=128 // m, m=m)
    assert np.array_equal(res["cand"], np.arange(4, 700 - 64))
    assert np.allclose(res["out"], _sdpa(Qg, K, V), atol=1e-12)


# ---------------------------------------------------------------------- window

def test_window_partitions_sequence():
    for n0, sink, local, U, steps in [(5000, 4, 512, 256, 2000), (600, 4, 512, 256, 900),
                                       (3, 4, 64, 16, 200), (1000, 4, 64, 0, 50)]:
        win = pk.Window(n0, sink, local, U)
        r_end_prev = win.r_end
        for t in range(steps):
            win.append()
            zones = [np.arange(0, win.sink_end), win.retrieval(),
                     np.arange(win.r_end, win.n - win.buf), np.arange(win.n - win.buf, win.n)]
            allpos = np.concatenate(zones)
            assert np.array_equal(allpos, np.arange(win.n))
            assert win.n - win.buf - win.r_end <= local
            lo, hi = win.end_step()
            assert lo == r_end_prev and hi == win.r_end
            r_end_prev = win.r_end
        if U and n0 >= sink + local:
            assert win.r_end == max(min(sink, n0), n0 - local) + U * (steps // U)


def test_recall_definition():
    assert pk.recall(np.array([1, 2, 3]), np.array([2, 3, 4, 5])) == 0.5


# ------------------------------------------------------ subspaces of m = 4

def check_m4_ids_and_top_rho(bucket_ids, centroid_scores, top_rho):
    """m = 4 (32 subspaces of 4 coordinates, 16 sign-pattern centroids each):
    ids by brute force over the 16 centroids (exact zeros present), and on
    integer queries the spec scores equal the exact scaled inner products with
    top-rho ties to the lower index."""
    r = np.random.default_rng(11)
    x = r.standard_normal((30, D)).astype(np.float32)
    x[r.random(x.shape) < 0.1] = 0.0
    ids = bucket_ids(x, 32, 4)
    C = np.stack([pk.centroid(c, 4) for c in range(16)])
    for i in range(x.shape[0]):
        for b in range(32):
            dots = C @ x[i, 4 * b:4 * b + 4].astype(np.float64)
            if ids[i, b] != max(range(16), key=lambda c: (dots[c], -c)):
                return False
    C2 = C * 2.0
    for _ in range(200):
        y = r.integers(-3, 4, size=4).astype(np.float32)
        sc = centroid_scores(y)
        if sc.shape != (16,) or not np.array_equal(sc.astype(np.float64), C2 @ y.astype(np.float64)):
            return False
        if list(top_rho(sc, 4)) != sorted(range(16), key=lambda c: (-float(C2[c] @ y), c))[:4]:
            return False
    return True


def test_m4_ids_and_top_rho():
    assert check_m4_ids_and_top_rho(pk.bucket_ids, pk.centroid_scores, pk.top_rho)


def test_m4_codes_follow_the_real_number_rule():
    """m = 4 codes with the m = 4 codebook: the fp32 rule agrees with the
    real-number bin rule |u_j| >= t_l away from the thresholds."""
    from oracle.codebook import lloyd_max
    _, t = lloyd_max(4)
    T32 = (t * t).astype(np.float32)
    r = np.random.default_rng(12)
    x = r.standard_normal((500, D)).astype(np.float32)
    nib, ss = pk.quantize_codes(x, T32, 32, 4)
    xb = x.reshape(-1, 32, 4).astype(np.float64)
    u = np.abs(xb) / np.linalg.norm(xb, axis=2, keepdims=True)
    mag = np.sum(u[..., None] >= t[None, None, None, :], axis=-1)
    far = np.min(np.abs(u[..., None] - t), axis=-1) > 1e-6
    assert np.array_equal((nib & 7)[far], mag[far])
    assert np.array_equal((nib >> 3) & 1, (xb < 0).astype(np.uint8))


def test_m4_rsq_ip_identity():
    """With identity quantisation (v = u) the m = 4 estimate is the exact
    summed inner product."""
    r = np.random.default_rng(13)
    s = _signs(13)
    K = r.standard_normal((50, D))
    Qg = r.standard_normal((4, D))
    x = pk.srht_matrix(s) @ K.T * math.sqrt(D)
    xb = x.T.reshape(-1, 32, 4)
    u = xb / np.linalg.norm(xb, axis=2, keepdims=True)
    w = pk.calibrate_w(x.T, u, np.ones((50, 32)), 32, 4)
    est = pk.rsq_ip_directions(u, w, Qg, s)
    assert np.allclose(est, K @ Qg.sum(0), rtol=1e-12, atol=1e-10)


def test_mutation_m4_tree_dropping_a_term_is_caught():
    def bad(y_b):
        y = np.asarray(y_b, np.float32).copy()
        y[3] = 0.0
        return pk.centroid_scores(y)
    assert not check_m4_ids_and_top_rho(pk.bucket_ids, bad, pk.top_rho)


# ------------------------------------------------------ subspaces of m = 16

def check_m16_ids_and_top_rho(bucket_ids, centroid_scores, top_rho):
    """m = 16 (8 subspaces of 16 coordinates, 65536 sign-pattern centroids each):
    ids by brute force over all 65536 centroids (exact zeros present), 16-bit;
    on integer queries the spec scores equal the exact scaled inner products
    (4 <c, y>), top-rho ties go to the lower index, rank 1 is the query's own
    sign pattern and rank 2 flips its smallest coordinate."""
    r = np.random.default_rng(21)
    x = r.standard_normal((5, D)).astype(np.float32)
    x[r.random(x.shape) < 0.1] = 0.0
    ids = bucket_ids(x, 8, 16)
    if ids.dtype != np.uint16 or ids.shape != (5, 8):
        return False
    C = np.stack([pk.centroid(c, 16) for c in range(1 << 16)])
    for i in range(x.shape[0]):
        for b in range(8):
            dots = C @ x[i, 16 * b:16 * b + 16].astype(np.float64)
            best = np.flatnonzero(dots == dots.max())[0]      # lowest index among the maxima
            if ids[i, b] != best:
                return False
    C4 = C * 4.0
    for t in range(12):
        y = r.integers(-3, 4, size=16).astype(np.float32)
        if t % 3 == 0:
            y = (r.permutation(16) + 1) * r.choice([-1, 1], 16)   # distinct magnitudes
            y = y.astype(np.float32)
        sc = centroid_scores(y)
        exact = C4 @ y.astype(np.float64)
        if sc.shape != (1 << 16,) or not np.array_equal(sc.astype(np.float64), exact):
            return False
        want = np.lexsort((np.arange(1 << 16), -exact))[:6]
        if list(top_rho(sc, 6)) != list(want):
            return False
        if t % 3 == 0:
            own = int(np.sum((y < 0).astype(np.int64) << np.arange(16)))
            small = int(np.argmin(np.abs(y)))
            if list(top_rho(sc, 2)) != [own, own ^ (1 << small)]:
                return False
    return True


def test_m16_ids_and_top_rho():
    assert check_m16_ids_and_top_rho(pk.bucket_ids, pk.centroid_scores, pk.top_rho)


def test_m16_codes_follow_the_real_number_rule():
    """m = 16 codes with the m = 16 codebook: the fp32 rule agrees with the
    real-number bin rule |u_j| >= t_l away from the thresholds."""
    from oracle.codebook import lloyd_max
    _, t = lloyd_max(16)
    T32 = (t * t).astype(np.float32)
    r = np.random.default_rng(22)
    x = r.standard_normal((500, D)).astype(np.float32)
    nib, ss = pk.quantize_codes(x, T32, 8, 16)
    xb = x.reshape(-1, 8, 16).astype(np.float64)
    assert np.allclose(ss, np.sum(xb * xb, axis=2), rtol=1e-6)
    u = np.abs(xb) / np.linalg.norm(xb, axis=2, keepdims=True)
    mag = np.sum(u[..., None] >= t[None, None, None, :], axis=-1)
    far = np.min(np.abs(u[..., None] - t), axis=-1) > 1e-6
    assert np.array_equal((nib & 7)[far], mag[far])
    assert np.array_equal((nib >> 3) & 1, (xb < 0).astype(np.uint8))


def test_m16_rsq_ip_identity():
    """With identity quantisation (v = u) the m = 16 estimate is the exact
    summed inner product."""
    r = np.random.default_rng(23)
    s = _signs(23)
    K = r.standard_normal((50, D))
    Qg = r.standard_normal((4, D))
    x = pk.srht_matrix(s) @ K.T * math.sqrt(D)
    xb = x.T.reshape(-1, 8, 16)
    u = xb / np.linalg.norm(xb, axis=2, keepdims=True)
    w = pk.calibrate_w(x.T, u, np.ones((50, 8)), 8, 16)
    est = pk.rsq_ip_directions(u, w, Qg, s)
    assert np.allclose(est, K @ Qg.sum(0), rtol=1e-12, atol=1e-10)


def test_m16_vote_table_follows_the_flip_structure():
    """m = 16 vote table: in real arithmetic a centroid's score is sum |y_j|
    minus twice the |y_j| of the coordinates where it differs from the query's
    own sign pattern, so a head's top 3 are its sign pattern, then the flips of
    its smallest and of its second-smallest coordinate (random normal queries:
    no near ties for fp32 rounding to reorder); weighted by rank and summed
    over the heads."""
    r = np.random.default_rng(24)
    s = _signs(24)
    Qg = r.standard_normal((2, D)).astype(np.float32)
    L, picks = pk.vote_table(Qg, s, 3, (3, 2, 1), n_sub=8, m=16)
    y = pk.srht_matrix(s) @ Qg.astype(np.float64).T * math.sqrt(D)
    want = np.zeros((8, 1 << 16), np.int64)
    for g in range(2):
        for b in range(8):
            yb = y[16 * b:16 * b + 16, g]
            # best flip sets of the own sign pattern: smallest sums of |y_j|
            a = np.abs(yb)
            own = int(np.sum((yb < 0).astype(np.int64) << np.arange(16)))
            order = np.argsort(a)
            sets = [(), (order[0],), (order[1],), (order[0], order[1]), (order[2],)]
            sets.sort(key=lambda f: sum(a[list(f)]))
            for rank, f in enumerate(sets[:3]):
                c = own
                for j in f:
                    c ^= 1 << int(j)
                want[b, c] += (3, 2, 1)[rank]
    assert np.array_equal(L.astype(np.int64), want)


def test_mutation_m16_tree_dropping_a_term_is_caught():
    def bad(y_b):
        y = np.asarray(y_b, np.float32).copy()
        y[11] = 0.0
        return pk.centroid_scores(y)
    assert not check_m16_ids_and_top_rho(pk.bucket_ids, bad, pk.top_rho)


@pytest.mark.parametrize("m", [4, 8, 16])
def test_zero_query_subspace_picks_lowest_centroids(m):
    """A rotated query subspace that is exactly zero ties all 2^m centroids, so
    each head picks centroids 0..rho-1 there and the vote table holds G times
    the rank weights on them (and nothing else in that subspace)."""
    r = np.random.default_rng(31)
    s = _signs(31)
    Y = r.integers(-2, 3, size=(3, D)).astype(np.float64)
    Y[:, 0:m] = 0.0                                        # subspace 0 of every head
    Qg = (Y @ scipy.linalg.hadamard(D).T) * s / D          # rotates back to exactly Y
    assert np.array_equal(pk.rotate_spec(Qg.astype(np.float32), s), Y.astype(np.float32))
    w = (5, 3, 2, 1)
    L, picks = pk.vote_table(Qg.astype(np.float32), s, 4, w, n_sub=D // m, m=m)
    assert np.array_equal(picks[:, 0], np.tile(np.arange(4), (3, 1)))
    want = np.zeros(1 << m, np.int64)
    want[:4] = 3 * np.array(w)
    assert np.array_equal(L[0].astype(np.int64), want)
