"""The pins have teeth: each plants a plausible mistake in a copy of an oracle
function (on the CPU) and checks that the pin written for it fails."""
import math

import numpy as np

from oracle import pariskv as pk
from tests import test_oracle_pins as pins
from tests.test_oracle_codebook import check_lloyd_max_conditions
from oracle.codebook import lloyd_max


def test_fwht_wrong_sign_is_caught():
    def bad(x):
        x = np.array(x, np.float32, copy=True)
        d = x.shape[-1]
        h = 1
        while h < d:
            y = x.reshape(x.shape[:-1] + (d // (2 * h), 2, h))
            lo, hi = y[..., 0, :].copy(), y[..., 1, :].copy()
            y[..., 0, :] = lo + hi
            y[..., 1, :] = hi - lo          # flipped subtraction
            h *= 2
        return x
    assert not pins.check_fwht_exact_on_integers(bad)


def test_fwht_missing_stage_is_caught():
    def bad(x):
        x = np.array(x, np.float32, copy=True)
        d = x.shape[-1]
        h = 2                               # skips the first stage
        while h < d:
            y = x.reshape(x.shape[:-1] + (d // (2 * h), 2, h))
            lo, hi = y[..., 0, :].copy(), y[..., 1, :].copy()
            y[..., 0, :], y[..., 1, :] = lo + hi, lo - hi
            h *= 2
        return x
    assert not pins.check_fwht_exact_on_integers(bad)


def test_bucket_id_bit_order_is_caught():
    def bad(x, n_sub, m):
        xb = np.asarray(x, np.float32).reshape(-1, n_sub, m)
        bits = (xb < 0).astype(np.int64)
        return np.sum(bits << (m - 1 - np.arange(m))[None, None, :], axis=-1).astype(np.uint8)
    assert not pins.check_bucket_ids_brute_force(bad)


def test_bucket_id_zero_tie_is_caught():
    def bad(x, n_sub, m):
        xb = np.asarray(x, np.float32).reshape(-1, n_sub, m)
        bits = (xb <= 0).astype(np.int64)   # zero -> upper centroid
        return np.sum(bits << np.arange(m)[None, None, :], axis=-1).astype(np.uint8)
    assert not pins.check_bucket_ids_brute_force(bad)


def test_top_rho_tie_break_is_caught():
    def bad(scores, rho):
        order = np.lexsort((-np.arange(scores.shape[0]), -scores.astype(np.float64)))
        return order[:rho]
    assert not pins.check_top_rho_brute_force(pk.centroid_scores, bad)


def test_vote_weights_reversed_is_caught():
    def bad(Qg, signs, rho, weights, n_sub=16, m=8):
        return pk.vote_table(Qg, signs, rho, tuple(reversed(weights)), n_sub, m)
    assert not pins.check_vote_table(bad)


def test_coarse_score_dropped_subspace_is_caught():
    def bad(ids, L):
        ids = np.asarray(ids, np.int64)
        return np.sum(L[np.arange(15)[None, :], ids[:, :15]].astype(np.int64), axis=1)
    assert not pins.check_coarse_scores(bad)


def test_selection_tie_break_is_caught():
    def bad(values, positions, count):
        order = np.lexsort((-positions, -np.asarray(values, np.float64)))
        return np.sort(positions[order[:count]])
    assert not pins.check_top_by_key(bad)


def test_w_missing_sqrt_d_is_caught():
    def bad(x, v, ss32, n_sub, m):
        return pk.calibrate_w(x, v, ss32, n_sub, m) * math.sqrt(n_sub * m)
    assert not pins.check_rsq_ip_identity(bad, pk.rsq_ip_directions)


def test_rsq_ip_transposed_rotation_is_caught():
    def bad(v, w, Qg, signs):
        v = np.asarray(v, np.float64)
        n, n_sub, m = v.shape
        R = pk.srht_matrix(signs).T         # transposed operand
        est = np.zeros(n)
        for q in np.atleast_2d(np.asarray(Qg, np.float64)):
            qn = np.linalg.norm(q)
            qt = (R @ q / qn).reshape(n_sub, m)
            est += qn * np.sum(np.asarray(w) * np.einsum("nbj,bj->nb", v, qt), axis=1)
        return est
    assert not pins.check_rsq_ip_identity(pk.calibrate_w, bad)


def test_attention_missing_scale_is_caught():
    def bad(Qg, K, V, attended):
        s = np.atleast_2d(Qg) @ np.asarray(K)[attended].T
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        return p @ np.asarray(V)[attended]
    assert not pins.check_attention_full(bad)


def test_codebook_wrong_prior_is_caught():
    c, t = lloyd_max(6)                     # codebook of the wrong dimension
    assert not check_lloyd_max_conditions(c, t)


def _w_alignment_variant(kind):
    """calibrate_w with the alignment <v_b, u_b> used in another way than the
    page's division: multiplied in, or the least-squares scale <v,u>/||v||^2."""
    def bad(x, v, ss32, n_sub, m):
        xb = np.asarray(x, np.float64).reshape(-1, n_sub, m)
        norm = np.sqrt(np.sum(xb * xb, axis=-1))
        u = xb / np.where(norm > 0, norm, 1.0)[..., None]
        v = np.asarray(v, np.float64)
        align = np.sum(v * u, axis=-1)
        if kind == "multiply":
            f = align
        else:
            f = align / np.sum(v * v, axis=-1)
        return np.where(np.asarray(ss32) != 0, norm / math.sqrt(n_sub * m) * f, 0.0)
    return bad


def test_w_alignment_multiplied_is_caught():
    for m in (8, 4, 16):
        assert not pins.check_rsq_ip_parallel_query(_w_alignment_variant("multiply"),
                                                    pk.rsq_ip_directions, 128 // m, m)


def test_w_least_squares_is_caught():
    for m in (8, 4, 16):
        assert not pins.check_rsq_ip_parallel_query(_w_alignment_variant("least_squares"),
                                                    pk.rsq_ip_directions, 128 // m, m)


def test_w_least_squares_passes_the_identity_pin():
    """Why the parallel-query pin is needed: with v = u both wrong forms equal
    the page's w, so the identity-quantisation pin cannot tell them apart."""
    assert pins.check_rsq_ip_identity(_w_alignment_variant("least_squares"), pk.rsq_ip_directions)
    assert pins.check_rsq_ip_identity(_w_alignment_variant("multiply"), pk.rsq_ip_directions)
