"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: bucket ids, nibbles, vote tables, coarse scores and candidate sets
bit-exact; w within 1e-6 relative; RSQ-IP estimates within 1e-4 of the sum of
absolute terms; fine sets identical except for members whose oracle estimate
ties the k-th within that tolerance; attention within 2e-2 (bf16) / 1e-5
(fp32) max-abs, against the oracle's attention over the same set.
"""
import numpy as np
import pytest
import torch

from oracle import pariskv as ok
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


def _full_check(wl, units=None, capacity=None, tag=""):
    units = list(range(wl.n_units)) if units is None else units
    gc.log(f"[{tag}] {wl.name} N={wl.n_tokens} units={len(units)}/{wl.n_units}")
    pkv = gc.make_ctx(wl, capacity=capacity)
    pkv.encode_keys(wl.n_tokens)
    q = gc.queries(wl)
    sel, sel_n = pkv.retrieve(q)
    out = pkv.sparse_attend(q, sel, sel_n)
    torch.cuda.synchronize()
    enc = gc.check_encode(wl, pkv, units)
    res = gc.check_retrieval(wl, pkv, units, sel, sel_n, enc)
    err = gc.check_attention(wl, pkv, units, sel, sel_n, out)
    rec, planted = gc.recall_report(wl, pkv, units, sel, sel_n)
    nd = sum(r["n_diff"] for r in res.values())
    gc.log(f"[{tag}] ok: attention max-abs {err:.3g}, fine-set tie swaps {nd}, "
           f"recall@k {rec:.3f}" + (f", planted recall {planted:.3f}" if planted is not None else ""))
    return pkv, sel, sel_n, out


def test_single_head_4k_f32():
    _full_check(W.single_head_f32(), tag="single-head")


def test_gqa_ragged_small():
    # several scan chunks per unit and a ragged tail; batch 2 x 8 kv heads
    _full_check(W.gqa_bf16(N=20011, batch=2, top_k=512), tag="ragged")


def test_gqa_32k():
    _full_check(W.gqa_bf16(N=32768), tag="gqa-32k")


def test_gqa_128k_batch4_planted():
    wl = W.gqa_128k_planted()
    pkv, sel, sel_n, out = _full_check(wl, units=[0, 13, 31], tag="gqa-128k")
    # every unit: k ascending positions inside the retrieval zone
    n, sink_end, r_end, _ = pkv.window()
    s = sel.cpu().numpy().reshape(wl.n_units, -1)
    assert np.all(sel_n.cpu().numpy() == wl.params.top_k)
    assert np.all(np.diff(s, axis=1) > 0) and s.min() >= sink_end and s.max() < r_end
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("m", [4, 16])
def test_gqa_128k_batch4_planted_subspace_widths(m):
    """The full 128K-token, batch-4 planted workload with m = 4 and m = 16
    subspaces, in the launch configuration the variant sweep times; two units
    against the oracle."""
    import dataclasses
    wl = W.gqa_128k_planted()
    wl.params = dataclasses.replace(wl.params, n_sub=128 // m, sub_dim=m)
    _full_check(wl, units=[5, 26], tag=f"gqa-128k-m{m}")


def test_maximum_capacity_single_head():
    """The largest context the library accepts: 2^24 tokens in one fp32 unit.
    Record offsets reach 2^31 bytes, the scan and rerank run 2048 chunks of
    8192 keys, and the 10 % coarse budget gives 1.68M candidates (the streaming
    fine selection).  Against the oracle: ids, codes and w of 4096 random
    positions, the vote table, those positions' coarse scores, the estimates of
    4096 random candidates, and the attention over the library's selection.
    Over all positions, exactly: the candidate set is the keys above the
    threshold plus the first ties in position order, and the fine set is the
    top-k of the candidates' estimates (ties to the lower position)."""
    N = 1 << 24
    wl = W.single_head_f32(N=N, threads=16)
    p = wl.params
    gc.log(f"[max-capacity] {wl.name} N={N}")
    pkv = gc.make_ctx(wl)
    pkv.encode_keys(N)
    q = gc.queries(wl)
    sel, sel_n = pkv.retrieve(q)
    out = pkv.sparse_attend(q, sel, sel_n)
    torch.cuda.synchronize()
    n, sink_end, r_end, _ = pkv.window()
    K, V, Qg = gc.unit_view(wl, 0)
    s = wl.signs()
    levels, sq_t = gc.tables(wl)
    r = np.random.default_rng(7)
    # encode, vote table and coarse scores at sampled positions
    P = np.sort(r.choice(np.arange(sink_end, r_end), 4096, replace=False))
    i_o, n_o, w_o = ok.encode_keys(K[P], s, levels, sq_t)
    ids = pkv.debug(0)[0].reshape(-1, 16)
    rec = pkv.debug(1)[0].reshape(-1, 128)
    assert np.array_equal(ids[P], i_o), "bucket ids differ"
    assert np.array_equal(rec[P, :64], n_o), "nibbles differ"
    w_g = rec[P, 64:].copy().view(np.float32).astype(np.float64)
    assert np.all(np.abs(w_g - w_o) <= gc.W_RTOL * np.maximum(np.abs(w_o), 1e-30)), "w differ"
    L, _ = ok.vote_table(Qg, s, p.rho, p.vote_weights)
    assert np.array_equal(pkv.debug(2)[0].reshape(16, 256).astype(np.int64), L.astype(np.int64))
    sc = pkv.debug(3)[0][:r_end - sink_end].astype(np.int64)
    assert np.array_equal(sc[P - sink_end], np.minimum(ok.coarse_scores(i_o, L), 255))
    # the candidate set over all positions, from the (sample-checked) scores
    meta = pkv.debug(6)[0]
    T, need, C = int(meta[0]), int(meta[1]), int(meta[2])
    N_r = r_end - sink_end
    assert C == ok.coarse_count(N_r, p.coarse_permille, p.top_k) and sc.max() < 255
    above = np.flatnonzero(sc > T)
    ties = np.flatnonzero(sc == T)
    assert above.size < C <= above.size + ties.size and need == C - above.size
    cand_want = np.sort(np.concatenate([above, ties[:need]])) + sink_end
    cand = pkv.debug(4)[0][:C]
    assert np.array_equal(cand, cand_want), "candidate set differs"
    # estimates at sampled candidates
    est = pkv.debug(5)[0][:C].astype(np.float64)
    Ci = np.sort(r.choice(C, 4096, replace=False))
    _, n_c, w_c = ok.encode_keys(K[cand[Ci]], s, levels, sq_t)
    e_o = ok.rsq_ip(n_c, w_c, Qg, s, levels)
    scale = gc.est_scale(n_c, w_c, Qg, s, levels)
    assert np.all(np.abs(est[Ci] - e_o) <= gc.EST_RTOL * np.maximum(scale, 1e-30)), "estimates differ"
    # the fine set from the (sample-checked) estimates
    k_eff = min(p.top_k, C)
    sel_g = sel.cpu().numpy().reshape(-1)[:k_eff]
    assert int(sel_n.cpu().item()) == k_eff
    assert np.array_equal(sel_g, np.sort(ok.top_by_key(est, cand, k_eff))), "fine set differs"
    err = gc.check_attention(wl, pkv, [0], sel, sel_n, out)
    gc.log(f"[max-capacity] ok: C={C}, T={T}, ties taken {need}, attention max-abs {err:.3g}")


def test_many_units():
    """Batch 128 x 8 kv heads = 1024 units (the units are the grid's y
    dimension of most kernels), short contexts; units spread over the batch
    against the oracle, through the separate calls and one fused decode step."""
    wl = W.gqa_bf16(N=2500, batch=128, top_k=64, n_local=128, buf_tokens=16)
    pkv, sel, sel_n, out = _full_check(wl, units=[0, 517, 1023], capacity=2600, tag="1024-units")
    dt = gc.torch_dtype(wl)
    Kn, Vn, Qn = W.decode_stream(wl, 1)
    out, sel, sel_n = pkv.decode_step(torch.from_numpy(Kn[0]).to(dt).cuda(),
                                      torch.from_numpy(Vn[0]).to(dt).cuda(),
                                      torch.from_numpy(Qn[0]).to(dt).cuda())
    torch.cuda.synchronize()
    Kall = np.concatenate([wl.K, np.moveaxis(Kn, 0, 2)], axis=2)
    Vall = np.concatenate([wl.V, np.moveaxis(Vn, 0, 2)], axis=2)
    full = W.Workload(wl.name, wl.batch, wl.n_kv, wl.group, wl.n_tokens + 1, wl.dtype, wl.params,
                      wl.sign_bits, Kall, Vall, Qn[0])
    enc = gc.check_encode(full, pkv, [3, 1000])
    gc.check_retrieval(full, pkv, [3, 1000], sel, sel_n, enc)
    gc.check_attention(full, pkv, [3, 1000], sel, sel_n, out)


def test_fine_selection_30k_candidates():
    """200K tokens with a 15 % coarse budget: about 30000 candidates per unit, past
    what the fused selection holds, so the fine top-k keeps 32 candidates per
    thread in registers (and the hot rows go to the attention launch)."""
    wl = W.gqa_bf16(N=200000, top_k=2048, permille=150, threads=16)
    _full_check(wl, units=[0, 6], tag="30k-candidates")


def test_fine_selection_39k_candidates():
    """A coarse budget of 39244 candidates (15 % of 261628): the register-held
    fine selection at 64 candidates per thread, narrowed first by the sampled
    threshold (about 4000 survivors of 39244)."""
    wl = W.gqa_bf16(N=262144, top_k=2048, permille=150, threads=16)
    C = ok.coarse_count(262144 - 4 - 512, 150, 2048)
    assert 32 * 1024 < C < 65536
    _full_check(wl, units=[2, 7], tag="fine-39k")


def test_fine_selection_39k_identical_keys():
    """39244 candidates whose estimates all tie: the sampled threshold keeps every
    candidate, more than the survivor buffer holds, so the full selection over
    the 64 register-held keys per thread decides (the lowest positions)."""
    wl = W.gqa_bf16(N=262144, top_k=2048, permille=150, threads=16)
    wl.K[:, :, 4:] = wl.K[:, :, 4:5]
    pkv, sel, sel_n, _ = _full_check(wl, units=[5], tag="fine-39k-identical")
    _, sink_end, _, _ = pkv.window()
    s = sel.cpu().numpy().reshape(wl.n_units, -1)
    assert np.array_equal(s[5], np.arange(sink_end, sink_end + 2048))


def test_dense_attention_matches_oracle():
    """pk_dense_attend: full attention over every stored token of each unit, against
    the oracle's attention over all positions; ragged last split."""
    wl = W.gqa_bf16(N=20011, batch=2, top_k=512)
    pkv = gc.make_ctx(wl)
    pkv.encode_keys(wl.n_tokens)
    q = gc.queries(wl)
    out = pkv.dense_attend(q).cpu().numpy().reshape(wl.n_units, wl.group, 128)
    for u in (0, 9, 15):
        K, V, Qg = gc.unit_view(wl, u)
        ref = ok.sparse_attention(Qg, K, V, np.arange(wl.n_tokens))
        e = float(np.max(np.abs(out[u] - ref)))
        assert e <= gc.ATT_TOL["bf16"], f"unit {u}: dense attention max-abs err {e:.3g}"


def test_all_keys_kept_is_full_attention():
    wl = W.gqa_bf16(N=3000, top_k=4096, permille=1000, n_local=64)
    pkv = gc.make_ctx(wl)
    pkv.encode_keys(wl.n_tokens)
    q = gc.queries(wl)
    sel, sel_n = pkv.retrieve(q)
    out = pkv.sparse_attend(q, sel, sel_n).cpu().numpy()
    assert np.all(sel_n.cpu().numpy() == 3000 - 4 - 64)
    for u in range(wl.n_units):
        K, V, Qg = gc.unit_view(wl, u)
        ref = ok.sparse_attention(Qg, K, V, np.arange(3000))
        assert np.max(np.abs(out.reshape(8, 4, 128)[u] - ref)) <= 2e-2


def test_empty_retrieval_zone():
    wl = W.gqa_bf16(N=300)                # shorter than sink + local
    pkv = gc.make_ctx(wl)
    pkv.encode_keys(300)
    q = gc.queries(wl)
    sel, sel_n = pkv.retrieve(q)
    out = pkv.sparse_attend(q, sel, sel_n).cpu().numpy().reshape(8, 4, 128)
    assert np.all(sel_n.cpu().numpy() == 0)
    for u in range(8):
        K, V, Qg = gc.unit_view(wl, u)
        assert np.max(np.abs(out[u] - ok.sparse_attention(Qg, K, V, np.arange(300)))) <= 2e-2


def test_retrieval_zone_smaller_than_k():
    _full_check(W.gqa_bf16(N=1000), tag="short")


def test_single_token_context():
    wl = W.single_head_f32(N=1)
    pkv = gc.make_ctx(wl)
    pkv.encode_keys(1)
    q = gc.queries(wl)
    sel, sel_n = pkv.retrieve(q)
    out = pkv.sparse_attend(q, sel, sel_n).cpu().numpy()
    assert sel_n.item() == 0
    assert np.max(np.abs(out[0, 0] - wl.V[0, 0, 0])) <= 1e-6


def test_fine_ties_identical_keys():
    """Every retrieval-zone key identical: all coarse scores and estimates tie, so
    candidates and the top-k are the lowest positions (degenerate value range)."""
    wl = W.gqa_bf16(N=20000, top_k=512, permille=100)
    wl.K[:, :, 4:] = wl.K[:, :, 4:5]
    pkv, sel, sel_n, _ = _full_check(wl, units=[0, 7], tag="identical")
    _, sink_end, _, _ = pkv.window()
    s = sel.cpu().numpy().reshape(wl.n_units, -1)
    assert np.array_equal(s[0], np.arange(sink_end, sink_end + 512))


@pytest.mark.parametrize("m", [8, 4, 16])
def test_saturated_coarse_scores(m):
    """A fifth of the keys equal to the query shared by the whole GQA group: those
    score the maximum B G w_max (every subspace's top centroid for every head):
    256 for m = 8 and 512 for m = 4, above the 255 a stored score holds, and
    they are more than the coarse budget, so the threshold is that maximum and
    the saturated keys are rescored from their ids (with the pair tables for
    m = 4).  For m = 16 the maximum is 128: no saturation, but thousands of
    keys tie at the threshold in the hashed tables."""
    import dataclasses
    wl = W.gqa_bf16(N=20000, top_k=512, permille=100)
    wl.params = dataclasses.replace(wl.params, n_sub=128 // m, sub_dim=m)
    G = wl.group
    for h in range(wl.n_kv):
        wl.Q[:, h * G:(h + 1) * G] = wl.Q[:, h * G:h * G + 1]
    pos = np.arange(4, 20000)
    hit = pos[pos % 5 == 0]
    for h in range(wl.n_kv):
        wl.K[:, h, hit] = wl.Q[:, h * G][:, None, :]
    pkv, sel, sel_n, _ = _full_check(wl, units=[0, 5], tag=f"saturated-m{m}")
    meta = pkv.debug(6)
    top = (128 // m) * G * 4
    assert meta[0][0] == top and meta[5][0] == top, meta[:, 0]


@pytest.mark.parametrize("rho,weights,permille", [
    (1, (1,), 50),                          # top centroid only
    (2, (2, 1), 100),                       # 10 % coarse budget
    (4, (8, 4, 2, 1), 50),                  # powers-of-two weights: 513 score bins
    (8, (8, 7, 6, 5, 4, 3, 2, 1), 80),      # widest probe, linear weights
])
def test_vote_variants(rho, weights, permille):
    """The page leaves the probe count, the hierarchical weights and the coarse
    fraction open: every stage stays bit-exact (ids, tables, scores, candidate
    sets) and within tolerance for other settings of them."""
    import dataclasses
    wl = W.gqa_bf16(N=24000, top_k=512, permille=permille)
    wl.params = dataclasses.replace(wl.params, rho=rho, vote_weights=tuple(weights))
    _full_check(wl, units=[0, 3, 6], tag=f"rho{rho}-w{'-'.join(map(str, weights))}-p{permille}")


@pytest.mark.parametrize("group,dtype", [(1, "bf16"), (2, "bf16"), (8, "bf16"), (4, "f32")])
def test_group_sizes_and_fp32(group, dtype):
    """Other query-group sizes (1, 2 and 8 query heads per kv head: the vote
    tables, the summed rerank query and the attention kernels for those widths)
    and an fp32 store with G = 4, through the separate calls and the fused decode
    step."""
    wl = W.gqa_bf16(N=12000, top_k=512, permille=80, group=group, dtype=dtype, buf_tokens=32,
                    n_local=64)
    pkv, sel, sel_n, out = _full_check(wl, units=[0, 5], capacity=12100, tag=f"g{group}-{dtype}")
    # one fused decode step (append + retrieve + attend) against the oracle too
    dt = gc.torch_dtype(wl)
    Kn, Vn, Qn = W.decode_stream(wl, 1)
    k = torch.from_numpy(Kn[0]).to(dt).cuda()
    v = torch.from_numpy(Vn[0]).to(dt).cuda()
    q = torch.from_numpy(Qn[0]).to(dt).cuda()
    out, sel, sel_n = pkv.decode_step(k, v, q)
    torch.cuda.synchronize()
    Kall = np.concatenate([wl.K, np.moveaxis(Kn, 0, 2)], axis=2)
    Vall = np.concatenate([wl.V, np.moveaxis(Vn, 0, 2)], axis=2)
    full = W.Workload(wl.name, wl.batch, wl.n_kv, wl.group, wl.n_tokens + 1, wl.dtype, wl.params,
                      wl.sign_bits, Kall, Vall, Qn[0])
    enc = gc.check_encode(full, pkv, [0, 5])
    gc.check_retrieval(full, pkv, [0, 5], sel, sel_n, enc)
    gc.check_attention(full, pkv, [0, 5], sel, sel_n, out)


def test_quantile_codebook():
    """The other reading of the Beta-prior codebook (equal-probability bins):
    nibbles bit-exact, w and the estimates within tolerance, sets and attention
    as usual, with the library's own quantile tables."""
    import dataclasses
    wl = W.gqa_bf16(N=20000, top_k=512, permille=80)
    wl.params = dataclasses.replace(wl.params, codebook="quantile")
    _full_check(wl, units=[0, 4, 7], tag="quantile-codebook")


@pytest.mark.parametrize("m,dtype,group", [(4, "bf16", 4), (4, "f32", 2), (16, "bf16", 4),
                                           (16, "f32", 8)])
def test_subspace_widths(m, dtype, group):
    """Other subspace widths.  m = 4: 32 subspaces of 16 sign-pattern centroids,
    two 4-bit ids per id byte, 32 scales in a 192-byte record.  m = 16: 8
    subspaces of 65536 centroids, 16-bit ids, hashed vote tables, 8 scales in
    a 96-byte record.  Each with its own codebook.  ids, codes, votes, scores
    and candidate sets bit-exact, w and estimates within tolerance, attention
    as usual; then 70 fused decode steps through two buffer fills, so the
    device also encodes evicted keys at that width."""
    import dataclasses
    wl = W.gqa_bf16(N=20011, top_k=512, permille=50, group=group, dtype=dtype, buf_tokens=32,
                    n_local=64)
    wl.params = dataclasses.replace(wl.params, n_sub=128 // m, sub_dim=m)
    steps = 70
    units = [0, 5]
    pkv, sel, sel_n, out = _full_check(wl, units=units, capacity=wl.n_tokens + steps,
                                       tag=f"m{m}-{dtype}-g{group}")
    dt = gc.torch_dtype(wl)
    Kn, Vn, Qn = W.decode_stream(wl, steps)
    for t in range(steps):
        out, sel, sel_n = pkv.decode_step(torch.from_numpy(Kn[t]).to(dt).cuda(),
                                          torch.from_numpy(Vn[t]).to(dt).cuda(),
                                          torch.from_numpy(Qn[t]).to(dt).cuda())
    torch.cuda.synchronize()
    n, sink_end, r_end, _ = pkv.window()
    assert n == wl.n_tokens + steps and r_end == wl.n_tokens - 64 + 2 * 32   # two evictions
    Kall = np.concatenate([wl.K, np.moveaxis(Kn, 0, 2)], axis=2)
    Vall = np.concatenate([wl.V, np.moveaxis(Vn, 0, 2)], axis=2)
    full = W.Workload(wl.name, wl.batch, wl.n_kv, wl.group, n, wl.dtype, wl.params, wl.sign_bits,
                      Kall, Vall, Qn[-1])
    enc = gc.check_encode(full, pkv, units)
    gc.check_retrieval(full, pkv, units, sel, sel_n, enc)
    gc.check_attention(full, pkv, units, sel, sel_n, out)
    gc.log(f"[m{m}-{dtype}-g{group}] decode steps ok (r_end {r_end})")


@pytest.mark.parametrize("m,rho,group", [(16, 8, 8), (4, 8, 2), (16, 1, 1)])
def test_subspace_width_probe_counts(m, rho, group):
    """Edges of the m = 4 and m = 16 query preparation: 8 probes of 16
    centroids (m = 4), 8 probes by 8 heads merged into one m = 16 table (64
    picks, every lane of the merge wave), and a single probe of a single head."""
    import dataclasses
    wl = W.gqa_bf16(N=16000, top_k=512, permille=60, group=group)
    wl.params = dataclasses.replace(wl.params, n_sub=128 // m, sub_dim=m, rho=rho,
                                    vote_weights=tuple(range(rho, 0, -1)))
    _full_check(wl, units=[1, 6], tag=f"m{m}-rho{rho}-g{group}")


@pytest.mark.parametrize("m", [4, 8, 16])
def test_tied_centroid_scores(m):
    """Queries whose rotated coordinates are exactly -1, 0 or +1, with whole
    subspaces zero: many centroid scores tie exactly (all 2^m of them in a zero
    subspace), so every width's top-rho must fall back to the lower index, and
    the m = 16 selection takes its widest pair search.  fp32 store, so that
    q = D H y / 128 is exact and rotates back to exactly y."""
    import dataclasses
    wl = W.gqa_bf16(N=12000, top_k=256, permille=50, dtype="f32", n_local=64)
    wl.params = dataclasses.replace(wl.params, n_sub=128 // m, sub_dim=m)
    r = np.random.default_rng(5)
    H = ok.sylvester_hadamard(128)
    Y = r.integers(-1, 2, size=wl.Q.shape).astype(np.float64)
    Y[..., 0:16] = 0.0                        # the first 16 rotated coordinates of every head
    Y[:, ::3, 48:64] = 0.0                    # and another block on every third head
    Q = (Y @ H.T) * wl.signs().astype(np.float64) / 128.0
    assert np.array_equal(ok.rotate_spec(Q.reshape(-1, 128).astype(np.float32), wl.signs()),
                          Y.reshape(-1, 128).astype(np.float32))
    wl.Q = Q.astype(np.float32)
    _full_check(wl, units=[0, 3, 7], tag=f"tied-m{m}")


def test_fine_ties_periodic_keys():
    """64 distinct keys repeated along the context: large groups of exactly tied
    estimates around the k-th (the bucket of the k-th holds a whole group)."""
    wl = W.gqa_bf16(N=20000, top_k=512, permille=100)
    src = 4 + (np.arange(4, 20000) - 4) % 64
    wl.K[:, :, 4:] = wl.K[:, :, src]
    _full_check(wl, units=[0, 7], tag="periodic")


def test_fine_two_key_groups():
    """Two distinct keys only (one every 40 positions, the other elsewhere): more
    than a thousand exact ties at the k-th estimate."""
    wl = W.gqa_bf16(N=65536, top_k=1024, permille=50)
    pos = np.arange(4, 65536)
    wl.K[:, :, pos] = np.where((pos % 40 == 0)[None, None, :, None], wl.K[:, :, 4:5], wl.K[:, :, 5:6])
    _full_check(wl, units=[0], tag="two-groups")


def test_host_mapped_store_matches_device_store():
    """K/V store in pinned host memory (hot zone mirrored in a device ring): the same
    window, selection and bit-identical output as a device store, across evictions."""
    T, N0 = 70, 40000
    wl = W.gqa_bf16(N=N0, top_k=512, n_local=256, buf_tokens=32)
    Kn, Vn, Qn = W.decode_stream(wl, T)
    a = gc.make_ctx(wl, capacity=N0 + T)
    b = gc.make_ctx(wl, capacity=N0 + T, host_mapped=True)
    assert b.K.device.type == "cpu" and b.K.is_pinned()
    a.encode_keys(N0)
    b.encode_keys(N0)
    dt = gc.torch_dtype(wl)
    for t in range(T):
        k = torch.from_numpy(Kn[t]).to(dt).cuda()
        v = torch.from_numpy(Vn[t]).to(dt).cuda()
        q = torch.from_numpy(Qn[t]).to(dt).cuda()
        out_a, sel_a, n_a = a.decode_step(k, v, q)
        out_b, sel_b, n_b = b.decode_step(k, v, q)
        assert a.window() == b.window()
        if t % 8 == 0 or t in (31, 32, 33, 63, 64, 65):
            torch.cuda.synchronize()
            assert torch.equal(n_a, n_b) and torch.equal(sel_a, sel_b)
            assert torch.equal(out_a, out_b), f"step {t}"
    torch.cuda.synchronize()
    assert torch.equal(a.K.cpu(), b.K) and torch.equal(a.V.cpu(), b.V)
    gc.log(f"[host-mapped] {T} steps identical to the device store, window {b.window()}")


def test_1m_context_host_mapped_store():
    """1M-token context per unit (8 kv heads, G=4) with the K/V store in pinned host
    memory: encode, retrieval and attention of one unit against the oracle."""
    N = 1 << 20
    gc.log("[1M] generating the workload ...")
    wl = W.gqa_bf16(N=N, batch=1, n_local=1024, threads=16, name="gqa_1m_b1_bf16")
    pkv = gc.make_ctx(wl, host_mapped=True)
    gc.log("[1M] store filled; encoding ...")
    pkv.encode_keys(N)
    q = gc.queries(wl)
    sel, sel_n = pkv.retrieve(q)
    out = pkv.sparse_attend(q, sel, sel_n)
    torch.cuda.synchronize()
    gc.log("[1M] checking unit 3 against the oracle ...")
    enc = gc.check_encode(wl, pkv, [3])
    res = gc.check_retrieval(wl, pkv, [3], sel, sel_n, enc)
    err = gc.check_attention(wl, pkv, [3], sel, sel_n, out)
    n, sink_end, r_end, _ = pkv.window()
    C = ok.coarse_count(r_end - sink_end, wl.params.coarse_permille, wl.params.top_k)
    gc.log(f"[1M] ok: C = {C}, tie swaps {res[3]['n_diff']}, attention max-abs {err:.3g}")


def test_drift_decode_16k_steps():
    """32768-token prefill, then 16384 decode steps whose key and query mean drifts by two
    standard deviations along a random direction (update buffer U = 256, k = 1024).
    Parity with the oracle at five steps spread over the run; recall@k against the exact
    top-k of the retrieval zone every 1024 steps (reported)."""
    T, N0 = 16384, 32768
    wl = W.gqa_bf16(N=N0, top_k=1024, buf_tokens=256)
    Kn, Vn, Qn = W.decode_stream(wl, T)
    pkv = gc.make_ctx(wl, capacity=N0 + T)
    pkv.encode_keys(N0)
    dt = gc.torch_dtype(wl)
    Kd = torch.from_numpy(Kn).to(dt).cuda()
    Vd = torch.from_numpy(Vn).to(dt).cuda()
    Qd = torch.from_numpy(Qn).to(dt).cuda()
    full = W.Workload(wl.name, wl.batch, wl.n_kv, wl.group, N0 + T, wl.dtype, wl.params,
                      wl.sign_bits, np.concatenate([wl.K, np.moveaxis(Kn, 0, 2)], axis=2),
                      np.concatenate([wl.V, np.moveaxis(Vn, 0, 2)], axis=2), wl.Q)
    check_at = {0, 4095, 8191, 12287, T - 1}
    curve = []
    for t in range(T):
        out, sel, sel_n = pkv.decode_step(Kd[t], Vd[t], Qd[t])
        if t in check_at or (t + 1) % 1024 == 0:
            torch.cuda.synchronize()
            full.Q = Qn[t]
            if t in check_at:
                enc = gc.check_encode(full, pkv, [0])
                gc.check_retrieval(full, pkv, [0], sel, sel_n, enc)
                gc.check_attention(full, pkv, [0], sel, sel_n, out)
            if (t + 1) % 1024 == 0:
                rec, _ = gc.recall_report(full, pkv, list(range(wl.n_units)), sel, sel_n)
                curve.append(rec)
                gc.log(f"[drift] step {t + 1}: window {pkv.window()}, recall@k {rec:.3f}")
    assert len(curve) == T // 1024 and all(0.0 <= r <= 1.0 for r in curve)


def test_decode_window_append_evict():
    """Appends through several buffer fills: the window mirror follows the oracle's,
    evicted keys are encoded exactly like a prefill encode, and sampled steps match."""
    T, N0 = 200, 4096
    wl = W.gqa_bf16(N=N0, top_k=256, n_local=128, buf_tokens=64)
    Kn, Vn, Qn = W.decode_stream(wl, T)
    pkv = gc.make_ctx(wl, capacity=N0 + T)
    pkv.encode_keys(N0)
    win = ok.Window(N0, 4, 128, 64)
    dt = gc.torch_dtype(wl)
    Kall = np.concatenate([wl.K, np.moveaxis(Kn, 0, 2)], axis=2)
    Vall = np.concatenate([wl.V, np.moveaxis(Vn, 0, 2)], axis=2)
    full = W.Workload(wl.name, wl.batch, wl.n_kv, wl.group, N0 + T, wl.dtype, wl.params,
                      wl.sign_bits, Kall, Vall, wl.Q)
    check_at = {0, 63, 64, 65, 127, 128, 199}
    for t in range(T):
        pkv.append(torch.from_numpy(Kn[t]).to(dt).cuda(), torch.from_numpy(Vn[t]).to(dt).cuda())
        win.append()
        assert pkv.window() == (win.n, win.sink_end, win.r_end, win.buf)
        q = torch.from_numpy(Qn[t]).to(dt).cuda()
        sel, sel_n = pkv.retrieve(q)
        out = pkv.sparse_attend(q, sel, sel_n)
        if t in check_at:
            torch.cuda.synchronize()
            full.Q = Qn[t]
            units = [0, 5]
            enc = gc.check_encode(full, pkv, units)
            gc.check_retrieval(full, pkv, units, sel, sel_n, enc)
            gc.check_attention(full, pkv, units, sel, sel_n, out)
            gc.log(f"[decode] step {t}: window {pkv.window()} ok")
        win.end_step()


def test_learned_centroids_match_oracle():
    """Comparison stage with centroids fitted by k-means to the prefill keys: the
    fitted tables are bit-exact against the oracle's fit, and so are the bucket ids
    of the prefill keys and of keys evicted during decoding, the vote tables, the
    coarse scores and candidate sets; estimates, selection and attention to the
    usual bars."""
    from oracle import kmeans as km
    T, N0, iters = 140, 3000, 3
    wl = W.gqa_bf16(N=N0, top_k=256, n_local=128, buf_tokens=64)
    Kn, Vn, Qn = W.decode_stream(wl, T)
    init = W.kmeans_init_positions(wl.n_units, N0)
    pkv = gc.make_ctx(wl, capacity=N0 + T)
    pkv.fit_centroids(N0, torch.from_numpy(init).cuda(), iters)
    pkv.encode_keys(N0)
    torch.cuda.synchronize()
    s = wl.signs()
    p = wl.params
    units = [0, 3, 6]
    import kv_cache_top_amd._native as nat
    cents = pkv.debug(nat.PK_DBG_CENTROIDS).reshape(wl.n_units, 16, 256, 8)
    ref = {}
    for u in units:
        K, _, _ = gc.unit_view(wl, u)
        c_o, _ = km.fit(K[:N0], s, init[u], iters)
        assert np.array_equal(cents[u], c_o), \
            f"unit {u}: centroids differ at {np.argwhere(cents[u] != c_o)[:4]}"
        ref[u] = c_o
    ids_fn = lambda u, keys: km.encode_ids(keys, s, ref[u])
    vote_fn = lambda u, Qg: km.vote_table(Qg, s, ref[u], p.rho, p.vote_weights)
    dt = gc.torch_dtype(wl)
    Kall = np.concatenate([wl.K, np.moveaxis(Kn, 0, 2)], axis=2)
    Vall = np.concatenate([wl.V, np.moveaxis(Vn, 0, 2)], axis=2)
    full = W.Workload(wl.name, wl.batch, wl.n_kv, wl.group, N0 + T, wl.dtype, wl.params,
                      wl.sign_bits, Kall, Vall, wl.Q)
    for t in range(T):
        pkv.append(torch.from_numpy(Kn[t]).to(dt).cuda(), torch.from_numpy(Vn[t]).to(dt).cuda())
        q = torch.from_numpy(Qn[t]).to(dt).cuda()
        sel, sel_n = pkv.retrieve(q)
        out = pkv.sparse_attend(q, sel, sel_n)
        if t in (0, 64, 65, 129):
            torch.cuda.synchronize()
            full.Q = Qn[t]
            enc = gc.check_encode(full, pkv, units, ids_fn=ids_fn)
            gc.check_retrieval(full, pkv, units, sel, sel_n, enc, vote_fn=vote_fn)
            gc.check_attention(full, pkv, units, sel, sel_n, out)
            gc.log(f"[learned] step {t}: window {pkv.window()} ok")


def test_decode_step_matches_separate_calls():
    """pk_decode_step (append fused into the first retrieval kernel) gives the same
    window, selection and output as append + retrieve + attend, across an eviction."""
    T, N0 = 80, 3000
    wl = W.gqa_bf16(N=N0, top_k=256, n_local=64, buf_tokens=32)
    Kn, Vn, Qn = W.decode_stream(wl, T)
    a = gc.make_ctx(wl, capacity=N0 + T)
    b = gc.make_ctx(wl, capacity=N0 + T)
    a.encode_keys(N0)
    b.encode_keys(N0)
    dt = gc.torch_dtype(wl)
    for t in range(T):
        k = torch.from_numpy(Kn[t]).to(dt).cuda()
        v = torch.from_numpy(Vn[t]).to(dt).cuda()
        q = torch.from_numpy(Qn[t]).to(dt).cuda()
        out_a, sel_a, n_a = a.decode_step(k, v, q)
        b.append(k, v)
        sel_b, n_b = b.retrieve(q)
        out_b = b.sparse_attend(q, sel_b, n_b)
        assert a.window() == b.window()
        if t % 10 == 0 or t in (31, 32, 33):
            torch.cuda.synchronize()
            assert torch.equal(n_a, n_b) and torch.equal(sel_a, sel_b)
            assert torch.equal(out_a, out_b)
    torch.cuda.synchronize()
    assert torch.equal(a.K, b.K) and torch.equal(a.V, b.V)


def test_decode_step_raw_matches_decode_step():
    """The raw-address entry of the binding issues the same pk_decode_step."""
    T, N0 = 12, 3000
    wl = W.gqa_bf16(N=N0, top_k=256, n_local=64, buf_tokens=8)
    Kn, Vn, Qn = W.decode_stream(wl, T)
    a = gc.make_ctx(wl, capacity=N0 + T)
    b = gc.make_ctx(wl, capacity=N0 + T)
    a.encode_keys(N0)
    b.encode_keys(N0)
    dt = gc.torch_dtype(wl)
    sel = torch.empty((wl.batch, wl.n_kv, 256), dtype=torch.int32, device="cuda")
    sel_n = torch.empty((wl.batch, wl.n_kv), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.batch, wl.n_kv * wl.group, 128), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for t in range(T):
        k = torch.from_numpy(Kn[t]).to(dt).cuda()
        v = torch.from_numpy(Vn[t]).to(dt).cuda()
        q = torch.from_numpy(Qn[t]).to(dt).cuda()
        out_a, sel_a, n_a = a.decode_step(k, v, q)
        b.decode_step_raw(k.data_ptr(), v.data_ptr(), q.data_ptr(), sel.data_ptr(),
                          sel_n.data_ptr(), out.data_ptr(), stream)
        torch.cuda.synchronize()
        assert a.window() == b.window()
        assert torch.equal(n_a, sel_n) and torch.equal(sel_a, sel) and torch.equal(out_a, out)


def test_profiling_counts_launches():
    wl = W.gqa_bf16(N=5000, top_k=256)
    pkv = gc.make_ctx(wl)
    pkv.profile(True)
    pkv.encode_keys(wl.n_tokens)
    q = gc.queries(wl)
    for _ in range(3):
        pkv.step(q)
    prof = pkv.profile_read()
    pkv.profile(False)
    for stage, n in (("encode", 1), ("qprep", 3), ("scan", 3), ("rerank", 3),
                     ("fine", 3), ("attend", 3), ("combine", 3)):
        assert prof[stage][1] == n, (stage, prof[stage])
        assert prof[stage][0] > 0
    assert prof["select"][1] == 0    # the coarse threshold is found inside the rerank launch


def test_deterministic():
    wl = W.gqa_bf16(N=20011, top_k=512)
    pkv = gc.make_ctx(wl)
    pkv.encode_keys(wl.n_tokens)
    q = gc.queries(wl)
    runs = []
    for _ in range(2):
        sel, sel_n = pkv.retrieve(q)
        out = pkv.sparse_attend(q, sel, sel_n)
        torch.cuda.synchronize()
        runs.append((sel.cpu().numpy(), out.cpu().numpy(), pkv.debug(5).copy()))
    assert np.array_equal(runs[0][0], runs[1][0])
    assert np.array_equal(runs[0][1].view(np.uint32), runs[1][1].view(np.uint32))
    assert np.array_equal(runs[0][2].view(np.uint32), runs[1][2].view(np.uint32))


def test_append_past_capacity_is_rejected():
    from kv_cache_top_amd import PkError
    wl = W.gqa_bf16(N=1000, buf_tokens=16, n_local=64)
    pkv = gc.make_ctx(wl, capacity=1001)
    pkv.encode_keys(1000)
    dt = gc.torch_dtype(wl)
    k = torch.zeros((1, 8, 128), dtype=dt, device="cuda")
    pkv.append(k, k)
    before = pkv.window()
    with pytest.raises(PkError):
        pkv.append(k, k)
    assert pkv.window() == before


def test_gather_reference_kernel():
    """The random-gather measurement reference runs for the record and row sizes
    the bench uses and leaves the sink alone (its checksum of zeros is 0)."""
    import ctypes
    import kv_cache_top_amd._native as nat
    arr = torch.zeros(1000 * 512, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    for rec_bytes in (16, 128, 256, 512):
        rows = arr.numel() // rec_bytes
        idx = torch.randint(0, rows, (5003,), device="cuda", generator=g, dtype=torch.int32)
        st = nat.lib.pk_gather_read(ctypes.c_void_p(arr.data_ptr()), rows, rec_bytes,
                                    ctypes.c_void_p(idx.data_ptr()), idx.numel(),
                                    ctypes.c_void_p(sink.data_ptr()), None, None)
        assert st == nat.PK_OK
    # timed forms: the call waits for the kernel and reports a positive duration
    us = ctypes.c_float(0.0)
    assert nat.lib.pk_gather_read(ctypes.c_void_p(arr.data_ptr()), arr.numel() // 256, 256,
                                  ctypes.c_void_p(idx.data_ptr()), idx.numel(),
                                  ctypes.c_void_p(sink.data_ptr()), ctypes.byref(us), None) == nat.PK_OK
    assert 0.0 < us.value < 1e6
    us.value = 0.0
    assert nat.lib.pk_stream_read(ctypes.c_void_p(arr.data_ptr()), arr.numel() - 16,
                                  ctypes.c_void_p(sink.data_ptr()), ctypes.byref(us), None) == nat.PK_OK
    assert 0.0 < us.value < 1e6
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


@pytest.mark.parametrize("m", [4, 16])
def test_learned_centroids_need_width_8(m):
    """The learned-centroid comparison stage fits 256 centroids of 8
    coordinates: other widths are refused (PK_ERR_UNSUPPORTED) before any
    device access, and the context then works as usual."""
    import ctypes
    import dataclasses
    import kv_cache_top_amd._native as nat
    wl = W.gqa_bf16(N=6000, top_k=256)
    wl.params = dataclasses.replace(wl.params, n_sub=128 // m, sub_dim=m)
    pkv = gc.make_ctx(wl)
    init = torch.zeros((wl.n_units, 256), dtype=torch.int32, device="cuda")
    st = nat.lib.pk_fit_centroids(pkv._ctx, wl.n_tokens, ctypes.c_void_p(init.data_ptr()), 3, None)
    assert st == nat.PK_ERR_UNSUPPORTED
    pkv.encode_keys(wl.n_tokens)
    q = gc.queries(wl)
    sel, sel_n = pkv.retrieve(q)
    torch.cuda.synchronize()
    enc = gc.check_encode(wl, pkv, [3])
    gc.check_retrieval(wl, pkv, [3], sel, sel_n, enc)


def test_misaligned_pointers_are_rejected():
    """A device pointer that is not 16-byte aligned (a query taken one element
    into a buffer) is refused on the host with PK_ERR_INVALID by every per-step
    entry point, nothing is launched, and the context is unchanged: the next
    call with aligned buffers matches the oracle."""
    import ctypes
    import kv_cache_top_amd._native as nat
    wl = W.gqa_bf16(N=9000, top_k=256, buf_tokens=16, n_local=64)
    pkv = gc.make_ctx(wl, capacity=9100)
    pkv.encode_keys(wl.n_tokens)
    q = gc.queries(wl)
    big = torch.empty(q.numel() + 8, dtype=q.dtype, device="cuda")
    qm = big[1:1 + q.numel()]                       # 2 bytes past an aligned address
    sel = torch.empty((1, 8, 256), dtype=torch.int32, device="cuda")
    sel_n = torch.empty((1, 8), dtype=torch.int32, device="cuda")
    out = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
    kv = torch.empty((1, 8, 128), dtype=q.dtype, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    before = pkv.window()
    lib, ctx = nat.lib, pkv._ctx
    assert lib.pk_retrieve(ctx, P(qm), P(sel), P(sel_n), None) == nat.PK_ERR_INVALID
    assert lib.pk_sparse_attend(ctx, P(qm), P(sel), P(sel_n), P(out), None) == nat.PK_ERR_INVALID
    assert lib.pk_dense_attend(ctx, P(qm), P(out), None) == nat.PK_ERR_INVALID
    assert lib.pk_decode_step(ctx, P(kv), P(kv), P(qm), P(sel), P(sel_n), P(out),
                              None) == nat.PK_ERR_INVALID
    kvm = torch.empty(kv.numel() + 8, dtype=kv.dtype, device="cuda")[3:3 + kv.numel()]
    assert lib.pk_append_decode_keys(ctx, P(kvm), P(kv), None) == nat.PK_ERR_INVALID
    assert pkv.window() == before
    sel, sel_n = pkv.retrieve(q)
    out = pkv.sparse_attend(q, sel, sel_n)
    torch.cuda.synchronize()
    enc = gc.check_encode(wl, pkv, [2])
    gc.check_retrieval(wl, pkv, [2], sel, sel_n, enc)
    gc.check_attention(wl, pkv, [2], sel, sel_n, out)


def test_create_out_of_device_memory_is_reported():
    """A context whose metadata cannot fit in device memory (64 x 8 units at
    2^24 tokens: 137 GB of ids and 1.1 TB of records) fails with PK_ERR_OOM
    before launching anything, frees what it had allocated, and a normal
    context works afterwards.  The store pointers are never touched by
    pk_create, so small tensors stand in for them."""
    import ctypes
    import kv_cache_top_amd._native as nat
    small = torch.zeros(4096, dtype=torch.bfloat16, device="cuda")
    cfg = nat.make_config()
    ctx = ctypes.c_void_p()
    free0, _ = torch.cuda.mem_get_info()
    st = nat.lib.pk_create(ctypes.byref(cfg), 64, 8, 32, 1 << 24, nat.PK_BF16,
                           ctypes.c_void_p(small.data_ptr()), ctypes.c_void_p(small.data_ptr()),
                           nat.PK_MEM_DEVICE, ctypes.byref(ctx))
    assert st == nat.PK_ERR_OOM and not ctx.value
    free1, _ = torch.cuda.mem_get_info()
    assert free1 >= free0 - (64 << 20), "partial allocations were not released"
    _full_check(W.gqa_bf16(N=9000, top_k=256), units=[0], tag="after-oom")
