"""GPU parity of the decode step exactly as the benchmark times it, and of the
window edges the other tests do not reach.

* The 128K-token, batch-4 planted workload with an update buffer of 256
  tokens, stepped with pk_decode_step through its first eviction: C = 6528
  candidates per unit, so the fine selection runs fused with the hot-zone
  attention splits holding 8 candidates per thread.
* A coarse budget of 13004 candidates (16 per thread in the fused launch).
* Empty sink and/or local zones (no always-attended rows at all).
* A pinned host-memory store whose prefill is shorter than the sink zone
  (the appended tokens are local tokens, kept in the device ring).
* A static retrieval + attention captured in a HIP graph and replayed.

Bars as in test_gpu_parity.py (ParisKV page, "Two-stage GPU-native retrieval
pipeline", "Sliding-window update mechanism", "UVA offloading").
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


def _extended(wl, Kn, Vn):
    """The workload with the decode tokens appended (what the oracle reads)."""
    return W.Workload(wl.name, wl.batch, wl.n_kv, wl.group, wl.n_tokens + Kn.shape[0], wl.dtype,
                      wl.params, wl.sign_bits,
                      np.concatenate([wl.K, np.moveaxis(Kn, 0, 2)], axis=2),
                      np.concatenate([wl.V, np.moveaxis(Vn, 0, 2)], axis=2), wl.Q,
                      wl.planted, wl.planted_dir, wl.seed, wl.layer)


def _step_and_check(wl, pkv, Kn, Vn, Qn, check_at, units, tag, host_window=None):
    """pk_decode_step over every token of the stream; full stage-by-stage checks of
    `units` at the steps in check_at (after the step, before the next append)."""
    dt = gc.torch_dtype(wl)
    Kd = torch.from_numpy(Kn).to(dt).cuda()
    Vd = torch.from_numpy(Vn).to(dt).cuda()
    Qd = torch.from_numpy(Qn).to(dt).cuda()
    full = _extended(wl, Kn, Vn)
    win = ok.Window(wl.n_tokens, wl.params.n_sink, wl.params.n_local, wl.params.buf_tokens)
    for t in range(Kn.shape[0]):
        out, sel, sel_n = pkv.decode_step(Kd[t], Vd[t], Qd[t])
        win.append()
        assert pkv.window() == (win.n, win.sink_end, win.r_end, win.buf), f"step {t}"
        if t in check_at:
            torch.cuda.synchronize()
            full.Q = Qn[t]
            n, sink_end, r_end, _ = pkv.window()
            if r_end > sink_end:
                enc = gc.check_encode(full, pkv, units)
                gc.check_retrieval(full, pkv, units, sel, sel_n, enc)
            else:
                assert np.all(sel_n.cpu().numpy() == 0)
            err = gc.check_attention(full, pkv, units, sel, sel_n, out)
            gc.log(f"[{tag}] step {t}: window {pkv.window()} ok, attention max-abs {err:.3g}")
        win.end_step()


def test_graded_decode_step_128k_batch4():
    """The benchmark's workload and call: 131072 tokens x batch 4 x 8 kv heads, G = 4,
    bf16, sink 4 + local 512 + update buffer 256, top-k 2048 of a 5 % coarse set
    (C = 6528), one pk_decode_step per token.  Units 0, 13 and 31 against the
    oracle on the first step, on the step that fills the buffer, and on the first
    step after the 256 oldest local tokens were evicted and encoded."""
    T = 258
    wl = W.gqa_128k_planted()
    wl.params.buf_tokens = 256
    gc.log(f"[graded] {wl.name}: {wl.n_units} units, U = 256, {T} decode steps")
    Kn, Vn, _ = W.decode_stream(wl, T, drift_sigma=0.0)
    Qn = W.query_pool(wl, T)
    pkv = gc.make_ctx(wl, capacity=wl.n_tokens + T + 8)
    pkv.encode_keys(wl.n_tokens)
    n_r = wl.n_tokens - 4 - 512
    C = ok.coarse_count(n_r, wl.params.coarse_permille, wl.params.top_k)
    assert 4096 < C <= 8192        # eight candidates per thread in the fused launch
    _step_and_check(wl, pkv, Kn, Vn, Qn, {0, 255, 256}, [0, 13, 31], "graded")
    n, sink_end, r_end, buf = pkv.window()
    assert r_end == wl.n_tokens - 512 + 256 and buf == 2


def test_fused_fine_16_candidates_per_thread():
    """A coarse budget of 13004 candidates (20 % of 65020): the fused fine +
    hot-zone launch holds 16 candidates per thread.  Decode steps through an
    eviction, two units against the oracle."""
    T = 70
    wl = W.gqa_bf16(N=65536, top_k=2048, permille=200, buf_tokens=64)
    Kn, Vn, Qn = W.decode_stream(wl, T)
    pkv = gc.make_ctx(wl, capacity=wl.n_tokens + T)
    pkv.encode_keys(wl.n_tokens)
    C = ok.coarse_count(wl.n_tokens - 4 - 512, 200, 2048)
    assert 8192 < C <= 16384
    _step_and_check(wl, pkv, Kn, Vn, Qn, {0, 63, 64, 69}, [0, 6], "fused-seg16")


@pytest.mark.parametrize("n_sink,n_local", [(0, 0), (4, 0), (0, 64)])
def test_empty_sink_or_local_static(n_sink, n_local):
    """No sink and/or no local window (static context): with neither, attention
    runs over the retrieved keys alone."""
    wl = W.gqa_bf16(N=5000, top_k=256, n_sink=n_sink, n_local=n_local)
    pkv = gc.make_ctx(wl)
    pkv.encode_keys(wl.n_tokens)
    n, sink_end, r_end, _ = pkv.window()
    assert sink_end == n_sink and r_end == wl.n_tokens - n_local
    q = gc.queries(wl)
    sel, sel_n = pkv.retrieve(q)
    out = pkv.sparse_attend(q, sel, sel_n)
    torch.cuda.synchronize()
    units = [0, 5]
    enc = gc.check_encode(wl, pkv, units)
    gc.check_retrieval(wl, pkv, units, sel, sel_n, enc)
    gc.check_attention(wl, pkv, units, sel, sel_n, out)
    assert torch.isfinite(out).all()


def test_empty_sink_decode_steps():
    """No sink tokens, local 64 + update buffer 32: fused decode steps through
    two evictions."""
    T = 70
    wl = W.gqa_bf16(N=3000, top_k=256, n_sink=0, n_local=64, buf_tokens=32)
    Kn, Vn, Qn = W.decode_stream(wl, T)
    pkv = gc.make_ctx(wl, capacity=wl.n_tokens + T)
    pkv.encode_keys(wl.n_tokens)
    _step_and_check(wl, pkv, Kn, Vn, Qn, {0, 31, 32, 64, 69}, [0, 7], "no-sink")


@pytest.mark.parametrize("host_mapped", [False, True])
def test_prefill_shorter_than_sink(host_mapped):
    """A 2-token prefill with n_sink = 4: the sink zone holds 2 tokens and every
    appended token is local (with a host-memory store, kept in the device ring's
    local rows).  Decode steps until the local window overflows into the
    retrieval zone; every step's attention against the oracle, for a device
    store and for a host-memory store."""
    T = 44
    wl = W.gqa_bf16(N=2, top_k=8, permille=500, n_sink=4, n_local=16, buf_tokens=8)
    Kn, Vn, Qn = W.decode_stream(wl, T)
    pkv = gc.make_ctx(wl, capacity=wl.n_tokens + T, host_mapped=host_mapped)
    pkv.encode_keys(wl.n_tokens)
    assert pkv.window() == (2, 2, 2, 0)
    _step_and_check(wl, pkv, Kn, Vn, Qn, set(range(T)), [0, 3, 7], "short-prefill"
                    + ("-host" if host_mapped else ""))
    n, sink_end, r_end, _ = pkv.window()
    assert sink_end == 2 and r_end > sink_end      # the retrieval zone was reached


def test_binding_rejects_bad_output_buffers():
    """retrieve / decode_step / sparse_attend check caller-supplied sel, sel_n and
    out (shape, dtype, contiguity, device) before calling the library."""
    wl = W.gqa_bf16(N=3000, top_k=256, buf_tokens=16)
    pkv = gc.make_ctx(wl, capacity=wl.n_tokens + 4)
    pkv.encode_keys(wl.n_tokens)
    q = gc.queries(wl)
    kn = torch.zeros((wl.batch, wl.n_kv, 128), dtype=torch.bfloat16, device="cuda")
    good_sel = torch.empty((wl.batch, wl.n_kv, 256), dtype=torch.int32, device="cuda")
    good_n = torch.empty((wl.batch, wl.n_kv), dtype=torch.int32, device="cuda")
    bad_sels = [torch.empty((wl.batch, wl.n_kv, 128), dtype=torch.int32, device="cuda"),
                torch.empty((wl.batch, wl.n_kv, 256), dtype=torch.int64, device="cuda"),
                torch.empty((wl.batch, wl.n_kv, 256), dtype=torch.int32),
                torch.empty((wl.batch, wl.n_kv, 512), dtype=torch.int32, device="cuda")[..., ::2]]
    for bad in bad_sels:
        with pytest.raises(ValueError):
            pkv.retrieve(q, sel=bad, sel_n=good_n)
        with pytest.raises(ValueError):
            pkv.decode_step(kn, kn, q, sel=bad, sel_n=good_n)
        with pytest.raises(ValueError):
            pkv.sparse_attend(q, bad, good_n)
    with pytest.raises(ValueError):
        pkv.retrieve(q, sel=good_sel, sel_n=torch.empty((wl.batch, 4), dtype=torch.int32,
                                                         device="cuda"))
    for bad_out in (torch.empty((wl.batch, wl.n_kv * 4, 128), dtype=torch.bfloat16, device="cuda"),
                    torch.empty((wl.batch, wl.n_kv * 4, 64), dtype=torch.float32, device="cuda"),
                    torch.empty((wl.batch, wl.n_kv * 4, 128), dtype=torch.float32)):
        with pytest.raises(ValueError):
            pkv.decode_step(kn, kn, q, sel=good_sel, sel_n=good_n, out=bad_out)
        with pytest.raises(ValueError):
            pkv.dense_attend(q, out=bad_out)
    assert pkv.window() == (wl.n_tokens, 4, wl.n_tokens - 512, 0)   # nothing was appended
    out, sel, sel_n = pkv.decode_step(kn, kn, q, sel=good_sel, sel_n=good_n)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


def test_graph_replay_of_static_retrieval():
    """pk_retrieve + pk_sparse_attend on a static context captured into a HIP
    graph: every replay, with new queries copied into the captured query buffer
    between replays and eager library calls on the same context in between,
    gives the eager calls' selection and output bit for bit (the coarse-score
    histogram is a single device table the fine selection zeroes, so nothing
    host-chosen changes between steps).  One replay is also checked against the
    oracle."""
    wl = W.gqa_bf16(N=20011, batch=2, top_k=512)
    pkv = gc.make_ctx(wl)
    pkv.encode_keys(wl.n_tokens)
    pool_np = W.query_pool(wl, 4)
    pool = torch.from_numpy(pool_np).to(torch.bfloat16).cuda()
    q = torch.empty_like(pool[0])
    shp_sel = (wl.batch, wl.n_kv, wl.params.top_k)
    sel = torch.empty(shp_sel, dtype=torch.int32, device="cuda")
    sel_n = torch.empty(shp_sel[:2], dtype=torch.int32, device="cuda")
    out = torch.empty((wl.batch, wl.n_kv * wl.group, 128), dtype=torch.float32, device="cuda")
    refs = []
    for i in range(4):
        q.copy_(pool[i])
        pkv.retrieve(q, sel, sel_n)
        pkv.sparse_attend(q, sel, sel_n, out)
        torch.cuda.synchronize()
        refs.append((sel.clone(), sel_n.clone(), out.clone()))
    sel_g, n_g, out_g = torch.empty_like(sel), torch.empty_like(sel_n), torch.empty_like(out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pkv.retrieve(q, sel_g, n_g, stream=side)
        pkv.sparse_attend(q, sel_g, n_g, out_g, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        pkv.retrieve(q, sel_g, n_g, stream=st)
        pkv.sparse_attend(q, sel_g, n_g, out_g, stream=st)
    for rep in range(3):
        for i in range(4):
            q.copy_(pool[i])
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(sel_g, refs[i][0]) and torch.equal(n_g, refs[i][1]), (rep, i)
            assert torch.equal(out_g, refs[i][2]), (rep, i)
            pkv.retrieve(q, sel, sel_n)          # eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(sel, refs[i][0])
    wl.Q = pool_np[3]
    units = [0, 11]
    enc = gc.check_encode(wl, pkv, units)
    gc.check_retrieval(wl, pkv, units, sel_g, n_g, enc)
    gc.check_attention(wl, pkv, units, sel_g, n_g, out_g)
    del g
