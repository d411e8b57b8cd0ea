"""pk_dense_attend_noalloc: the dense attention with its split partials in the
library's static device scratch array instead of memory allocated on first
use.  Called through the C ABI and checked against pk_dense_attend on two calls
in a row (the second over a smaller context), against the oracle on sampled
units, and for its size limit."""
import ctypes

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


def _noalloc(nat, pkv, q, out):
    st = torch.cuda.current_stream().cuda_stream
    return nat.lib.pk_dense_attend_noalloc(pkv._ctx, ctypes.c_void_p(q.data_ptr()),
                                           ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st))


def test_noalloc_dense_attention_matches_allocating_call():
    import kv_cache_top_amd._native as nat
    assert nat.lib.pk_noalloc_scratch_bytes() == 64 << 20
    for tag, wl, units in (("larger", W.gqa_bf16(N=20011, batch=2, top_k=512), [0, 15]),
                           ("smaller", W.gqa_bf16(N=3001, batch=1, top_k=256), [2])):
        pkv = gc.make_ctx(wl)
        pkv.encode_keys(wl.n_tokens)
        q = gc.queries(wl)
        ref = pkv.dense_attend(q)
        out = torch.full_like(ref, float("nan"))
        gc.log(f"[no-alloc] {tag}: {wl.n_units} units x {wl.n_tokens} tokens")
        assert _noalloc(nat, pkv, q, out) == nat.PK_OK
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{tag}: differs from pk_dense_attend"
        o = out.cpu().numpy().reshape(wl.n_units, wl.group, 128)
        for u in units:
            K, V, Qg = gc.unit_view(wl, u)
            want = ok.sparse_attention(Qg, K, V, np.arange(wl.n_tokens))
            err = float(np.max(np.abs(o[u] - want)))
            assert err <= gc.ATT_TOL[wl.dtype], f"{tag}, unit {u}: max-abs {err:.3g}"
        pkv.close()


def test_noalloc_rejects_partials_beyond_the_scratch():
    """32 units x 4 heads x 1024 splits of 130 floats is 68.2 MB > 64 MiB: refused
    with PK_ERR_CAPACITY before any launch; a fitting call works afterwards."""
    import kv_cache_top_amd._native as nat
    from kv_cache_top_amd import ParisKV
    N = 131072
    pkv = ParisKV(batch=4, n_kv=8, n_q=32, capacity=N, dtype=torch.bfloat16, top_k=2048,
                  n_local=512, sign_bits=(1, 2))
    pkv.K.zero_()
    pkv.V.zero_()
    pkv.encode_keys(N)
    q = torch.zeros((4, 32, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((4, 32, 128), dtype=torch.float32, device="cuda")
    assert _noalloc(nat, pkv, q, out) == nat.PK_ERR_CAPACITY
    pkv.close()
    wl = W.gqa_bf16(N=4096, batch=1, top_k=256)
    small = gc.make_ctx(wl)
    small.encode_keys(wl.n_tokens)
    q = gc.queries(wl)
    ref = small.dense_attend(q)
    out = torch.empty_like(ref)
    assert _noalloc(nat, small, q, out) == nat.PK_OK
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
