"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, validates its arguments before touching a device, and computes the
same codebook as the oracle (bit-exact fp32 tables)."""
import ctypes
import os
import re

import numpy as np
import pytest

from tests.conftest import ROOT

nat = pytest.importorskip("kv_cache_top_amd._native", reason="libpariskv.so not built")
from oracle.codebook import spec_tables  # noqa: E402

HEADER = os.path.join(ROOT, "include", "pariskv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pk_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    fns = declared_functions()
    for name in ("pk_encode_keys", "pk_append_decode_keys", "pk_retrieve", "pk_sparse_attend"):
        assert name in fns


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(nat.LIB_PATH)
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, missing
    assert set(declared_functions()) == set(nat.SIGNATURES), "binding and header disagree"


def test_status_strings():
    for s in range(-6, 1):
        assert nat.lib.pk_status_string(s)
    assert nat.lib.pk_status_string(-99) == b"unknown status"


def test_library_codebook_matches_oracle_bit_exact():
    for kind in ("lloyd_max", "quantile"):
        for m in (4, 8, 16):
            lv, th = nat.codebook(m, kind)
            c32, T32 = spec_tables(m, kind=kind)
            assert np.array_equal(lv.view(np.uint32), c32.view(np.uint32)), (kind, m)
            assert np.array_equal(th.view(np.uint32), T32.view(np.uint32)), (kind, m)


def test_codebook_rejects_bad_arguments():
    lv = (ctypes.c_float * 8)()
    th = (ctypes.c_float * 7)()
    assert nat.lib.pk_codebook(1, 8, lv, th) == nat.PK_ERR_INVALID
    assert nat.lib.pk_codebook(8, 4, lv, th) == nat.PK_ERR_INVALID
    assert nat.lib.pk_codebook(8, 8, None, th) == nat.PK_ERR_INVALID


def _create(cfg, batch=1, n_kv=8, n_q=32, cap=1000, dtype=nat.PK_BF16, k=16, v=16, mem=0):
    ctx = ctypes.c_void_p()
    st = nat.lib.pk_create(ctypes.byref(cfg) if cfg is not None else None, batch, n_kv, n_q, cap,
                           dtype, ctypes.c_void_p(k), ctypes.c_void_p(v), mem, ctypes.byref(ctx))
    return st, ctx


@pytest.mark.parametrize("field,value,expect", [
    ("head_dim", 64, nat.PK_ERR_UNSUPPORTED),
    ("n_sub", 8, nat.PK_ERR_INVALID),            # B * m != d
    ("sub_dim", 16, nat.PK_ERR_INVALID),
    ("rho", 0, nat.PK_ERR_INVALID),
    ("rho", 9, nat.PK_ERR_INVALID),
    ("coarse_permille", 0, nat.PK_ERR_INVALID),
    ("coarse_permille", 1001, nat.PK_ERR_INVALID),
    ("top_k", 0, nat.PK_ERR_INVALID),
    ("n_sink", -1, nat.PK_ERR_INVALID),
    ("buf_tokens", 600, nat.PK_ERR_INVALID),     # larger than n_local
])
def test_create_validates_config(field, value, expect):
    cfg = nat.make_config()
    setattr(cfg, field, value)
    st, ctx = _create(cfg)
    assert st == expect and not ctx.value


def test_create_validates_shapes_and_pointers():
    cfg = nat.make_config()
    assert _create(None)[0] == nat.PK_ERR_INVALID
    assert _create(cfg, batch=0)[0] == nat.PK_ERR_INVALID
    assert _create(cfg, n_q=30)[0] == nat.PK_ERR_INVALID          # not a multiple of n_kv
    assert _create(cfg, n_q=8 * 3)[0] == nat.PK_ERR_UNSUPPORTED   # G = 3
    assert _create(cfg, n_q=8 * 32)[0] == nat.PK_ERR_INVALID      # G = 32
    assert _create(cfg, cap=0)[0] == nat.PK_ERR_INVALID
    assert _create(cfg, cap=(1 << 24) + 1)[0] == nat.PK_ERR_UNSUPPORTED
    assert _create(cfg, batch=70000, n_kv=1, n_q=4)[0] == nat.PK_ERR_UNSUPPORTED   # units > 65535
    assert _create(cfg, batch=1 << 20, n_kv=1 << 12, n_q=1 << 14)[0] == nat.PK_ERR_UNSUPPORTED
    assert _create(cfg, dtype=7)[0] == nat.PK_ERR_INVALID
    assert _create(cfg, k=0)[0] == nat.PK_ERR_INVALID
    assert _create(cfg, k=24)[0] == nat.PK_ERR_INVALID            # not 16-byte aligned
    assert _create(cfg, mem=5)[0] == nat.PK_ERR_INVALID
    big = nat.make_config(vote_weights=(200, 1, 1, 1))
    assert _create(big)[0] == nat.PK_ERR_INVALID                  # G * weight > 255
    zero = nat.make_config(vote_weights=(4, 3, 0, 1))
    assert _create(zero)[0] == nat.PK_ERR_INVALID
    # subspace widths: m = 4, 8 and 16 are built, m = 2 (B = 64) is valid but not built
    assert _create(nat.make_config(n_sub=64, sub_dim=2))[0] == nat.PK_ERR_UNSUPPORTED
    # m = 4: a vote-table byte sums two subspaces' votes, so 2 * G * weight <= 255
    assert _create(nat.make_config(n_sub=32, sub_dim=4, vote_weights=(32, 1, 1, 1)))[0] == \
        nat.PK_ERR_INVALID


def test_calls_reject_null_context():
    p = ctypes.c_void_p(16)
    assert nat.lib.pk_encode_keys(None, 10, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_append_decode_keys(None, p, p, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_retrieve(None, p, p, p, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_sparse_attend(None, p, p, p, p, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_dense_attend(None, p, p, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_fit_centroids(None, 4096, p, 3, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_decode_step(None, p, p, p, p, p, p, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_debug_copy(None, 0, p, 1, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_debug_size(None, 0) == 0
    nat.lib.pk_destroy(None)


def test_measurement_references_validate_arguments():
    p, i = ctypes.c_void_p(16), ctypes.c_void_p(64)
    assert nat.lib.pk_stream_read(None, 16, p, None, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_stream_read(ctypes.c_void_p(24), 16, p, None, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_stream_read(p, 24, p, None, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_gather_read(None, 10, 128, i, 4, p, None, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_gather_read(p, 10, 128, None, 4, p, None, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_gather_read(ctypes.c_void_p(24), 10, 128, i, 4, p, None, None) == nat.PK_ERR_INVALID
    for rb in (0, 8, 24, 2048):
        assert nat.lib.pk_gather_read(p, 10, rb, i, 4, p, None, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_gather_read(p, 0, 128, i, 4, p, None, None) == nat.PK_ERR_INVALID
    assert nat.lib.pk_gather_read(p, 10, 128, i, 0, p, None, None) == nat.PK_ERR_INVALID


def test_no_device_is_reported_without_a_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, ctx = _create(nat.make_config())
    assert st == nat.PK_ERR_NO_DEVICE and not ctx.value
    st, ctx = _create(nat.make_config(n_sub=32, sub_dim=4, vote_weights=(31, 1, 1, 1)))
    assert st == nat.PK_ERR_NO_DEVICE and not ctx.value   # a valid m = 4 configuration
    st, ctx = _create(nat.make_config(n_sub=8, sub_dim=16, vote_weights=(63, 1, 1, 1)))
    assert st == nat.PK_ERR_NO_DEVICE and not ctx.value   # a valid m = 16 configuration


def test_noalloc_entry_point_validates_without_a_device():
    """pk_dense_attend_noalloc refuses a null context before any device work, and
    reports the size of its scratch array."""
    assert nat.lib.pk_noalloc_scratch_bytes() == 64 << 20
    assert nat.lib.pk_dense_attend_noalloc(None, None, None, None) == nat.PK_ERR_INVALID
