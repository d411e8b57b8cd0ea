"""ctypes binding of libpariskv.so (the C ABI in include/pariskv.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of the library.  torch supplies device memory and streams.  There is
no fallback: if the library is missing or fails to load, importing this
module raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpariskv.so")

PK_OK, PK_ERR_INVALID, PK_ERR_NO_DEVICE, PK_ERR_OOM, PK_ERR_CAPACITY, PK_ERR_HIP, \
    PK_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
PK_F32, PK_BF16 = 0, 1
PK_MEM_DEVICE, PK_MEM_HOST_MAPPED = 0, 1
STAGES = ("encode", "append", "qprep", "scan", "select", "rerank", "fine", "attend", "combine")
(PK_DBG_IDS, PK_DBG_REC, PK_DBG_LUT, PK_DBG_SCORES, PK_DBG_CAND, PK_DBG_EST,
 PK_DBG_NCAND, PK_DBG_CENTROIDS) = range(8)

# every function the header declares, with its ctypes signature
_c_void_p, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


class PkConfig(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("n_sub", ctypes.c_int32),
        ("sub_dim", ctypes.c_int32),
        ("rho", ctypes.c_int32),
        ("vote_weight", ctypes.c_uint8 * 8),
        ("coarse_permille", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_sink", ctypes.c_int32),
        ("n_local", ctypes.c_int32),
        ("buf_tokens", ctypes.c_int32),
        ("sign_bits", ctypes.c_uint64 * 2),
        ("codebook", ctypes.c_int32),
    ]


SIGNATURES = {
    "pk_create": (_i32, [ctypes.POINTER(PkConfig), _i32, _i32, _i32, _i64, _i32, _c_void_p,
                         _c_void_p, _i32, ctypes.POINTER(_c_void_p)]),
    "pk_destroy": (None, [_c_void_p]),
    "pk_encode_keys": (_i32, [_c_void_p, _i64, _c_void_p]),
    "pk_append_decode_keys": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "pk_retrieve": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "pk_sparse_attend": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                _c_void_p]),
    "pk_decode_step": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                              _c_void_p, _c_void_p]),
    "pk_dense_attend": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "pk_dense_attend_noalloc": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "pk_noalloc_scratch_bytes": (_sz, []),
    "pk_fit_centroids": (_i32, [_c_void_p, _i64, _c_void_p, _i32, _c_void_p]),
    "pk_codebook": (_i32, [_i32, _i32, ctypes.POINTER(ctypes.c_float),
                           ctypes.POINTER(ctypes.c_float)]),
    "pk_codebook_quantile": (_i32, [_i32, _i32, ctypes.POINTER(ctypes.c_float),
                                    ctypes.POINTER(ctypes.c_float)]),
    "pk_status_string": (ctypes.c_char_p, [_i32]),
    "pk_get_window": (_i32, [_c_void_p, ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                             ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "pk_profile_enable": (_i32, [_c_void_p, _i32]),
    "pk_profile_read": (_i32, [_c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    "pk_debug_size": (_sz, [_c_void_p, _i32]),
    "pk_debug_copy": (_i32, [_c_void_p, _i32, _c_void_p, _sz, _c_void_p]),
    "pk_stream_read": (_i32, [_c_void_p, _sz, _c_void_p, ctypes.POINTER(ctypes.c_float),
                              _c_void_p]),
    "pk_gather_read": (_i32, [_c_void_p, _i64, _i32, _c_void_p, _i64, _c_void_p,
                              ctypes.POINTER(ctypes.c_float), _c_void_p]),
}


def _preload_torch_hip_runtime():
    """The library takes torch's device pointers and streams, so the process
    must hold one HIP runtime: torch's.  Its bundled libamdhip64 has the same
    soname as the system one, so loading it first (globally) makes the
    dynamic linker bind libpariskv.so to it."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        return
    hip = os.path.join(os.path.dirname(spec.origin), "lib", "libamdhip64.so")
    if os.path.exists(hip):
        ctypes.CDLL(hip, mode=ctypes.RTLD_GLOBAL)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python kv_cache_top_amd/build.py)")
    _preload_torch_hip_runtime()
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class PkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.pk_status_string(status).decode()} ({status})")


def check(status: int, where: str) -> None:
    if status != PK_OK:
        raise PkError(status, where)


def codebook(sub_dim: int = 8, kind: str = "lloyd_max"):
    """(levels fp32[8], squared thresholds fp32[7]) as computed by the library (host
    only); kind "lloyd_max" (pk_codebook) or "quantile" (pk_codebook_quantile)."""
    import numpy as np
    lv = (ctypes.c_float * 8)()
    th = (ctypes.c_float * 7)()
    fn = lib.pk_codebook if kind == "lloyd_max" else lib.pk_codebook_quantile
    check(fn(sub_dim, 8, lv, th), "pk_codebook")
    return np.array(lv[:], np.float32), np.array(th[:], np.float32)


def make_config(*, rho=4, vote_weights=(4, 3, 2, 1), coarse_permille=50, top_k=2048, n_sink=4,
                n_local=512, buf_tokens=0, sign_bits=(0, 0), head_dim=128, n_sub=16,
                sub_dim=8, codebook=0) -> PkConfig:
    cfg = PkConfig()
    cfg.head_dim, cfg.n_sub, cfg.sub_dim, cfg.rho = head_dim, n_sub, sub_dim, rho
    for i in range(8):
        cfg.vote_weight[i] = int(vote_weights[i]) if i < len(vote_weights) else 0
    cfg.coarse_permille, cfg.top_k = coarse_permille, top_k
    cfg.n_sink, cfg.n_local, cfg.buf_tokens = n_sink, n_local, buf_tokens
    cfg.sign_bits[0], cfg.sign_bits[1] = int(sign_bits[0]), int(sign_bits[1])
    cfg.codebook = codebook
    return cfg
