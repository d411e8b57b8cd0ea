"""Python front end of the ParisKV decode path on MI355X.

`ParisKV` owns a library context over a K/V store.  torch allocates the store
and the outputs and supplies the current HIP stream; every computation runs
in libpariskv.so's kernels.  There is no CPU fallback.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _native as nat


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_DT = {torch.float32: nat.PK_F32, torch.bfloat16: nat.PK_BF16}


class ParisKV:
    """One layer's KV cache with ParisKV retrieval.

    Stores are [batch, n_kv, capacity, 128] in `dtype`; pass your own (device,
    or pinned host memory with host_mapped=True) or let the class allocate
    device ones.  Queries are [batch, n_q, 128] in the same dtype.
    """

    def __init__(self, *, batch: int, n_kv: int, n_q: int, capacity: int,
                 dtype: torch.dtype = torch.bfloat16, config: nat.PkConfig | None = None,
                 k_store: torch.Tensor | None = None, v_store: torch.Tensor | None = None,
                 host_mapped: bool = False, device: str | torch.device = "cuda", **cfg_kw):
        if not torch.cuda.is_available():
            raise RuntimeError("ParisKV needs a ROCm GPU (gfx950); no device is visible")
        if dtype not in _DT:
            raise ValueError(f"unsupported dtype {dtype}")
        self.cfg = config if config is not None else nat.make_config(**cfg_kw)
        self.batch, self.n_kv, self.n_q, self.capacity, self.dtype = batch, n_kv, n_q, capacity, dtype
        self.group = n_q // n_kv
        shape = (batch, n_kv, capacity, 128)

        def alloc():
            if host_mapped:   # pinned host memory, addressable by the device
                return torch.empty(shape, dtype=dtype, pin_memory=True)
            return torch.empty(shape, dtype=dtype, device=device)
        if k_store is None:
            k_store = alloc()
        if v_store is None:
            v_store = alloc()
        for t in (k_store, v_store):
            if tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous():
                raise ValueError(f"store must be a contiguous {dtype} tensor of shape {shape}")
            if host_mapped and (t.device.type != "cpu" or not t.is_pinned()):
                raise ValueError("host_mapped stores must be pinned host tensors")
            if not host_mapped and t.device.type != "cuda":
                raise ValueError("device stores must be GPU tensors")
        self.K, self.V = k_store, v_store
        self.device = torch.device(device)
        self._ctx = ctypes.c_void_p()
        nat.check(nat.lib.pk_create(ctypes.byref(self.cfg), batch, n_kv, n_q, capacity, _DT[dtype],
                                    _ptr(k_store), _ptr(v_store),
                                    nat.PK_MEM_HOST_MAPPED if host_mapped else nat.PK_MEM_DEVICE,
                                    ctypes.byref(self._ctx)), "pk_create")
        self._decode_fn = nat.lib.pk_decode_step

    # -- lifecycle ---------------------------------------------------------
    def close(self) -> None:
        if self._ctx:
            nat.lib.pk_destroy(self._ctx)
            self._ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- the four calls of the decode path ----------------------------------
    def encode_keys(self, n_tokens: int, stream=None) -> None:
        nat.check(nat.lib.pk_encode_keys(self._ctx, n_tokens, _stream(stream)), "pk_encode_keys")

    def fit_centroids(self, n_tokens: int, init_pos: torch.Tensor, iters: int, stream=None) -> None:
        """Learned-centroid comparison stage (pk_fit_centroids): k-means tables from
        the first n_tokens stored keys; call before encode_keys.  init_pos: device
        int32 [batch * n_kv, 256] initial positions."""
        if (init_pos.dtype != torch.int32 or init_pos.device.type != "cuda"
                or tuple(init_pos.shape) != (self.batch * self.n_kv, 256) or not init_pos.is_contiguous()):
            raise ValueError("init_pos must be a contiguous cuda int32 tensor [units, 256]")
        nat.check(nat.lib.pk_fit_centroids(self._ctx, n_tokens, _ptr(init_pos), iters, _stream(stream)),
                  "pk_fit_centroids")

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
        self._check_rows(k_new, (self.batch, self.n_kv, 128))
        self._check_rows(v_new, (self.batch, self.n_kv, 128))
        nat.check(nat.lib.pk_append_decode_keys(self._ctx, _ptr(k_new), _ptr(v_new), _stream(stream)),
                  "pk_append_decode_keys")

    def retrieve(self, q: torch.Tensor, sel: torch.Tensor | None = None,
                 sel_n: torch.Tensor | None = None, stream=None):
        self._check_rows(q, (self.batch, self.n_q, 128))
        if sel is None:
            sel = torch.empty((self.batch, self.n_kv, self.cfg.top_k), dtype=torch.int32, device=q.device)
        if sel_n is None:
            sel_n = torch.empty((self.batch, self.n_kv), dtype=torch.int32, device=q.device)
        self._check_sel(sel, sel_n)
        nat.check(nat.lib.pk_retrieve(self._ctx, _ptr(q), _ptr(sel), _ptr(sel_n), _stream(stream)),
                  "pk_retrieve")
        return sel, sel_n

    def sparse_attend(self, q: torch.Tensor, sel: torch.Tensor, sel_n: torch.Tensor,
                      out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        self._check_rows(q, (self.batch, self.n_q, 128))
        self._check_sel(sel, sel_n)
        if out is None:
            out = torch.empty((self.batch, self.n_q, 128), dtype=torch.float32, device=q.device)
        self._check_out(out)
        nat.check(nat.lib.pk_sparse_attend(self._ctx, _ptr(q), _ptr(sel), _ptr(sel_n), _ptr(out),
                                           _stream(stream)), "pk_sparse_attend")
        return out

    def dense_attend(self, q: torch.Tensor, out: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
        """Full attention over every stored token (pk_dense_attend): the dense
        decode attention the retrieval replaces, for comparison."""
        self._check_rows(q, (self.batch, self.n_q, 128))
        if out is None:
            out = torch.empty((self.batch, self.n_q, 128), dtype=torch.float32, device=q.device)
        self._check_out(out)
        nat.check(nat.lib.pk_dense_attend(self._ctx, _ptr(q), _ptr(out), _stream(stream)),
                  "pk_dense_attend")
        return out

    def step(self, q: torch.Tensor, stream=None):
        """Retrieve then attend; returns (out, sel, sel_n)."""
        sel, sel_n = self.retrieve(q, stream=stream)
        return self.sparse_attend(q, sel, sel_n, stream=stream), sel, sel_n

    def decode_step(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                    sel: torch.Tensor | None = None, sel_n: torch.Tensor | None = None,
                    out: torch.Tensor | None = None, stream=None):
        """Append the new token, retrieve and attend in one call (pk_decode_step);
        returns (out, sel, sel_n)."""
        self._check_rows(k_new, (self.batch, self.n_kv, 128))
        self._check_rows(v_new, (self.batch, self.n_kv, 128))
        self._check_rows(q, (self.batch, self.n_q, 128))
        dev = q.device
        if sel is None:
            sel = torch.empty((self.batch, self.n_kv, self.cfg.top_k), dtype=torch.int32, device=dev)
        if sel_n is None:
            sel_n = torch.empty((self.batch, self.n_kv), dtype=torch.int32, device=dev)
        if out is None:
            out = torch.empty((self.batch, self.n_q, 128), dtype=torch.float32, device=dev)
        self._check_sel(sel, sel_n)
        self._check_out(out)
        nat.check(nat.lib.pk_decode_step(self._ctx, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(sel),
                                         _ptr(sel_n), _ptr(out), _stream(stream)), "pk_decode_step")
        return out, sel, sel_n

    def decode_step_raw(self, k_new: int, v_new: int, q: int, sel: int, sel_n: int, out: int,
                        stream: int) -> None:
        """pk_decode_step on raw device addresses and a raw hipStream_t (no
        checks): for callers that validated their buffers once and issue many
        steps, where per-call tensor handling would cost more than the launch."""
        nat.check(self._decode_fn(self._ctx, k_new, v_new, q, sel, sel_n, out, stream),
                  "pk_decode_step")

    def profile(self, on: bool = True) -> None:
        """Start (or stop) per-stage kernel timing with HIP events."""
        nat.check(nat.lib.pk_profile_enable(self._ctx, 1 if on else 0), "pk_profile_enable")

    def profile_read(self) -> dict:
        """{stage: (total_ms, launches)} since profiling was enabled."""
        n = len(nat.STAGES)
        ms = (ctypes.c_double * n)()
        ln = (ctypes.c_int64 * n)()
        nat.check(nat.lib.pk_profile_read(self._ctx, ms, ln), "pk_profile_read")
        return {name: (ms[i], ln[i]) for i, name in enumerate(nat.STAGES)}

    # -- introspection -------------------------------------------------------
    def window(self):
        vals = [ctypes.c_int64() for _ in range(4)]
        nat.check(nat.lib.pk_get_window(self._ctx, *[ctypes.byref(v) for v in vals]), "pk_get_window")
        return tuple(v.value for v in vals)   # (n_tokens, sink_end, r_end, buf)

    _DBG_DTYPE = {nat.PK_DBG_IDS: np.uint8, nat.PK_DBG_REC: np.uint8, nat.PK_DBG_LUT: np.uint8,
                  nat.PK_DBG_SCORES: np.uint8, nat.PK_DBG_CAND: np.int32, nat.PK_DBG_EST: np.float32,
                  nat.PK_DBG_NCAND: np.int32, nat.PK_DBG_CENTROIDS: np.float32}

    def debug(self, what: int, stream=None) -> np.ndarray:
        n = nat.lib.pk_debug_size(self._ctx, what)
        buf = np.empty(n, np.uint8)
        nat.check(nat.lib.pk_debug_copy(self._ctx, what, buf.ctypes.data_as(ctypes.c_void_p), n,
                                        _stream(stream)), "pk_debug_copy")
        arr = buf.view(self._DBG_DTYPE[what])
        units = self.batch * self.n_kv
        return arr.reshape(units, -1)

    def _check_sel(self, sel: torch.Tensor, sel_n: torch.Tensor):
        """The kernels write top_k positions per unit into sel and a count per unit
        into sel_n: both must be contiguous device int32 tensors of exactly that size."""
        for t, shape, name in ((sel, (self.batch, self.n_kv, self.cfg.top_k), "sel"),
                               (sel_n, (self.batch, self.n_kv), "sel_n")):
            if (t.dtype != torch.int32 or tuple(t.shape) != shape or not t.is_contiguous()
                    or t.device.type != "cuda"):
                raise ValueError(f"{name} must be a contiguous cuda int32 tensor of shape {shape}, "
                                 f"got {tuple(t.shape)} {t.dtype} on {t.device}")

    def _check_out(self, out: torch.Tensor):
        shape = (self.batch, self.n_q, 128)
        if (out.dtype != torch.float32 or tuple(out.shape) != shape or not out.is_contiguous()
                or out.device.type != "cuda"):
            raise ValueError(f"out must be a contiguous cuda float32 tensor of shape {shape}, "
                             f"got {tuple(out.shape)} {out.dtype} on {out.device}")

    def _check_rows(self, t: torch.Tensor, shape):
        if tuple(t.shape) != shape or t.dtype != self.dtype or not t.is_contiguous():
            raise ValueError(f"expected a contiguous {self.dtype} tensor of shape {shape}, "
                             f"got {tuple(t.shape)} {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError("inputs must be device tensors")
