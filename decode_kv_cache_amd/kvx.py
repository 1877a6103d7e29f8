"""Thin ctypes binding of libkvx (C ABI: include/kvx.h).

Argument marshalling only: every step of the transfer runs in libkvx's HIP
kernels; torch supplies device memory (``data_ptr()``), streams
(``cuda_stream``) and events (``cuda_event``).  The Python names are the C
names.  A failing call raises :class:`KvxError` with the C status and
``kvx_last_error()``.  If ``libkvx.so`` has not been built the first call
raises; nothing falls back to another implementation.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np
import torch  # imported before libkvx so that both share torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvx.so")

KVX_OK, KVX_E_INVAL, KVX_E_RANGE, KVX_E_DUPDST, KVX_E_MISMATCH, KVX_E_UNSUPPORTED, KVX_E_NOMEM, KVX_E_HIP = range(8)
KVX_NHD, KVX_HND = 0, 1
KVX_PLAN_HOST_ONLY = 1
KVX_PLAN_OVERLAP = 2
KVX_PLAN_RUNS = 4
LAYOUTS = {"NHD": KVX_NHD, "HND": KVX_HND}


class kvx_pool_desc(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("num_blocks", C.c_int32), ("block_size", C.c_int32),
                ("num_heads", C.c_int32), ("head_dim", C.c_int32), ("elem_bytes", C.c_int32),
                ("layout", C.c_int32), ("k_base", C.POINTER(C.c_void_p)), ("v_base", C.POINTER(C.c_void_p)),
                ("k_scale", C.POINTER(C.c_void_p)), ("v_scale", C.POINTER(C.c_void_p)),
                ("sliding_window", C.c_int32)]


class kvx_state_pool_desc(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("num_slots", C.c_int32), ("slot_bytes", C.c_int64 * 2),
                ("base", C.POINTER(C.c_void_p) * 2)]


class kvx_run(C.Structure):
    _fields_ = [("src0", C.c_int32), ("dst0", C.c_int32), ("nblk", C.c_int32), ("tail", C.c_int32)]


class kvx_launch_shape(C.Structure):
    _fields_ = [("pieces", C.c_int64), ("piece_bytes", C.c_int32), ("lanes", C.c_int32), ("vectors", C.c_int32),
                ("run_table", C.c_int32)]


class kvx_triple(C.Structure):
    _fields_ = [("src_off", C.c_int64), ("dst_off", C.c_int64), ("len", C.c_int64)]


_P = C.c_void_p
_I32, _I64, _U32 = C.c_int32, C.c_int64, C.c_uint32
_SIGS = {
    "kvx_abi_version": (_I32, []),
    "kvx_status_str": (C.c_char_p, [C.c_int]),
    "kvx_last_error": (C.c_char_p, []),
    "kvx_tokens_to_move": (_I64, [_I64, _I64]),
    "kvx_should_reuse": (_I32, [_I64, _I64]),
    "kvx_pool_create": (C.c_int, [C.POINTER(kvx_pool_desc), C.POINTER(_P)]),
    "kvx_state_pool_create": (C.c_int, [C.POINTER(kvx_state_pool_desc), C.POINTER(_P)]),
    "kvx_pool_destroy": (None, [_P]),
    "kvx_plan": (C.c_int, [_P, _P, _I32, _P, _P, _P, _P, _P, _U32, _P, C.POINTER(_P)]),
    "kvx_plan_noalloc": (C.c_int, [_P, _P, _I32, _P, _P, _P, _P, _P, _U32, _P, C.POINTER(_P)]),
    "kvx_plan_runs": (C.c_int, [_P, _P, _I64, C.POINTER(_I64)]),
    "kvx_plan_triples": (C.c_int, [_P, _I32, _I32, _P, _I64, C.POINTER(_I64)]),
    "kvx_plan_bytes": (C.c_int, [_P, C.POINTER(_I64), C.POINTER(_I64)]),
    "kvx_plan_launch_shape": (C.c_int, [_P, C.POINTER(kvx_launch_shape)]),
    "kvx_plan_wait": (C.c_int, [_P]),
    "kvx_plan_destroy_after": (C.c_int, [_P, _P]),
    "kvx_plan_reclaim": (C.c_int, [_I32, C.POINTER(_I64)]),
    "kvx_plan_destroy": (None, [_P]),
    "kvx_push_layer": (C.c_int, [_P, _I32, _P, _P]),
    "kvx_push_layer_timed": (C.c_int, [_P, _I32, _P, _P, _P, _P]),
    "kvx_push_many": (C.c_int, [_P, _P, _I32, _P, _P]),
    "kvx_push_many_timed": (C.c_int, [_P, _P, _I32, _P, _P, _P, _P]),
    "kvx_staging_bytes": (C.c_int, [_P, _I32, _I32, C.POINTER(_I64)]),
    "kvx_pack": (C.c_int, [_P, _I32, _I32, _P, _I64, _P]),
    "kvx_unpack": (C.c_int, [_P, _I32, _I32, _P, _I64, _P]),
    "kvx_copy_heads": (C.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P]),
    "kvx_copy_heads_layers": (C.c_int, [_P, _I32, _I32, _I32, _I32, _I32, _P, _P]),
    "kvx_queue_create": (C.c_int, [_P, C.POINTER(_P)]),
    "kvx_queue_push": (C.c_int, [_P, _P, _I32, _P]),
    "kvx_queue_push_heads": (C.c_int, [_P, _P, _I32, _I32, _I32, _I32, _P]),
    "kvx_queue_flush": (C.c_int, [_P]),
    "kvx_queue_stats": (C.c_int, [_P, C.POINTER(_I64), C.POINTER(_I64), C.POINTER(_I64)]),
    "kvx_queue_destroy": (C.c_int, [_P]),
}
_D = C.c_double
_U64 = C.c_uint64
_SIGS.update({
    "kvx_xfer_create": (C.c_int, [_P, _P, _P, C.POINTER(_P)]),
    "kvx_xfer_destroy": (None, [_P]),
    "kvx_xfer_register": (C.c_int, [_P, _U64, _U32, _P, _P, _I64, _D, C.POINTER(_I32)]),
    "kvx_xfer_prefill": (C.c_int, [_P, _U64, _U32, _I64, _P, _I64, _D, C.POINTER(_I32)]),
    "kvx_xfer_save_layer": (C.c_int, [_P, _U64, _U32, _I32, _P, _D, C.POINTER(_I32)]),
    "kvx_xfer_save_layer_many": (C.c_int, [_P, _I32, _P, _I64, _P, _P, _D, _P]),
    "kvx_xfer_seal": (C.c_int, [_P, _U64, _U32, C.POINTER(_I32)]),
    "kvx_xfer_poll": (C.c_int, [_P, _D]),
    "kvx_xfer_complete": (C.c_int, [_P, _U64, _U32, _I32, _I32]),
    "kvx_xfer_status": (C.c_int, [_P, _U64, C.POINTER(_U32), C.POINTER(_I32)]),
    "kvx_xfer_pop_finished": (C.c_int, [_P, _P, _P, _P, _I64, C.POINTER(_I64)]),
    "kvx_xfer_recompute_blocks": (C.c_int, [_P, _U64, _P, _I64, C.POINTER(_I64)]),
    "kvx_xfer_issued": (C.c_int, [_P, _I64, _P, _P, _P, _I64, C.POINTER(_I64)]),
    "kvx_xfer_forget": (C.c_int, [_P, _U64]),
})
EXPORTED = tuple(_SIGS)
KVX_REQ_PENDING, KVX_REQ_DONE, KVX_REQ_FAILED, KVX_REQ_EXPIRED = range(4)
KVX_XFER_HOST_ONLY = 1
KVX_XFER_LOG = 2


class kvx_xfer_config(C.Structure):
    _fields_ = [("defer_timeout_s", C.c_double), ("transfer_timeout_s", C.c_double), ("flags", C.c_uint32)]

_lib = None


def lib() -> C.CDLL:
    """Load libkvx.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decode_kv_cache_amd.build`")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


class KvxError(RuntimeError):
    def __init__(self, fn: str, code: int):
        L = lib()
        self.code = code
        self.status = L.kvx_status_str(code).decode()
        self.detail = L.kvx_last_error().decode()
        super().__init__(f"{fn}: {self.status}: {self.detail}")


def _check(fn: str, rc: int) -> None:
    if rc != KVX_OK:
        raise KvxError(fn, rc)


def _stream(s) -> Optional[int]:
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _event(e) -> Optional[int]:
    if e is None:
        return None
    if isinstance(e, int):
        return e or None
    return e.cuda_event or None


def kvx_abi_version() -> int:
    return lib().kvx_abi_version()


def kvx_tokens_to_move(prompt_len: int, num_computed: int = 0) -> int:
    return lib().kvx_tokens_to_move(prompt_len, num_computed)


def kvx_should_reuse(reusable_tokens: int, threshold: int) -> bool:
    return bool(lib().kvx_should_reuse(reusable_tokens, threshold))


def _require_device_tensor(fn: str, what: str, t, dtype) -> None:
    """Refuse what the kernels cannot address safely: a host tensor, a tensor
    on another device than the current one, a strided view (its span is not
    numel x element size) or the wrong element type."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{fn}: {what} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{fn}: {what} is a host tensor; the kernels need device memory")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{fn}: {what} lives on cuda:{t.device.index}, the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{fn}: {what} must be {dtype}, got {t.dtype}")


class Pool:
    """Owns a kvx_pool handle.  ``k_bases``/``v_bases``: one device address per
    logical layer (may repeat; ``v_bases`` None for a pool of one latent
    region); ``k_scales``/``v_scales``: fp32[num_blocks] addresses per layer
    or None.  ``keep`` holds tensors alive with the pool."""

    def __init__(self, *, num_blocks, block_size, num_heads, head_dim, elem_bytes, layout,
                 k_bases: Sequence[int], v_bases: Optional[Sequence[int]], k_scales=None, v_scales=None,
                 sliding_window: int = 0, keep=()):
        L = len(k_bases)
        arr = C.c_void_p * L
        self._kb = arr(*k_bases)
        self._vb = arr(*v_bases) if v_bases is not None else None
        self._ks = arr(*k_scales) if k_scales is not None else None
        self._vs = arr(*v_scales) if v_scales is not None else None
        d = kvx_pool_desc(L, num_blocks, block_size, num_heads, head_dim, elem_bytes,
                          LAYOUTS.get(layout, layout), self._kb, self._vb, self._ks, self._vs, sliding_window)
        h = C.c_void_p()
        _check("kvx_pool_create", lib().kvx_pool_create(C.byref(d), C.byref(h)))
        self.handle, self._L = h, lib()
        self.num_layers, self.num_blocks, self.block_size = L, num_blocks, block_size
        self.num_heads, self.head_dim, self.elem_bytes = num_heads, head_dim, elem_bytes
        self.layout = layout
        self.regions = 1 if v_bases is None else 2
        self.sliding_window = sliding_window
        self.keep = keep

    def close(self):
        if getattr(self, "handle", None):
            self._L.kvx_pool_destroy(self.handle)
            self.handle = None

    __del__ = close


def kvx_pool_create(*, kv, scales=None, num_layers: int, num_blocks: int, block_size: int,
                    num_heads: int, head_dim: int, elem_bytes: int, layout="NHD", phys=None,
                    sliding_window: int = 0) -> Pool:
    """Register a pool stored as one tensor ``kv`` of shape [P, R, region]
    (P physical layer slabs; R = 2 regions K then V, or R = 1 latent region)
    with optional fp32 ``scales`` of shape [P, R, num_blocks].  Logical layer
    l uses slab ``phys(l)`` (default l)."""
    phys = phys or (lambda l: l)
    block_bytes = block_size * num_heads * head_dim * elem_bytes
    _require_device_tensor("kvx_pool_create", "kv", kv, torch.uint8)
    if kv.dim() != 3 or kv.shape[1] not in (1, 2):
        raise ValueError(f"kvx_pool_create: kv must be uint8 [slabs, 1 or 2 regions, region bytes], got "
                         f"{tuple(kv.shape)}")
    if kv.shape[2] < num_blocks * block_bytes:
        raise ValueError(f"kvx_pool_create: a region holds {kv.shape[2]} bytes, {num_blocks} blocks of "
                         f"{block_bytes} bytes need {num_blocks * block_bytes}")
    slabs = [phys(l) for l in range(num_layers)]
    if any(not 0 <= p < kv.shape[0] for p in slabs):
        raise ValueError(f"kvx_pool_create: a layer maps outside the {kv.shape[0]} slabs of kv")
    if scales is not None:
        _require_device_tensor("kvx_pool_create", "scales", scales, torch.float32)
        if scales.dim() != 3 or tuple(scales.shape[:2]) != tuple(kv.shape[:2]) or scales.shape[2] < num_blocks:
            raise ValueError(f"kvx_pool_create: scales must be float32 [{kv.shape[0]}, {kv.shape[1]}, "
                             f">={num_blocks}], got {tuple(scales.shape)}")
        if scales.device != kv.device:
            raise ValueError("kvx_pool_create: scales and kv live on different devices")
    two = kv.shape[1] == 2
    kb = [kv[phys(l), 0].data_ptr() for l in range(num_layers)]
    vb = [kv[phys(l), 1].data_ptr() for l in range(num_layers)] if two else None
    ks = vs = None
    if scales is not None:
        ks = [scales[phys(l), 0].data_ptr() for l in range(num_layers)]
        vs = [scales[phys(l), 1].data_ptr() for l in range(num_layers)] if two else None
    return Pool(num_blocks=num_blocks, block_size=block_size, num_heads=num_heads, head_dim=head_dim,
                elem_bytes=elem_bytes, layout=layout, k_bases=kb, v_bases=vb, k_scales=ks, v_scales=vs,
                sliding_window=sliding_window, keep=(kv, scales))


class StatePool:
    """Owns a kvx_pool handle of a state-slot pool (kvx_state_pool_create)."""

    def __init__(self, *, num_slots: int, slot_bytes, bases0: Sequence[int], bases1: Sequence[int], keep=()):
        L = len(bases0)
        arr = C.c_void_p * L
        self._b = (arr(*bases0), arr(*bases1))
        d = kvx_state_pool_desc(L, num_slots, (C.c_int64 * 2)(*slot_bytes),
                                (C.POINTER(C.c_void_p) * 2)(self._b[0], self._b[1]))
        h = C.c_void_p()
        _check("kvx_state_pool_create", lib().kvx_state_pool_create(C.byref(d), C.byref(h)))
        self.handle, self._L = h, lib()
        self.num_layers, self.num_slots, self.slot_bytes = L, num_slots, tuple(slot_bytes)
        self.keep = keep

    def close(self):
        if getattr(self, "handle", None):
            self._L.kvx_pool_destroy(self.handle)
            self.handle = None

    __del__ = close


def kvx_state_pool_create(*, regions: Sequence[torch.Tensor], num_slots: int, slot_bytes) -> StatePool:
    """Register a state pool stored as two uint8 tensors [layers, num_slots *
    slot_bytes[r]] (r = 0: convolution state, 1: SSM state)."""
    if len(regions) != 2:
        raise ValueError("kvx_state_pool_create: two regions (convolution state, SSM state)")
    for r, t in enumerate(regions):
        _require_device_tensor("kvx_state_pool_create", f"regions[{r}]", t, torch.uint8)
        if t.dim() != 2 or t.shape[1] < num_slots * slot_bytes[r]:
            raise ValueError(f"kvx_state_pool_create: regions[{r}] must be uint8 [layers, >={num_slots} x "
                             f"{slot_bytes[r]}], got {tuple(t.shape)}")
    if regions[0].shape[0] != regions[1].shape[0] or regions[0].device != regions[1].device:
        raise ValueError("kvx_state_pool_create: both regions need the same layer count and device")
    L = regions[0].shape[0]
    return StatePool(num_slots=num_slots, slot_bytes=slot_bytes,
                     bases0=[regions[0][l].data_ptr() for l in range(L)],
                     bases1=[regions[1][l].data_ptr() for l in range(L)], keep=tuple(regions))


class Plan:
    """Owns a kvx_plan_t handle.  close() and garbage collection call
    kvx_plan_destroy, which drains the device first; a plan used on one
    stream is better released with close_after(stream), which does not wait."""

    def __init__(self, handle, src: Pool, dst: Pool):
        self.handle, self.src, self.dst, self._L = handle, src, dst, lib()

    def runs(self) -> np.ndarray:
        n = C.c_int64()
        _check("kvx_plan_runs", lib().kvx_plan_runs(self.handle, None, 0, C.byref(n)))
        out = (kvx_run * max(n.value, 1))()
        _check("kvx_plan_runs", lib().kvx_plan_runs(self.handle, out, n.value, C.byref(n)))
        return np.frombuffer(out, np.int32, count=4 * n.value).reshape(-1, 4).copy()

    def triples(self, layer: int = 0, kv: int = 0) -> np.ndarray:
        n = C.c_int64()
        _check("kvx_plan_triples", lib().kvx_plan_triples(self.handle, layer, kv, None, 0, C.byref(n)))
        out = (kvx_triple * max(n.value, 1))()
        _check("kvx_plan_triples", lib().kvx_plan_triples(self.handle, layer, kv, out, n.value, C.byref(n)))
        return np.frombuffer(out, np.int64, count=3 * n.value).reshape(-1, 3).copy()

    def launch_shape(self) -> dict:
        s = kvx_launch_shape()
        _check("kvx_plan_launch_shape", lib().kvx_plan_launch_shape(self.handle, C.byref(s)))
        return {"pieces": s.pieces, "piece_bytes": s.piece_bytes, "lanes": s.lanes, "vectors": s.vectors,
                "run_table": bool(s.run_table)}

    def bytes_per_layer(self):
        r, w = C.c_int64(), C.c_int64()
        _check("kvx_plan_bytes", lib().kvx_plan_bytes(self.handle, C.byref(r), C.byref(w)))
        return r.value, w.value

    def close(self):
        if getattr(self, "handle", None):
            self._L.kvx_plan_destroy(self.handle)
            self.handle = None

    def close_after(self, stream=None):
        """kvx_plan_destroy_after: freed once the work enqueued on ``stream``
        so far has finished, without waiting on the host."""
        if getattr(self, "handle", None):
            h, self.handle = self.handle, None
            _check("kvx_plan_destroy_after", self._L.kvx_plan_destroy_after(h, _stream(stream)))

    __del__ = close


def kvx_plan_reclaim(wait: bool = False) -> int:
    """Free released plans whose work has finished; returns how many remain."""
    n = C.c_int64()
    _check("kvx_plan_reclaim", lib().kvx_plan_reclaim(int(wait), C.byref(n)))
    return n.value


def _csr(tables):
    off = np.zeros(len(tables) + 1, np.int64)
    off[1:] = np.cumsum([len(t) for t in tables])
    ids = (np.concatenate([np.asarray(t, np.int32) for t in tables]) if len(tables) else np.zeros(0, np.int32))
    return off, np.ascontiguousarray(ids, np.int32)


def kvx_plan(src: Pool, dst: Pool, num_tokens: Sequence[int], src_tables: Sequence[Sequence[int]],
             dst_tables: Sequence[Sequence[int]], *, host_only: bool = False, overlap: bool = False,
             runs: bool = False, stream=None) -> Plan:
    """Build a plan.  ``num_tokens[r]`` tokens of request r move; its block
    lists are ``src_tables[r]`` / ``dst_tables[r]`` (each at least as long as
    its side needs).  ``overlap``: KVX_PLAN_OVERLAP (the caller keeps several
    of the plan's device calls in flight at once); ``runs``: KVX_PLAN_RUNS
    (streaming launches read run tables instead of cut pieces)."""
    R = len(num_tokens)
    if len(src_tables) != R or len(dst_tables) != R:
        raise ValueError("one src and one dst block list per request")
    nt = np.ascontiguousarray(num_tokens, dtype=np.int64)
    so, sid = _csr(src_tables)
    do, did = _csr(dst_tables)
    h = C.c_void_p()
    us = None if host_only else _stream(stream)
    rc = lib().kvx_plan(src.handle, dst.handle, R, nt.ctypes.data, so.ctypes.data, do.ctypes.data,
                        sid.ctypes.data if sid.size else None, did.ctypes.data if did.size else None,
                        (KVX_PLAN_HOST_ONLY if host_only else 0) | (KVX_PLAN_OVERLAP if overlap else 0)
                        | (KVX_PLAN_RUNS if runs else 0), us,
                        C.byref(h))
    _check("kvx_plan", rc)
    return Plan(h, src, dst)


def kvx_plan_noalloc(src: Pool, dst: Pool, num_tokens: Sequence[int], src_tables: Sequence[Sequence[int]],
                     dst_tables: Sequence[Sequence[int]], *, overlap: bool = False, runs: bool = False,
                     stream=None) -> Plan:
    """kvx_plan whose device work list lives in the library's static scratch
    array (no device allocation); valid until the next kvx_plan_noalloc on
    the device."""
    R = len(num_tokens)
    if len(src_tables) != R or len(dst_tables) != R:
        raise ValueError("one src and one dst block list per request")
    nt = np.ascontiguousarray(num_tokens, dtype=np.int64)
    so, sid = _csr(src_tables)
    do, did = _csr(dst_tables)
    h = C.c_void_p()
    rc = lib().kvx_plan_noalloc(src.handle, dst.handle, R, nt.ctypes.data, so.ctypes.data, do.ctypes.data,
                                sid.ctypes.data if sid.size else None, did.ctypes.data if did.size else None,
                                (KVX_PLAN_OVERLAP if overlap else 0) | (KVX_PLAN_RUNS if runs else 0),
                                _stream(stream), C.byref(h))
    _check("kvx_plan_noalloc", rc)
    return Plan(h, src, dst)


def kvx_plan_raw(src: Pool, dst: Pool, num_requests: int, num_tokens, src_offsets, dst_offsets, src_ids,
                 dst_ids, flags: int = KVX_PLAN_HOST_ONLY, stream=None):
    """Direct call with raw arrays (numpy) for error-path tests; returns
    (status, Plan or None)."""
    h = C.c_void_p()
    keep = [None if a is None else np.ascontiguousarray(a)
            for a in (num_tokens, src_offsets, dst_offsets, src_ids, dst_ids)]
    rc = lib().kvx_plan(src.handle if src else None, dst.handle if dst else None, num_requests,
                        *(None if a is None else a.ctypes.data for a in keep), flags, stream, C.byref(h))
    return rc, (Plan(h, src, dst) if rc == KVX_OK else None)


def kvx_plan_wait(plan: Plan) -> None:
    """Wait on the host for the plan's descriptor upload (before capturing
    its device calls into a graph)."""
    _check("kvx_plan_wait", lib().kvx_plan_wait(plan.handle))


def kvx_push_layer(plan: Plan, layer: int, ready=None, stream=None) -> None:
    _check("kvx_push_layer", lib().kvx_push_layer(plan.handle, layer, _event(ready), _stream(stream)))


def kvx_push_layer_timed(plan: Plan, layer: int, started, finished, ready=None, stream=None) -> None:
    """kvx_push_layer with the kernel's own start/end timestamps recorded into
    two timing-enabled torch.cuda.Event objects."""
    for e in (started, finished):
        if e is not None and not e.cuda_event:
            # torch creates the underlying event lazily; make it exist first
            e.record(torch.cuda.current_stream())
    _check("kvx_push_layer_timed", lib().kvx_push_layer_timed(
        plan.handle, layer, _event(ready), _stream(stream), _event(started), _event(finished)))


def kvx_push_many(plans: Sequence[Plan], layers: Sequence[int], ready=None, stream=None) -> None:
    """Push layers[i] of plans[i] for every i, batched into few launches."""
    n = len(plans)
    if len(layers) != n:
        raise ValueError("one layer per plan")
    hp = (C.c_void_p * max(n, 1))(*[p.handle for p in plans])
    ly = np.ascontiguousarray(layers, dtype=np.int32)
    _check("kvx_push_many", lib().kvx_push_many(hp, ly.ctypes.data if n else None, n, _event(ready),
                                                _stream(stream)))


def kvx_push_many_timed(plans: Sequence[Plan], layers: Sequence[int], started, finished, ready=None,
                        stream=None) -> None:
    """kvx_push_many with its launches' start and end dispatch timestamps
    recorded into two timing-enabled torch.cuda.Event objects."""
    n = len(plans)
    if len(layers) != n:
        raise ValueError("one layer per plan")
    for e in (started, finished):
        if e is not None and not e.cuda_event:
            e.record(torch.cuda.current_stream())
    hp = (C.c_void_p * max(n, 1))(*[p.handle for p in plans])
    ly = np.ascontiguousarray(layers, dtype=np.int32)
    _check("kvx_push_many_timed", lib().kvx_push_many_timed(hp, ly.ctypes.data if n else None, n, _event(ready),
                                                            _stream(stream), _event(started), _event(finished)))


def kvx_staging_bytes(plan: Plan, l0: int, l1: int) -> int:
    b = C.c_int64()
    _check("kvx_staging_bytes", lib().kvx_staging_bytes(plan.handle, l0, l1, C.byref(b)))
    return b.value


def _staging_cap(fn: str, staging: torch.Tensor) -> int:
    _require_device_tensor(fn, "staging", staging, None)
    return staging.numel() * staging.element_size()


def kvx_pack(plan: Plan, l0: int, l1: int, staging: torch.Tensor, stream=None) -> None:
    cap = _staging_cap("kvx_pack", staging)
    _check("kvx_pack", lib().kvx_pack(plan.handle, l0, l1, staging.data_ptr(), cap, _stream(stream)))


def kvx_unpack(plan: Plan, l0: int, l1: int, staging: torch.Tensor, stream=None) -> None:
    cap = _staging_cap("kvx_unpack", staging)
    _check("kvx_unpack", lib().kvx_unpack(plan.handle, l0, l1, staging.data_ptr(), cap, _stream(stream)))


def kvx_copy_heads(plan: Plan, layer: int, src_head0: int, dst_head0: int, num_heads: int,
                   ready=None, stream=None) -> None:
    _check("kvx_copy_heads", lib().kvx_copy_heads(plan.handle, layer, src_head0, dst_head0, num_heads,
                                                  _event(ready), _stream(stream)))


def kvx_copy_heads_layers(plan: Plan, l0: int, l1: int, src_head0: int, dst_head0: int, num_heads: int,
                          ready=None, stream=None) -> None:
    """kvx_copy_heads over layers [l0, l1), up to 32 layers per launch."""
    _check("kvx_copy_heads_layers", lib().kvx_copy_heads_layers(plan.handle, l0, l1, src_head0, dst_head0,
                                                                num_heads, _event(ready), _stream(stream)))


class Queue:
    """Owns a kvx_queue handle: the layer write queue of one stream
    (kvx_queue_push per layer save, kvx_queue_flush before waiting)."""

    def __init__(self, stream=None):
        h = C.c_void_p()
        _check("kvx_queue_create", lib().kvx_queue_create(_stream(stream), C.byref(h)))
        self.handle, self._L = h, lib()

    def push(self, plan: Plan, layer: int, ready=None) -> None:
        _check("kvx_queue_push", lib().kvx_queue_push(self.handle, plan.handle, layer, _event(ready)))

    def push_heads(self, plan: Plan, layer: int, src_head0: int, dst_head0: int, num_heads: int,
                   ready=None) -> None:
        _check("kvx_queue_push_heads", lib().kvx_queue_push_heads(self.handle, plan.handle, layer, src_head0,
                                                                  dst_head0, num_heads, _event(ready)))

    def flush(self) -> None:
        _check("kvx_queue_flush", lib().kvx_queue_flush(self.handle))

    def stats(self):
        """(writes queued, launch groups enqueued) so far."""
        return self.stats3()[:2]

    def stats3(self):
        """(writes queued, launch groups enqueued, kernel launches) so far."""
        w, g, n = C.c_int64(), C.c_int64(), C.c_int64()
        _check("kvx_queue_stats", lib().kvx_queue_stats(self.handle, C.byref(w), C.byref(g), C.byref(n)))
        return w.value, g.value, n.value

    def close(self) -> None:
        if getattr(self, "handle", None):
            h, self.handle = self.handle, None
            _check("kvx_queue_destroy", self._L.kvx_queue_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kvx_queue_create(stream=None) -> Queue:
    return Queue(stream)


class Xfer:
    """Owns a kvx_xfer handle: the transfer state machine of kvx_xfer.h.
    Methods return the C call's `accepted` flag where it has one."""

    def __init__(self, producer: Pool, *, defer_timeout: float = 60.0, transfer_timeout: float = 30.0,
                 host_only: bool = False, log: bool = False, stream=None):
        """``log``: KVX_XFER_LOG (keep the issued-write log that issued() reads)."""
        cfg = kvx_xfer_config(defer_timeout, transfer_timeout,
                              (KVX_XFER_HOST_ONLY if host_only else 0) | (KVX_XFER_LOG if log else 0))
        h = C.c_void_p()
        st = None if host_only else _stream(stream)
        _check("kvx_xfer_create", lib().kvx_xfer_create(producer.handle, C.byref(cfg), st, C.byref(h)))
        self.handle, self.producer, self._L = h, producer, lib()
        self._consumers = {}   # the C side keeps pool pointers: keep the Pool objects alive

    def _acc(self, name, *args) -> bool:
        acc = C.c_int32(-1)
        _check(name, getattr(lib(), name)(self.handle, *args, C.byref(acc)))
        return bool(acc.value)

    def register(self, req: int, attempt: int, consumer: Pool, dst_ids, now: float) -> bool:
        a = np.ascontiguousarray(dst_ids, np.int32)
        self._consumers[id(consumer)] = consumer
        return self._acc("kvx_xfer_register", req, attempt, consumer.handle, a.ctypes.data if a.size else None,
                         a.size, now)

    def prefill(self, req: int, attempt: int, num_tokens: int, src_ids, now: float) -> bool:
        a = np.ascontiguousarray(src_ids, np.int32)
        return self._acc("kvx_xfer_prefill", req, attempt, num_tokens, a.ctypes.data if a.size else None, a.size, now)

    def save_layer(self, req: int, attempt: int, layer: int, now: float, ready=None) -> bool:
        return self._acc("kvx_xfer_save_layer", req, attempt, layer, _event(ready), now)

    def save_layer_many(self, layer: int, reqs, attempts, now: float, ready=None):
        r = np.ascontiguousarray(reqs, np.uint64)
        a = np.ascontiguousarray(attempts, np.uint32)
        acc = np.zeros(len(r), np.int32)
        _check("kvx_xfer_save_layer_many", lib().kvx_xfer_save_layer_many(
            self.handle, layer, _event(ready), len(r), r.ctypes.data if r.size else None,
            a.ctypes.data if a.size else None, now, acc.ctypes.data if acc.size else None))
        return [bool(v) for v in acc]

    def seal(self, req: int, attempt: int) -> bool:
        return self._acc("kvx_xfer_seal", req, attempt)

    def poll(self, now: float) -> None:
        _check("kvx_xfer_poll", lib().kvx_xfer_poll(self.handle, now))

    def complete(self, req: int, attempt: int, layer: int, ok: bool = True) -> None:
        _check("kvx_xfer_complete", lib().kvx_xfer_complete(self.handle, req, attempt, layer, int(ok)))

    def status(self, req: int):
        a, st = C.c_uint32(), C.c_int32()
        rc = lib().kvx_xfer_status(self.handle, req, C.byref(a), C.byref(st))
        if rc == KVX_E_RANGE:
            return None
        _check("kvx_xfer_status", rc)
        return a.value, st.value

    def pop_finished(self, cap: int = 1024):
        r = (C.c_uint64 * cap)()
        a = (C.c_uint32 * cap)()
        st = (C.c_int32 * cap)()
        n = C.c_int64()
        _check("kvx_xfer_pop_finished", lib().kvx_xfer_pop_finished(self.handle, r, a, st, cap, C.byref(n)))
        return [(r[i], a[i], st[i]) for i in range(n.value)]

    def recompute_blocks(self, req: int):
        n = C.c_int64()
        rc = lib().kvx_xfer_recompute_blocks(self.handle, req, None, 0, C.byref(n))
        if rc == KVX_E_RANGE:
            return None
        _check("kvx_xfer_recompute_blocks", rc)
        out = (C.c_int32 * max(n.value, 1))()
        _check("kvx_xfer_recompute_blocks", lib().kvx_xfer_recompute_blocks(self.handle, req, out, n.value,
                                                                            C.byref(n)))
        return list(out[:n.value])

    def issued(self, first: int = 0, cap: int = 1 << 16):
        r = (C.c_uint64 * cap)()
        a = (C.c_uint32 * cap)()
        ly = (C.c_int32 * cap)()
        n = C.c_int64()
        _check("kvx_xfer_issued", lib().kvx_xfer_issued(self.handle, first, r, a, ly, cap, C.byref(n)))
        return [(r[i], a[i], ly[i]) for i in range(n.value)]

    def forget(self, req: int) -> None:
        _check("kvx_xfer_forget", lib().kvx_xfer_forget(self.handle, req))

    def close(self):
        if getattr(self, "handle", None):
            self._L.kvx_xfer_destroy(self.handle)
            self.handle = None

    __del__ = close
