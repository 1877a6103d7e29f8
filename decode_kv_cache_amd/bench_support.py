"""ctypes binding of libkvx_bench.so: the synthetic layer-compute kernel, a
plain contiguous copy and a cache-flush fill (measurement helpers; not part of
the transfer path)."""
from __future__ import annotations

import ctypes as C
import os

import torch

from .kvx import _stream

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvx_bench.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decode_kv_cache_amd.build`")
        h = C.CDLL(LIB_PATH)
        P, I32, I64, U32 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32
        h.kvxb_layer_compute.argtypes = [P, I32, I32, P, P, P, I32, I64, U32, P]
        h.kvxb_copy.argtypes = [P, P, I64, I32, P]
        h.kvxb_fill.argtypes = [P, I64, U32, P]
        h.kvxb_copy_segments.argtypes = [P, P, I32, I64, I32, P]
        h.kvxb_stream_create_cu_mask.argtypes = [P, I32, C.POINTER(P)]
        h.kvxb_stream_destroy.argtypes = [P]
        for f in (h.kvxb_layer_compute, h.kvxb_copy, h.kvxb_fill, h.kvxb_copy_segments,
                  h.kvxb_stream_create_cu_mask, h.kvxb_stream_destroy):
            f.restype = C.c_int
        _lib = h
    return _lib


def _ok(name, rc):
    if rc != 0:
        raise RuntimeError(f"{name} failed: hipError {rc}")


def layer_compute(sink: torch.Tensor, iters: int, grid: int, k_region=None, v_region=None,
                  blocks: torch.Tensor = None, block_bytes: int = 0, canary: int = 0, stream=None):
    assert sink.numel() >= grid * 256 and sink.dtype == torch.float32
    if k_region is not None:
        assert blocks.dtype == torch.int32 and blocks.is_cuda
        assert int(blocks.max()) * block_bytes + 16 <= k_region.numel()
    _ok("kvxb_layer_compute", lib().kvxb_layer_compute(
        sink.data_ptr(), iters, grid,
        None if k_region is None else k_region.data_ptr(), None if v_region is None else v_region.data_ptr(),
        None if blocks is None else blocks.data_ptr(), 0 if blocks is None else blocks.numel(),
        block_bytes, canary & 0xFFFFFFFF, _stream(stream)))


def copy(dst: torch.Tensor, src: torch.Tensor, nbytes: int, grid: int = 4096, stream=None):
    assert nbytes <= dst.numel() * dst.element_size() and nbytes <= src.numel() * src.element_size()
    _ok("kvxb_copy", lib().kvxb_copy(dst.data_ptr(), src.data_ptr(), nbytes, grid, _stream(stream)))


def fill(dst: torch.Tensor, value: int = 0, stream=None):
    nbytes = dst.numel() * dst.element_size()
    _ok("kvxb_fill", lib().kvxb_fill(dst.data_ptr(), nbytes - nbytes % 16, value, _stream(stream)))


def copy_segments(src_ptrs: torch.Tensor, dst_ptrs: torch.Tensor, seg_bytes: int, shape: int, stream=None):
    """Plain copy of len(src_ptrs) segments of seg_bytes (device int64 address
    arrays; the caller guarantees every segment lies inside its allocation).
    shape 0: one-wave workgroups of 32 KiB chunks; 1: four-wave workgroups of
    4 KiB chunks."""
    assert src_ptrs.dtype == torch.int64 and dst_ptrs.dtype == torch.int64 and src_ptrs.is_cuda
    assert src_ptrs.numel() == dst_ptrs.numel()
    _ok("kvxb_copy_segments", lib().kvxb_copy_segments(src_ptrs.data_ptr(), dst_ptrs.data_ptr(), src_ptrs.numel(),
                                                       seg_bytes, shape, _stream(stream)))


class CuMaskStream:
    """A stream restricted to the compute units of `cus` (default priority);
    ``.torch`` wraps it for torch events and kernel launches."""

    def __init__(self, cus, num_cus: int):
        words = (num_cus + 31) // 32
        mask = (C.c_uint32 * words)()
        for cu in cus:
            mask[cu // 32] |= 1 << (cu % 32)
        h = C.c_void_p()
        _ok("kvxb_stream_create_cu_mask", lib().kvxb_stream_create_cu_mask(mask, words, C.byref(h)))
        self.handle = h.value
        self.torch = torch.cuda.ExternalStream(self.handle)
        self.cus = list(cus)

    def close(self):
        if self.handle:
            torch.cuda.synchronize()
            _ok("kvxb_stream_destroy", lib().kvxb_stream_destroy(self.handle))
            self.handle = None
