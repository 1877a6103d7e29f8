"""libkvx: paged-KV block transfer between a producer (prefill) pool and a
consumer (decode) pool on one MI355X.

``decode_kv_cache_amd.kvx`` is the thin ctypes binding of the C ABI declared in
``include/kvx.h`` (the HIP kernels live in ``csrc/``); ``workloads`` holds the
seeded synthetic inputs.
"""
