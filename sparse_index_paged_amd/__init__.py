"""Packed QSA decode for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libqsa.so`` (built from ``csrc/`` by
``build.py``).  Every step of the decode and of the quantize + scatter
write runs in the library's HIP kernels;
this module only turns torch tensors into ``qsa_tensor`` descriptors and
passes torch's current HIP stream.  If the library is missing the import of
``decode`` fails loudly -- there is no fallback.
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    ABI_VERSION,
    KvPool,
    QsaError,
    TieredPool,
    abi_version,
    debug_audit_counters,
    debug_counter_ptr,
    debug_counters,
    debug_device_error,
    decode,
    decode_noalloc,
    decode_tiered,
    get_option,
    index,
    index_reserve,
    kv_store,
    kv_store_tiered,
    lib_path,
    load_library,
    plan,
    set_option,
    workspace_attach,
    workspace_bytes,
    workspace_detach,
    workspace_release,
    workspace_reserve,
    workspace_reset,
)

__all__ = [
    "decode", "decode_noalloc", "kv_store", "decode_tiered", "kv_store_tiered", "index", "index_reserve", "plan", "workspace_reserve", "workspace_attach",
    "workspace_detach", "workspace_reset", "workspace_release",
    "workspace_bytes", "set_option", "get_option", "debug_counters", "debug_counter_ptr", "debug_audit_counters",
    "debug_device_error", "abi_version", "load_library", "lib_path", "QsaError", "TieredPool", "KvPool",
    "ABI_VERSION",
]
