"""MI355X-native routed-MoE layer over a cross-layer LRU expert slot cache.

The compute path is ``libmc.so`` (hand-written HIP for gfx950 plus a C++ host
branch) behind the C ABI in ``include/mc.h``; this package is its thin Python
binding (``_lib``) and the torch-based memory plumbing (``runtime``).
"""
from . import _lib  # noqa: F401
from ._lib import (MC_BF16, MC_MXFP4, Banks, Cache, HostPool, McError, abi_version,  # noqa: F401
                   cache_reset, decode_ws_bytes, fetch_fraction_q16, fill_slots, finish_bf16,
                   host_experts, hybrid_split_merge, lib, make_banks, make_cache, make_hybrid,
                   moe_experts_decode, moe_route, moe_route_lookup, slot_cache_lookup_evict,
                   bandwidth_profile, recommend_backend, cache_install)
