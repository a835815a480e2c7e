"""ctypes binding of ``libmc.so`` (argument marshalling only).

Every function here forwards to the C ABI declared in ``include/mc.h`` with plain
pointers taken from torch tensors; no arithmetic of the MoE path happens in Python.
torch supplies device memory, pinned host memory and streams.  If the shared
library is missing, importing this module raises — there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmc.so")

MC_OK, MC_EINVAL, MC_ENOMEM, MC_EHIP, MC_EUNSUPPORTED, MC_EDEVICE = 0, -1, -2, -3, -4, -5
MC_BF16, MC_MXFP4 = 0, 1
MC_SPLIT_SUBMIT, MC_MERGE = 0, 1
FMT = {"bf16": MC_BF16, "mxfp4": MC_MXFP4}
STAT_NAMES = ("hits", "misses", "fills", "host", "evictions", "calls", "err", "reserved")


class McError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__("%s -> %d: %s" % (fn, code, msg))
        self.code = code


class Banks(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("H", C.c_int32), ("I", C.c_int32), ("reserved", C.c_int32),
                ("n", C.c_int64), ("gate_up", C.c_void_p), ("gate_up_scale", C.c_void_p),
                ("down", C.c_void_p), ("down_scale", C.c_void_p)]


class Cache(C.Structure):
    _fields_ = [("L", C.c_int32), ("E", C.c_int32), ("S", C.c_int32), ("reserved", C.c_int32),
                ("slot_of", C.c_void_p), ("id_of", C.c_void_p), ("stamp", C.c_void_p),
                ("clock", C.c_void_p), ("stats", C.c_void_p)]


class Prefetch(C.Structure):
    _fields_ = [("host_src", C.POINTER(Banks)), ("first_flat", C.c_int64), ("dst", C.POINTER(Banks)),
                ("copy", C.c_void_p), ("dst_free", C.c_void_p), ("done", C.c_void_p)]


class BwProfile(C.Structure):
    _fields_ = [("pcie_gbs", C.c_double), ("cpu_gbs", C.c_double), ("pcie_ov_gbs", C.c_double),
                ("cpu_ov_gbs", C.c_double), ("expert_bytes", C.c_double), ("frac_q16", C.c_uint32),
                ("hybrid", C.c_int32)]


class FillList(C.Structure):
    _fields_ = [("host", C.POINTER(Banks)), ("fill_flat", C.c_void_p), ("fill_slot", C.c_void_p),
                ("n_fill", C.c_void_p), ("kcap", C.c_int32), ("mode", C.c_int32),
                ("down_after", C.c_void_p)]


MC_BANK_GATE_UP, MC_BANK_GATE_UP_SCALE, MC_BANK_DOWN, MC_BANK_DOWN_SCALE, MC_BANK_ALL = 1, 2, 4, 8, 15
MC_FILL_THROUGH, MC_FILL_GATE_UP, MC_FILL_WITH_GATE_UP = 0, 1, 2


class Hybrid(C.Structure):
    _fields_ = [("x_bf16", C.c_void_p), ("ids_raw", C.c_void_p), ("slots", C.c_void_p),
                ("w", C.c_void_p), ("T", C.c_int32), ("k", C.c_int32), ("layer", C.c_int32),
                ("E", C.c_int32), ("n_tok", C.c_void_p), ("host", C.POINTER(Banks)),
                ("pool", C.c_void_p), ("pinned_stage", C.c_void_p), ("stage_bytes", C.c_size_t),
                ("gpu_w", C.c_void_p), ("host_ids", C.c_void_p), ("y_acc", C.c_void_p),
                ("y_host", C.c_void_p), ("y_bf16", C.c_void_p)]


_P = C.c_void_p
_I32 = C.c_int32
_SIGS = {
    "mc_abi_version": (C.c_int, []),
    "mc_last_error": (C.c_char_p, []),
    "mc_cache_reset": (C.c_int, [C.POINTER(Cache), _P]),
    "mc_fetch_fraction_q16": (C.c_uint32, [C.c_double] * 4),
    "moe_route": (C.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "slot_cache_lookup_evict": (C.c_int, [C.POINTER(Cache), _I32, _P, _I32, _I32, _P, C.c_uint32,
                                          _I32, _I32, _P, _P, _P, _P, _P, _P, _I32, _P]),
    "moe_route_lookup": (C.c_int, [_P, _I32, _P, _P, C.POINTER(Cache), _I32, _I32, _I32, _P, C.c_uint32,
                                   _I32, _I32, _P, _P, _P, _P, _P, _P, _I32, _P]),
    "mc_fill_slots": (C.c_int, [C.POINTER(Banks), C.POINTER(Banks), _P, _P, _P, _I32, _P]),
    "mc_cache_install": (C.c_int, [C.POINTER(Cache), _P, _I32, _P]),
    "mc_host_forget": (C.c_int, [_P, C.c_size_t]),
    "mc_fill_slots_banks": (C.c_int, [C.POINTER(Banks), C.POINTER(Banks), _P, _P, _P, _I32, C.c_uint32, _P]),
    "moe_experts_decode_ws_bytes": (C.c_size_t, [_I32, _I32, _I32, _I32]),
    "moe_experts_decode": (C.c_int, [_P, _P, _P, _I32, _I32, _P, C.POINTER(Banks), C.POINTER(Banks),
                                     _P, C.c_size_t, _P, _I32, _P, _P, C.POINTER(FillList)]),
    "moe_experts_decode_noalloc": (C.c_int, [_P, _P, _P, _I32, _I32, _P, C.POINTER(Banks), C.POINTER(Banks),
                                             _P, _I32, _P, _P, C.POINTER(FillList)]),
    "moe_experts_decode_noalloc_max_bytes": (C.c_size_t, []),
    "mc_prefill_sort_routes": (C.c_int, [_P, _I32, _I32, _P, _I32, _P, C.c_size_t, _P, _P, _P, _P]),
    "moe_experts_prefill_ws_bytes": (C.c_size_t, [_I32, _I32, _I32, _I32, _I32]),
    "moe_experts_prefill": (C.c_int, [_P, _P, _P, _I32, _I32, _P, _I32, C.POINTER(Banks), _P, C.c_size_t,
                                      _P, _P, C.POINTER(Prefetch)]),
    "moe_experts_prefill_part": (C.c_int, [_P, _P, _P, _I32, _I32, _P, _I32, C.POINTER(Banks), _P, _I32, _P,
                                           C.c_size_t, _P, _P, _P]),
    "moe_experts_prefill_status": (C.c_int, [_P, _P, C.POINTER(C.c_uint32)]),
    "mc_host_pool_create": (_P, [_I32, _P]),
    "mc_host_pool_destroy": (None, [_P]),
    "mc_host_pool_cpus": (C.c_int32, [_P, _P, _I32]),
    "mc_host_experts": (C.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, C.POINTER(Banks), _P]),
    "mc_bandwidth_profile": (C.c_int, [C.POINTER(Banks), C.POINTER(Banks), _P, _I32, C.c_double, C.c_double,
                                       _P, C.POINTER(BwProfile)]),
    "mc_recommend_backend": (C.c_int32, [C.c_double, C.c_double, C.c_double]),
    "mc_hybrid_stage_bytes": (C.c_size_t, [_I32, _I32, _I32]),
    "mc_hybrid_stage_alloc": (C.c_void_p, [C.c_size_t]),
    "mc_hybrid_stage_free": (C.c_int, [C.c_void_p]),
    "mc_hybrid_stage_errors": (C.c_uint32, [C.c_void_p]),
    "hybrid_split_merge": (C.c_int, [C.POINTER(Hybrid), _I32, _P]),
    "mc_finish_bf16": (C.c_int, [_P, _I32, _I32, _P, _P, _P]),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmc.so is not built (run python -m expert_cache_offloaded_amd.build)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def declared_symbols():
    return list(_SIGS)


def last_error() -> str:
    return lib().mc_last_error().decode()


def _check(fn: str, rc: int) -> int:
    if rc != MC_OK:
        raise McError(fn, rc, last_error())
    return rc


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ---------------------------------------------------------------- descriptors

def make_banks(fmt: str, H: int, I: int, tensors: Dict[str, "object"]) -> Banks:
    """Bank descriptor over tensors whose leading dim is the entry (slot / flat id)."""
    b = Banks()
    b.fmt = FMT[fmt]
    b.H, b.I = H, I
    b.n = tensors["gate_up"].shape[0]
    b.gate_up = _ptr(tensors["gate_up"])
    b.down = _ptr(tensors["down"])
    b.gate_up_scale = _ptr(tensors.get("gate_up_scale"))
    b.down_scale = _ptr(tensors.get("down_scale"))
    return b


def make_cache(L: int, E: int, S: int, t: Dict[str, "object"]) -> Cache:
    c = Cache()
    c.L, c.E, c.S = L, E, S
    c.slot_of, c.id_of, c.stamp = _ptr(t["slot_of"]), _ptr(t["id_of"]), _ptr(t["stamp"])
    c.clock, c.stats = _ptr(t["clock"]), _ptr(t["stats"])
    return c


# ---------------------------------------------------------------- calls

def abi_version() -> int:
    return lib().mc_abi_version()


def fetch_fraction_q16(b_p: float, b_h: float, p_ov: float = 0.0, c_ov: float = 0.0) -> int:
    return int(lib().mc_fetch_fraction_q16(b_p, b_h, p_ov, c_ov))


def cache_reset(cache: Cache, stream=None) -> None:
    _check("mc_cache_reset", lib().mc_cache_reset(C.byref(cache), _stream(stream)))


def moe_route(logits, k: int, renorm: int, topk_ids, topk_w, stream=None) -> None:
    T, E = logits.shape
    _check("moe_route", lib().moe_route(_ptr(logits), T, E, k, renorm, _ptr(topk_ids),
                                        _ptr(topk_w), _stream(stream)))


def slot_cache_lookup_evict(cache: Cache, layer: int, ids, n_tok, frac_q16: int, fixed_cap: int,
                            min_fill: int, slots, fill_flat, fill_slot, n_fill, host_flat, n_host,
                            stream=None) -> None:
    T, k = ids.shape
    _check("slot_cache_lookup_evict", lib().slot_cache_lookup_evict(
        C.byref(cache), layer, _ptr(ids), T, k, _ptr(n_tok), frac_q16, fixed_cap, min_fill,
        _ptr(slots), _ptr(fill_flat), _ptr(fill_slot), _ptr(n_fill), _ptr(host_flat), _ptr(n_host),
        fill_flat.numel(), _stream(stream)))


def moe_route_lookup(logits, renorm: int, ids, w, cache: Cache, layer: int, n_tok, frac_q16: int,
                     fixed_cap: int, min_fill: int, slots, fill_flat, fill_slot, n_fill, host_flat,
                     n_host, stream=None) -> None:
    T, k = ids.shape
    _check("moe_route_lookup", lib().moe_route_lookup(
        _ptr(logits), renorm, _ptr(ids), _ptr(w), C.byref(cache), layer, T, k, _ptr(n_tok), frac_q16,
        fixed_cap, min_fill, _ptr(slots), _ptr(fill_flat), _ptr(fill_slot), _ptr(n_fill),
        _ptr(host_flat), _ptr(n_host), fill_flat.numel(), _stream(stream)))


def host_forget(ptr: int, nbytes: int = 0) -> int:
    """Drop the library's remembered device translations of pinned host memory in
    [ptr, ptr + nbytes) (mc_host_forget); returns how many were dropped."""
    rc = lib().mc_host_forget(ptr, nbytes)
    if rc < 0:
        raise McError("mc_host_forget", rc, last_error())
    return rc


def cache_install(cache: Cache, flat, stream=None) -> None:
    """flat[i] (device int32) becomes resident in slot i; the cache must be empty there."""
    _check("mc_cache_install", lib().mc_cache_install(C.byref(cache), _ptr(flat), flat.numel(),
                                                      _stream(stream)))


def fill_slots_banks(host: Banks, pool: Banks, fill_flat, fill_slot, n_fill, banks: int, stream=None) -> None:
    _check("mc_fill_slots_banks", lib().mc_fill_slots_banks(
        C.byref(host), C.byref(pool), _ptr(fill_flat), _ptr(fill_slot), _ptr(n_fill), fill_flat.numel(),
        banks, _stream(stream)))


def fill_slots(host: Banks, pool: Banks, fill_flat, fill_slot, n_fill, stream=None) -> None:
    _check("mc_fill_slots", lib().mc_fill_slots(C.byref(host), C.byref(pool), _ptr(fill_flat),
                                                _ptr(fill_slot), _ptr(n_fill), fill_flat.numel(),
                                                _stream(stream)))


def decode_ws_bytes(T: int, k: int, H: int, I: int) -> int:
    return int(lib().moe_experts_decode_ws_bytes(T, k, H, I))


def make_fill_list(host: Banks, fill_flat, fill_slot, n_fill, mode: int = MC_FILL_THROUGH,
                   down_after=None) -> FillList:
    """Fill list of a lookup call for fill-through decode (device tensors).  mode: one of
    MC_FILL_THROUGH, MC_FILL_GATE_UP, MC_FILL_WITH_GATE_UP.  down_after: a recorded
    torch.cuda.Event the down pass waits for (or None)."""
    f = FillList()
    f.host = C.pointer(host)
    f.fill_flat = _ptr(fill_flat)
    f.fill_slot = _ptr(fill_slot)
    f.n_fill = _ptr(n_fill)
    f.kcap = fill_flat.numel()
    f.mode = mode
    f.down_after = down_after.cuda_event if down_after is not None else None
    f._keep = (host, fill_flat, fill_slot, n_fill, down_after)
    return f


def moe_experts_decode(x, slots, w, n_tok, pool: Banks, shared: Optional[Banks], ws, y_acc,
                       accumulate: int = 1, y_bf16=None, stream=None,
                       fill: Optional[FillList] = None) -> None:
    T, k = slots.shape
    _check("moe_experts_decode", lib().moe_experts_decode(
        _ptr(x), _ptr(slots), _ptr(w), T, k, _ptr(n_tok), C.byref(pool),
        C.byref(shared) if shared is not None else None, _ptr(ws), ws.numel() * ws.element_size(),
        _ptr(y_acc), accumulate, _ptr(y_bf16), _stream(stream),
        C.byref(fill) if fill is not None else None))


def moe_experts_decode_noalloc(x, slots, w, n_tok, pool: Banks, shared: Optional[Banks], y_acc,
                               accumulate: int = 1, y_bf16=None, stream=None,
                               fill: Optional[FillList] = None) -> None:
    """moe_experts_decode with the library's own scratch array as workspace (no allocation)."""
    T, k = slots.shape
    _check("moe_experts_decode_noalloc", lib().moe_experts_decode_noalloc(
        _ptr(x), _ptr(slots), _ptr(w), T, k, _ptr(n_tok), C.byref(pool),
        C.byref(shared) if shared is not None else None, _ptr(y_acc), accumulate, _ptr(y_bf16),
        _stream(stream), C.byref(fill) if fill is not None else None))


def decode_noalloc_max_bytes() -> int:
    return int(lib().moe_experts_decode_noalloc_max_bytes())


def finish_bf16(y_acc, n_tok, y_bf16, stream=None) -> None:
    T, H = y_acc.shape
    _check("mc_finish_bf16", lib().mc_finish_bf16(_ptr(y_acc), T, H, _ptr(n_tok), _ptr(y_bf16),
                                                  _stream(stream)))


def prefill_sort_routes(ids, n_tok, E: int, ws, counts, offsets, perm, stream=None) -> None:
    T, k = ids.shape
    _check("mc_prefill_sort_routes", lib().mc_prefill_sort_routes(
        _ptr(ids), T, k, _ptr(n_tok), E, _ptr(ws), ws.numel() * ws.element_size(), _ptr(counts),
        _ptr(offsets), _ptr(perm), _stream(stream)))


def prefill_status(ws, stream=None):
    """(rc, status bits) of the last moe_experts_prefill on workspace ws (synchronises)."""
    st = C.c_uint32(0)
    rc = lib().moe_experts_prefill_status(_ptr(ws), _stream(stream), C.byref(st))
    return rc, int(st.value)


def prefill_ws_bytes(T: int, k: int, E: int, H: int, I: int) -> int:
    return int(lib().moe_experts_prefill_ws_bytes(T, k, E, H, I))


def make_prefetch(host: Banks, first_flat: int, dst: Banks, copy_stream) -> Prefetch:
    """Prefetch descriptor; ordering with the compute stream is left to the caller's
    stream/event waits (dst_free and done are NULL)."""
    p = Prefetch()
    p.host_src = C.pointer(host)
    p.first_flat = first_flat
    p.dst = C.pointer(dst)
    p.copy = copy_stream.cuda_stream
    p.dst_free = None
    p.done = None
    p._keep = (host, dst)
    return p


def moe_experts_prefill(x, ids, w, n_tok, E: int, layer_buf: Banks, ws, y, nxt: Optional[Prefetch] = None,
                        stream=None) -> None:
    T, k = ids.shape
    _check("moe_experts_prefill", lib().moe_experts_prefill(
        _ptr(x), _ptr(ids), _ptr(w), T, k, _ptr(n_tok), E, C.byref(layer_buf), _ptr(ws),
        ws.numel() * ws.element_size(), _ptr(y), _stream(stream), C.byref(nxt) if nxt is not None else None))


PF_SORT, PF_EXPERTS, PF_COMBINE, PF_ALL = 1, 2, 4, 7


def moe_experts_prefill_part(x, ids, w, n_tok, E: int, part_buf: Banks, entry_of, steps: int, ws, counts=None,
                             y=None, stream=None) -> None:
    """One or more steps of a prefill layer (PF_SORT / PF_EXPERTS / PF_COMBINE) on ws."""
    T, k = ids.shape
    _check("moe_experts_prefill_part", lib().moe_experts_prefill_part(
        _ptr(x), _ptr(ids), _ptr(w), T, k, _ptr(n_tok), E, C.byref(part_buf), _ptr(entry_of), steps, _ptr(ws),
        ws.numel() * ws.element_size(), _ptr(counts), _ptr(y), _stream(stream)))


class HostPool:
    """Persistent CPU worker pool (library-owned threads)."""

    def __init__(self, n_threads: int, cpu_ids=None):
        arr = None
        if cpu_ids is not None:
            arr = (C.c_int32 * len(cpu_ids))(*cpu_ids)
        self.handle = lib().mc_host_pool_create(n_threads, arr)
        if not self.handle:
            raise McError("mc_host_pool_create", -1, last_error())
        self.n_threads = n_threads

    def cpus(self):
        """The CPU each pool thread is pinned to (-1 = not pinned); thread 0 is the dispatcher."""
        arr = (C.c_int32 * self.n_threads)()
        n = lib().mc_host_pool_cpus(self.handle, arr, self.n_threads)
        if n < 0:
            raise McError("mc_host_pool_cpus", n, last_error())
        return list(arr)

    def close(self):
        if self.handle:
            lib().mc_host_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def host_experts(pool: Optional[HostPool], x, ids, w, layer: int, E: int, host: Banks, y) -> None:
    """Synchronous host expert FFN over host tensors (x bf16 as int16/uint16 bits)."""
    T, k = ids.shape
    _check("mc_host_experts", lib().mc_host_experts(
        pool.handle if pool else None, _ptr(x), _ptr(ids), _ptr(w), T, k, layer, E, C.byref(host),
        _ptr(y)))


def hybrid_stage_bytes(T: int, k: int, H: int) -> int:
    return int(lib().mc_hybrid_stage_bytes(T, k, H))


class HybridStage:
    """Pinned staging memory of one hybrid layer call (fine-grained, from the library)."""

    def __init__(self, T: int, k: int, H: int):
        self.nbytes = hybrid_stage_bytes(T, k, H)
        self.ptr = lib().mc_hybrid_stage_alloc(self.nbytes)
        if not self.ptr:
            raise MemoryError(lib().mc_last_error().decode())

    def data_ptr(self) -> int:
        return self.ptr

    def numel(self) -> int:
        return self.nbytes

    def element_size(self) -> int:
        return 1

    def errors(self) -> int:
        """Merge waits on this stage that ran out (0 when every host branch answered)."""
        return int(lib().mc_hybrid_stage_errors(self.ptr))

    def close(self) -> None:
        if self.ptr:
            _check("mc_hybrid_stage_free", lib().mc_hybrid_stage_free(self.ptr))
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_hybrid(x, ids_raw, slots, w, layer: int, E: int, n_tok, host: Banks, pool: HostPool,
                stage, gpu_w, host_ids, y_acc, y_host, y_bf16) -> Hybrid:
    h = Hybrid()
    h.x_bf16, h.ids_raw, h.slots, h.w = _ptr(x), _ptr(ids_raw), _ptr(slots), _ptr(w)
    h.T, h.k = ids_raw.shape
    h.layer, h.E = layer, E
    h.n_tok = _ptr(n_tok)
    h.host = C.pointer(host)
    h.pool = pool.handle
    h.pinned_stage = _ptr(stage)
    h.stage_bytes = stage.numel() * stage.element_size()
    h.gpu_w, h.host_ids = _ptr(gpu_w), _ptr(host_ids)
    h.y_acc, h.y_host, h.y_bf16 = _ptr(y_acc), _ptr(y_host), _ptr(y_bf16)
    h._keep = (host,)
    return h


def hybrid_split_merge(h: Hybrid, phase: int, stream=None) -> None:
    _check("hybrid_split_merge", lib().hybrid_split_merge(C.byref(h), phase, _stream(stream)))


def recommend_backend(cpu_gbs: float, pcie_gbs: float, threshold: float = 2.0) -> str:
    """'hybrid' iff cpu_gbs > threshold * pcie_gbs, else 'offload'."""
    return "hybrid" if lib().mc_recommend_backend(cpu_gbs, pcie_gbs, threshold) else "offload"


def bandwidth_profile(host: Banks, pool: Banks, workers: Optional[HostPool], n_experts: int,
                      seconds: float = 1.0, threshold: float = 2.0, stream=None) -> dict:
    """Start-up bandwidth profile (synchronous): stand-alone and overlapped rates of the
    fill kernel and the host expert kernel, the fetched fraction and the backend."""
    out = BwProfile()
    _check("mc_bandwidth_profile", lib().mc_bandwidth_profile(
        C.byref(host), C.byref(pool), workers.handle if workers is not None else None, n_experts, seconds,
        threshold, _stream(stream), C.byref(out)))
    return {"pcie_gbs": out.pcie_gbs, "cpu_gbs": out.cpu_gbs, "pcie_ov_gbs": out.pcie_ov_gbs,
            "cpu_ov_gbs": out.cpu_ov_gbs, "expert_bytes": out.expert_bytes, "frac_q16": out.frac_q16,
            "backend": "hybrid" if out.hybrid else "offload", "threshold": threshold}
