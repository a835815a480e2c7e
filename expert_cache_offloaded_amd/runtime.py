"""Device/host memory plumbing and the per-layer call sequence of the decode path.

torch allocates every buffer (device tensors, pinned host tensors) and provides the
stream; each step of the path is one call into ``libmc.so``:

  moe_route_lookup (= moe_route + slot_cache_lookup_evict) -> [hybrid_split_merge(SPLIT)]
            -> moe_experts_decode (its gate_up launch also carries the fill of the chosen
               misses, mc_fill_slots) -> [hybrid_split_merge(MERGE)]

which follows [jjl357] "6.8 CPU 与 GPU 并发执行的顺序" and [wanger] "代码全链路":
the host branch is started before the fills and the GPU experts, and the two
partials are merged at the end.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from . import _lib as L

_NP2T = {"uint8": torch.uint8, "uint16": torch.int16}


def bank_shapes(H: int, I: int, fmt: str):
    if fmt == "bf16":
        return {"gate_up": ((2 * I, H), torch.int16), "down": ((H, I), torch.int16)}
    return {"gate_up": ((2 * I, H // 2), torch.uint8), "gate_up_scale": ((2 * I, H // 32), torch.uint8),
            "down": ((H, I // 2), torch.uint8), "down_scale": ((H, I // 32), torch.uint8)}


def alloc_banks(n: int, H: int, I: int, fmt: str, device=None, pin: bool = False) -> Dict[str, torch.Tensor]:
    out = {}
    for name, (shp, dt) in bank_shapes(H, I, fmt).items():
        if device is not None and device != "cpu":
            out[name] = torch.empty((n,) + shp, dtype=dt, device=device)
        else:
            out[name] = torch.empty((n,) + shp, dtype=dt, pin_memory=pin)
    return out


class BankSet:
    """Tensors of one bank set plus its C descriptor."""

    def __init__(self, tensors: Dict[str, torch.Tensor], H: int, I: int, fmt: str):
        self.t, self.H, self.I, self.fmt = tensors, H, I, fmt
        self.desc = L.make_banks(fmt, H, I, tensors)

    @property
    def n(self) -> int:
        return self.t["gate_up"].shape[0]

    def entry(self, i: int) -> "BankSet":
        """A one-entry view (e.g. one layer's shared expert)."""
        return BankSet({k: v[i:i + 1] for k, v in self.t.items()}, self.H, self.I, self.fmt)


class CacheState:
    """Device tables of the cross-layer LRU (caller-owned memory)."""

    def __init__(self, L_: int, E: int, S: int, device="cuda"):
        self.L, self.E, self.S = L_, E, S
        self.t = {"slot_of": torch.empty(L_ * E, dtype=torch.int32, device=device),
                  "id_of": torch.empty(S, dtype=torch.int32, device=device),
                  "stamp": torch.empty(S, dtype=torch.int64, device=device),
                  "clock": torch.empty(1, dtype=torch.int64, device=device),
                  "stats": torch.empty(8, dtype=torch.int64, device=device)}
        self.desc = L.make_cache(L_, E, S, self.t)

    def reset(self, stream=None):
        L.cache_reset(self.desc, stream)

    def state(self) -> dict:
        return {k: v.cpu().numpy() for k, v in self.t.items()}


@dataclass
class DecodeBuffers:
    """Fixed-shape workspaces of one decode layer call (capacity T tokens x k routes)."""
    T: int
    k: int
    H: int
    I: int
    device: str = "cuda"

    def __post_init__(self):
        d, T, k = self.device, self.T, self.k
        i32 = dict(dtype=torch.int32, device=d)
        self.ids = torch.empty((T, k), **i32)
        self.w = torch.empty((T, k), dtype=torch.float32, device=d)
        self.slots = torch.empty((T, k), **i32)
        self.fill_flat = torch.empty(T * k, **i32)
        self.fill_slot = torch.empty(T * k, **i32)
        self.n_fill = torch.zeros(1, **i32)
        self.host_flat = torch.empty(T * k, **i32)
        self.n_host = torch.zeros(1, **i32)
        self.gpu_w = torch.empty((T, k), dtype=torch.float32, device=d)
        self.host_ids = torch.empty((T, k), **i32)
        self.y_acc = torch.empty((T, self.H), dtype=torch.float32, device=d)
        self.y_host = torch.empty((T, self.H), dtype=torch.float32, device=d)
        self.y = torch.empty((T, self.H), dtype=torch.int16, device=d)
        self.ws = torch.zeros(L.decode_ws_bytes(T, k, self.H, self.I) // 4 + 4, dtype=torch.float32, device=d)


class DecodeLayer:
    """Runs one decode layer call through the C ABI (offload or hybrid mode)."""

    def __init__(self, cache: CacheState, host: BankSet, pool: BankSet, shared: Optional[BankSet],
                 bufs: DecodeBuffers, frac_q16: int = 1 << 16, fixed_cap: int = 1, min_fill: int = 1,
                 renorm: int = 1, hybrid: bool = False, host_pool: Optional[L.HostPool] = None,
                 fill_mode: Optional[str] = None):
        self.cache, self.host, self.pool, self.shared, self.b = cache, host, pool, shared, bufs
        self.frac_q16, self.fixed_cap, self.min_fill, self.renorm = frac_q16, fixed_cap, min_fill, renorm
        self.hybrid = hybrid
        self.host_pool = host_pool
        if not hybrid and pool.n < bufs.T * bufs.k:
            # with fewer slots than routes a call can overflow misses to the host set,
            # which only the hybrid branch computes
            raise ValueError("offload mode needs at least T*k = %d slots (pool has %d); use hybrid"
                             % (bufs.T * bufs.k, pool.n))
        # how the chosen misses reach their slots:
        #   copy    mc_fill_slots, then the expert pass reads the slots
        #   through the expert pass reads the filled experts from the host and writes the slots
        #   split   the gate_up pass fills through its banks while mc_fill_slots_banks copies
        #           the down banks on a side stream; the down pass waits for that copy
        #   fused   the gate_up pass fills through its banks and its launch also copies the
        #           down banks (one launch, one stream); the down pass reads the slots
        # default: fused for one token (the measured fastest), copy for several (their gate_up
        # pass runs on the matrix cores, which would wait on host reads)
        if fill_mode is None:
            fill_mode = "fused" if bufs.T == 1 else "copy"
        if fill_mode not in ("copy", "through", "split", "fused"):
            raise ValueError("fill_mode must be copy, through, split or fused")
        self.fill_mode = fill_mode
        self.fill = None
        if fill_mode == "split":
            self.side = torch.cuda.Stream()
            self.ev_lookup = torch.cuda.Event()
            self.ev_fill = torch.cuda.Event()
            self.ev_fill.record()            # creates the event, so its handle can go in the list
            self.fill = L.make_fill_list(host.desc, bufs.fill_flat, bufs.fill_slot, bufs.n_fill,
                                         mode=L.MC_FILL_GATE_UP, down_after=self.ev_fill)
        elif fill_mode == "through":
            self.fill = L.make_fill_list(host.desc, bufs.fill_flat, bufs.fill_slot, bufs.n_fill)
        elif fill_mode == "fused":
            self.fill = L.make_fill_list(host.desc, bufs.fill_flat, bufs.fill_slot, bufs.n_fill,
                                         mode=L.MC_FILL_WITH_GATE_UP)
        if hybrid:
            self.stage = L.HybridStage(bufs.T, bufs.k, bufs.H)
        self._hy = {}
        self._sh = {}

    def __call__(self, layer: int, logits: torch.Tensor, x: torch.Tensor, n_tok=None, stream=None):
        """logits fp32 [T, E], x bf16 bits [T, H] (device) -> self.b.y (bf16 bits)."""
        b = self.b
        # route + lookup in one launch (same results as moe_route then slot_cache_lookup_evict)
        L.moe_route_lookup(logits, self.renorm, b.ids, b.w, self.cache.desc, layer, n_tok, self.frac_q16,
                           self.fixed_cap, self.min_fill, b.slots, b.fill_flat, b.fill_slot, b.n_fill,
                           b.host_flat, b.n_host, stream)
        if self.hybrid:
            key = (layer, x.data_ptr(), None if n_tok is None else n_tok.data_ptr())
            hy = self._hy.get(key)
            if hy is None:
                hy = L.make_hybrid(x, b.ids, b.slots, b.w, layer, self.cache.E, n_tok, self.host.desc,
                                   self.host_pool, self.stage, b.gpu_w, b.host_ids, b.y_acc, b.y_host, b.y)
                self._hy[key] = hy
            L.hybrid_split_merge(hy, L.MC_SPLIT_SUBMIT, stream)
            w_gpu = b.gpu_w
        else:
            w_gpu = b.w
        if self.fill_mode == "copy":
            L.fill_slots(self.host.desc, self.pool.desc, b.fill_flat, b.fill_slot, b.n_fill, stream)
        elif self.fill_mode == "split":
            cur = stream if stream is not None else torch.cuda.current_stream()
            self.ev_lookup.record(cur)
            self.side.wait_event(self.ev_lookup)
            L.fill_slots_banks(self.host.desc, self.pool.desc, b.fill_flat, b.fill_slot, b.n_fill,
                               L.MC_BANK_DOWN | L.MC_BANK_DOWN_SCALE, self.side)
            self.ev_fill.record(self.side)
        sh = self._shared_desc(layer)
        if self.hybrid:
            # GPU partial in fp32; the merge adds the host partial and rounds once
            L.moe_experts_decode(x, b.slots, w_gpu, n_tok, self.pool.desc, sh, b.ws, b.y_acc,
                                 accumulate=0, y_bf16=None, stream=stream, fill=self.fill)
            L.hybrid_split_merge(hy, L.MC_MERGE, stream)
        else:
            L.moe_experts_decode(x, b.slots, w_gpu, n_tok, self.pool.desc, sh, b.ws, b.y_acc,
                                 accumulate=0, y_bf16=b.y, stream=stream, fill=self.fill)
        return b.y

    def rebind(self, cache: "CacheState", pool: "BankSet") -> None:
        """Point this layer at a rebuilt cache and pool (after ``resize_pool``)."""
        if not self.hybrid and pool.n < self.b.T * self.b.k:
            raise ValueError("offload mode needs at least T*k = %d slots (pool has %d); use hybrid"
                             % (self.b.T * self.b.k, pool.n))
        self.cache, self.pool = cache, pool

    def _shared_desc(self, layer):
        if self.shared is None:
            return None
        d = self._sh.get(layer)
        if d is None:
            d = self._sh[layer] = self.shared.entry(layer)
        return d.desc


def save_bw_profile(path: str, profile: dict, fmt: str, gpu_name: str) -> None:
    """Store a bandwidth profile (from ``bandwidth_profile``) under (GPU, expert format):
    [wanger] "1. 启动时" — the engine looks the fraction up by the experts' format and the
    GPU at start-up.  JSON {gpu_name: {fmt: profile}}, merged into an existing file."""
    import json
    import os
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data.setdefault(gpu_name, {})[fmt] = profile
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    os.replace(tmp, path)


def load_fetch_fraction(path: str, fmt: str, gpu_name: str) -> int:
    """frac_q16 of the stored profile for (GPU, format), or 0 — the fixed-cap mode that
    [wanger] "1. 启动时" falls back to when there is no usable profile."""
    import json
    import os
    if not os.path.exists(path):
        return 0
    with open(path) as f:
        data = json.load(f)
    prof = data.get(gpu_name, {}).get(fmt)
    if not prof:
        return 0
    return int(prof.get("frac_q16", 0))


def static_placement(warm_ids, cap: int):
    """Static (prefill-time) placement: the `cap` flat ids routed most often over a
    warm-up window (host int array of any shape, one entry per routed id, occurrences
    counted), equal counts in the order of first appearance ([qiita] "5. デコード側の答え
    その1").  Returns int32 ids in rank order, for ``cache_install``."""
    flat = np.asarray(warm_ids, dtype=np.int64).ravel()
    flat = flat[flat >= 0]
    if flat.size == 0:
        return np.zeros(0, dtype=np.int32)
    vals, first, counts = np.unique(flat, return_index=True, return_counts=True)
    order = np.lexsort((first, -counts))         # count descending, then first appearance
    return vals[order[:cap]].astype(np.int32)


class PrefillRunner:
    """Prefill over the decode slot pool ([jjl357] "4.3 为什么不用三缓冲或更大缓存", "4.4").

    The layer buffers are slot ranges of the pool itself, so no separate staging
    memory exists and the experts still in them when prefill ends become decode's
    initial cache:
      * S >= 2E: whole-layer double buffer in slots [0, E) and [E, 2E) (layer l + 1
        streams host -> HBM on a copy stream while layer l computes);
      * S < 2E: two layers do not fit, so each layer loads only its routed experts, on
        demand, after its routing (the pages' fallback).  The routed experts are taken in
        groups of G = S // 2 that ping-pong between slots [0, G) and [G, 2G): group g + 1
        streams in on the copy stream while group g computes (S = 1: one slot, no
        overlap).  The layer runs as moe_experts_prefill_part steps — sort (which also
        gives the route counts, read back to the host), the experts of each group, one
        combine — and its output is bit-identical to the whole-layer call.
    After the last layer the experts left in the buffers are installed in the cache
    (mc_cache_install on the freshly reset tables)."""

    def __init__(self, cache: "CacheState", host: "BankSet", pool: "BankSet", T: int, k: int):
        E = cache.E
        if pool.n < 1:
            raise ValueError("prefill needs at least one slot")
        self.cache, self.host, self.pool, self.T, self.k = cache, host, pool, T, k
        self.double = pool.n >= 2 * E
        dev = pool.t["gate_up"].device
        if self.double:
            self.G, nb = E, 2
        else:
            self.G, nb = max(1, pool.n // 2), (2 if pool.n >= 2 else 1)
        self.bufs = [BankSet({n: v[b * self.G:(b + 1) * self.G] for n, v in pool.t.items()}, pool.H, pool.I,
                             pool.fmt) for b in range(nb)]
        self.ws = torch.empty(L.prefill_ws_bytes(T, k, E, pool.H, pool.I), dtype=torch.uint8, device=dev)
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        if not self.double:
            self.counts = torch.empty(E, dtype=torch.int32, device=dev)
            self.entry_of = torch.empty(((E + self.G - 1) // self.G, E), dtype=torch.int32, device=dev)
        self.groups = []            # per layer: the expert groups loaded (on-demand mode)

    def _copy_layer(self, layer: int, b: int, stream) -> None:
        E = self.cache.E
        with torch.cuda.stream(stream):
            for n, v in self.bufs[b].t.items():
                v.copy_(self.host.t[n][layer * E:(layer + 1) * E], non_blocking=True)

    def _copy_group(self, layer: int, experts, b: int, stream) -> None:
        """Host experts layer*E + experts[j] -> entry j of buffer b, one copy per run of
        consecutive ids and bank."""
        E = self.cache.E
        j = 0
        with torch.cuda.stream(stream):
            while j < len(experts):
                r = j
                while r + 1 < len(experts) and experts[r + 1] == experts[r] + 1:
                    r += 1
                f0 = layer * E + int(experts[j])
                for n, v in self.bufs[b].t.items():
                    v[j:r + 1].copy_(self.host.t[n][f0:f0 + r - j + 1], non_blocking=True)
                j = r + 1

    def run(self, logits, x, ys, renorm: int = 1):
        """logits: list of L device fp32 [T, E]; x: device bf16 bits [T, H]; ys: list of L
        device bf16 [T, H] outputs.  Resets the cache first; returns the installed ids
        (flat id per slot, -1 = left empty)."""
        Lc, E = self.cache.L, self.cache.E
        comp = torch.cuda.current_stream()
        self.cache.reset(comp)
        nb = len(self.bufs)
        copy = torch.cuda.Stream()
        done = [torch.cuda.Event() for _ in range(nb)]
        free = [torch.cuda.Event() for _ in range(nb)]
        held = [[] for _ in range(nb)]          # flat ids each buffer holds
        copy.wait_stream(comp)
        if self.double:
            self._copy_layer(0, 0, copy)
            done[0].record(copy)
            for layer in range(Lc):
                b = layer % 2
                comp.wait_event(done[b])
                nxt = None
                if layer + 1 < Lc:
                    copy.wait_event(free[1 - b])
                    nxt = L.make_prefetch(self.host.desc, (layer + 1) * E, self.bufs[1 - b].desc, copy)
                L.moe_route(logits[layer], self.k, renorm, self.ids, self.w, comp)
                L.moe_experts_prefill(x, self.ids, self.w, None, E, self.bufs[b].desc, self.ws, ys[layer], nxt,
                                      comp)
                if nxt is not None:
                    done[1 - b].record(copy)
                free[b].record(comp)
                held[b] = list(range(layer * E, (layer + 1) * E))
        else:
            self.groups = []
            G = self.G
            for layer in range(Lc):
                L.moe_route(logits[layer], self.k, renorm, self.ids, self.w, comp)
                L.moe_experts_prefill_part(x, self.ids, self.w, None, E, self.bufs[0].desc, None, L.PF_SORT,
                                           self.ws, counts=self.counts, stream=comp)
                routed = np.nonzero(self.counts.cpu().numpy())[0]      # waits for the sort
                groups = [routed[i:i + G] for i in range(0, len(routed), G)]
                self.groups.append(groups)
                eo = np.full((max(1, len(groups)), E), -1, dtype=np.int32)
                for g, grp in enumerate(groups):
                    eo[g, grp] = np.arange(len(grp), dtype=np.int32)
                self.entry_of[:len(eo)].copy_(torch.from_numpy(eo))
                # the layer's last group lands in the last buffer, so the residents left
                # at the end fill a prefix of the pool
                h0 = len(groups) % 2 if nb == 2 else 0
                for g, grp in enumerate(groups):
                    b = (h0 + g) % nb
                    copy.wait_event(free[b])
                    self._copy_group(layer, grp, b, copy)
                    done[b].record(copy)
                    comp.wait_event(done[b])
                    L.moe_experts_prefill_part(x, self.ids, self.w, None, E, self.bufs[b].desc, self.entry_of[g],
                                               L.PF_EXPERTS, self.ws, stream=comp)
                    free[b].record(comp)
                    held[b] = [layer * E + int(e) for e in grp]
                L.moe_experts_prefill_part(x, self.ids, self.w, None, E, self.bufs[0].desc, None, L.PF_COMBINE,
                                           self.ws, y=ys[layer], stream=comp)
        # the experts left in the buffers become the decode cache
        flats = []
        for b in range(nb):
            flats.extend(held[b] + [-1] * (self.G - len(held[b])))
        while flats and flats[-1] == -1:
            flats.pop()
        if flats:
            L.cache_install(self.cache.desc, torch.tensor(flats, dtype=torch.int32, device=self.ws.device), comp)
        return flats


def resize_pool(layers, new_S: int, stream=None):
    """Elastic resize of the expert slot pool at a safe point ([jjl357] "7.2 为什么只能在
    safe point 调整"): wait until no queued work can still use an old slot address, size a
    new pool of new_S slots, rebuild the cache tables empty, keep the host expert pool
    untouched, and let later misses refill the hot experts through the normal path.
    Rebinds every DecodeLayer of `layers` (they share one cache and pool) and returns
    (cache, pool); graphs captured against the old pool must be captured again."""
    if not layers:
        raise ValueError("resize_pool: no layers")
    torch.cuda.synchronize()                     # the safe point
    old = layers[0]
    L_, E = old.cache.L, old.cache.E
    pool = BankSet(alloc_banks(new_S, old.pool.H, old.pool.I, old.pool.fmt,
                               device=old.pool.t["gate_up"].device), old.pool.H, old.pool.I, old.pool.fmt)
    cache = CacheState(L_, E, new_S, device=old.cache.t["slot_of"].device)
    cache.reset(stream)
    for dl in layers:
        dl.rebind(cache, pool)
    return cache, pool
