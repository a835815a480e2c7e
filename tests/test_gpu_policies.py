"""GPU: the cache policies the pages compare, on the library's own lookup kernel —
the cross-layer LRU and a static (prefill-time) placement kept fixed — against the
oracle, bit for bit, on the Qiita replay trace and on the Qwen-shaped trace."""
import numpy as np
import pytest
import torch

import synth
from oracle import LruOracle, static_miss_counts, static_resident_set

pytestmark = pytest.mark.gpu


def _run(cs, ids_dev, steps, L, frac, cap, min_fill, T, k):
    from expert_cache_offloaded_amd import slot_cache_lookup_evict
    i32 = dict(dtype=torch.int32, device="cuda")
    slots = torch.empty((T, k), **i32)
    ff, fs, hf = (torch.empty(T * k, **i32) for _ in range(3))
    nf, nh = torch.empty(1, **i32), torch.empty(1, **i32)
    for s in range(steps):
        for l in range(L):
            slot_cache_lookup_evict(cs.desc, l, ids_dev[s, l], None, frac, cap, min_fill, slots, ff, fs, nf,
                                    hf, nh)
    torch.cuda.synchronize()
    return cs.state()


def test_qiita_replay_lru_and_static():
    """[qiita] "5.": 64 of 256 slots on a trace of the page's process (locality 0.95): LRU
    (offload, every miss fetched) and the static placement of the 64 most frequent ids of
    the first 512 steps (no fill, no eviction).  Miss counts and tables equal the oracle's;
    the rates are the page's 3.8 % and 72.7 % within the golden files' tolerances."""
    from expert_cache_offloaded_amd import cache_install
    from expert_cache_offloaded_amd.runtime import CacheState, static_placement
    E, K, steps = 256, 8, 20000
    tr = synth.drifting_working_set(E, K, steps, 0.95, 20260825)
    ids_dev = torch.from_numpy(tr.reshape(steps, 1, 1, K)).cuda()
    # LRU
    cs = CacheState(1, E, 64)
    cs.reset()
    st = _run(cs, ids_dev, steps, 1, 1 << 16, 1, 1, 1, K)
    o = LruOracle(1, E, 64)
    for s in range(steps):
        o.lookup(0, tr[s:s + 1], 1 << 16, 1, 1)
    assert np.array_equal(st["stats"], o.stats)
    assert np.array_equal(st["slot_of"], o.slot_of) and np.array_equal(st["stamp"], o.stamp)
    lru_rate = o.stats[1] / (o.stats[0] + o.stats[1])
    # static: fixed placement, lookups that never fill or evict
    placed = static_placement(tr[:512], 64)
    assert placed.tolist() == static_resident_set(tr[:512], 64)
    cs2 = CacheState(1, E, 64)
    cs2.reset()
    cache_install(cs2.desc, torch.from_numpy(placed).cuda())
    st2 = _run(cs2, ids_dev, steps, 1, 0, 0, 0, 1, K)
    miss, acc = static_miss_counts(tr, placed)
    assert int(st2["stats"][1]) == miss and int(st2["stats"][0]) == acc - miss
    assert int(st2["stats"][2]) == 0 and int(st2["stats"][4]) == 0      # no fill, no eviction
    assert abs(100.0 * miss / acc - 72.7) <= 2.5 and abs(100.0 * lru_rate - 3.8) <= 0.15
    assert lru_rate < 0.05 < 0.7 < miss / acc


def test_qwen_shaped_lru_vs_static():
    """The Qwen-shaped trace (40 layers, E=256, top-8, locality 0.8) with 600 slots: LRU
    against a static placement of the 600 flat ids most routed over the first 64 steps,
    both on the device, both equal to the oracle's counts."""
    from expert_cache_offloaded_amd import cache_install
    from expert_cache_offloaded_amd.runtime import CacheState, static_placement
    cfg = synth.CONFIGS["qwen_decode"]
    steps, warm = 256, 64
    tr = synth.trace(cfg, steps=steps)                     # [steps, L, 1, k]
    ids_dev = torch.from_numpy(np.ascontiguousarray(tr)).cuda()
    flat = tr + (np.arange(cfg.L) * cfg.E)[None, :, None, None]
    cs = CacheState(cfg.L, cfg.E, cfg.S)
    cs.reset()
    st = _run(cs, ids_dev, steps, cfg.L, 1 << 16, 1, 1, 1, cfg.k)
    o = LruOracle(cfg.L, cfg.E, cfg.S)
    for s in range(steps):
        for l in range(cfg.L):
            o.lookup(l, tr[s, l], 1 << 16, 1, 1)
    assert np.array_equal(st["stats"], o.stats)
    placed = static_placement(flat[:warm], cfg.S)
    assert placed.tolist() == static_resident_set(flat[:warm], cfg.S)
    cs2 = CacheState(cfg.L, cfg.E, cfg.S)
    cs2.reset()
    cache_install(cs2.desc, torch.from_numpy(placed).cuda())
    st2 = _run(cs2, ids_dev, steps, cfg.L, 0, 0, 0, 1, cfg.k)
    miss, acc = static_miss_counts(flat.reshape(steps, -1), placed)
    assert int(st2["stats"][1]) == miss and int(st2["stats"][0]) == acc - miss
    print("qwen-shaped, 600 slots, %d steps: LRU miss %.4f, static miss %.4f"
          % (steps, o.stats[1] / (o.stats[0] + o.stats[1]), miss / acc))
