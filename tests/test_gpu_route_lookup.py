"""GPU parity: moe_route and slot_cache_lookup_evict against the oracle (bit-exact ints)."""
import numpy as np
import pytest
import torch

import synth
from oracle import LruOracle, route

pytestmark = pytest.mark.gpu


def _route_gpu(lg, k, renorm):
    from expert_cache_offloaded_amd import moe_route
    T = lg.shape[0]
    d = torch.from_numpy(np.ascontiguousarray(lg, dtype=np.float32)).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe_route(d, k, renorm, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("renorm", [1, 0])
def test_route_trace_logits(renorm):
    for name in ("tiny", "qwen_decode", "zipf_decode"):
        cfg = synth.CONFIGS[name].with_(steps=3, T=4 if name != "qwen_decode" else 1)
        tr = synth.trace(cfg)
        for s in range(cfg.steps):
            lg = synth.step_logits(cfg, tr[s], s).reshape(-1, cfg.E)
            ids, w = _route_gpu(lg, cfg.k, renorm)
            rid, rw = route(lg, cfg.k, renorm)
            assert np.array_equal(ids, rid), name
            assert np.max(np.abs(w - rw) / np.maximum(rw, 1e-30)) < (2e-6 if renorm else 1e-5)


def test_route_prefill_and_edges():
    cfg = synth.CONFIGS["prefill"]
    lg = synth.uniform_logits(cfg)
    for renorm in (0, 1):
        ids, w = _route_gpu(lg, cfg.k, renorm)
        rid, rw = route(lg, cfg.k, renorm)
        assert np.array_equal(ids, rid)
        assert np.max(np.abs(w - rw)) < 2e-6
    r = np.random.default_rng(9)
    # ties, a single expert, the largest E, k = 32, a ragged T
    cases = [np.zeros((3, 16), np.float32),
             np.round(r.standard_normal((37, 64)) * 2).astype(np.float32),
             r.standard_normal((5, 1)).astype(np.float32),
             r.standard_normal((7, 1024)).astype(np.float32)]
    for lg, k in zip(cases, (4, 8, 1, 32)):
        ids, w = _route_gpu(lg, k, 1)
        rid, rw = route(lg, k, 1)
        assert np.array_equal(ids, rid)
        assert np.max(np.abs(w - rw)) < 2e-6


class GpuLookup:
    def __init__(self, L_, E, S, T, k):
        from expert_cache_offloaded_amd.runtime import CacheState
        self.cs = CacheState(L_, E, S)
        self.cs.reset()
        self.T, self.k = T, k
        i32 = dict(dtype=torch.int32, device="cuda")
        self.ids = torch.empty((T, k), **i32)
        self.slots = torch.empty((T, k), **i32)
        self.ff = torch.empty(T * k, **i32)
        self.fs = torch.empty(T * k, **i32)
        self.nf = torch.empty(1, **i32)
        self.hf = torch.empty(T * k, **i32)
        self.nh = torch.empty(1, **i32)
        self.ntok = torch.empty(1, **i32)

    def __call__(self, layer, ids, frac, cap=1, min_fill=1, n_tok=None):
        from expert_cache_offloaded_amd import slot_cache_lookup_evict
        self.ids.copy_(torch.from_numpy(ids))
        nt = None
        if n_tok is not None:
            self.ntok.fill_(n_tok)
            nt = self.ntok
        slot_cache_lookup_evict(self.cs.desc, layer, self.ids, nt, frac, cap, min_fill, self.slots,
                                self.ff, self.fs, self.nf, self.hf, self.nh)
        torch.cuda.synchronize()
        nf, nh = int(self.nf.item()), int(self.nh.item())
        return {"slots": self.slots.cpu().numpy(),
                "fills": list(zip(self.ff[:nf].cpu().tolist(), self.fs[:nf].cpu().tolist())),
                "host": self.hf[:nh].cpu().tolist()}


def _compare_state(g, o):
    st = g.cs.state()
    assert np.array_equal(st["slot_of"], o.slot_of)
    assert np.array_equal(st["id_of"], o.id_of)
    assert np.array_equal(st["stamp"], o.stamp)
    assert int(st["clock"][0]) == o.clock
    assert np.array_equal(st["stats"], o.stats)


@pytest.mark.parametrize("frac,cap", [(1 << 16, 1), (1 << 15, 1), (0, 1), (21845, 1), (1, 1)])
def test_lookup_tiny_trace(frac, cap):
    cfg = synth.CONFIGS["tiny"]
    tr = synth.trace(cfg)
    g = GpuLookup(cfg.L, cfg.E, cfg.S, cfg.T, cfg.k)
    o = LruOracle(cfg.L, cfg.E, cfg.S)
    for s in range(cfg.steps):
        ids = tr[s, 0]
        a = g(0, ids, frac, cap)
        b = o.lookup(0, ids, frac, cap, 1)
        assert np.array_equal(a["slots"], b["slots"]), s
        assert a["fills"] == b["fills"], s
        assert a["host"] == b["host"], s
        _compare_state(g, o)


def test_lookup_qwen_shaped_trace():
    cfg = synth.CONFIGS["qwen_decode"].with_(steps=40)
    tr = synth.trace(cfg)
    g = GpuLookup(cfg.L, cfg.E, cfg.S, 1, cfg.k)
    o = LruOracle(cfg.L, cfg.E, cfg.S)
    n = 0
    for s in range(cfg.steps):
        for l in range(cfg.L):
            a = g(l, tr[s, l], 1 << 16)
            b = o.lookup(l, tr[s, l], 1 << 16)
            assert np.array_equal(a["slots"], b["slots"])
            assert a["fills"] == b["fills"] and a["host"] == b["host"]
            n += 1
            if n % 64 == 0:
                _compare_state(g, o)
    _compare_state(g, o)
    assert o.stats[4] > 0          # the pool wrapped: evictions happened


@pytest.mark.parametrize("L_,E,S,steps", [(6, 256, 256, 12), (6, 256, 1024, 12), (12, 1024, 4096, 24),
                                          (12, 1024, 4097, 24)])
def test_lookup_zipf_batched_valid_count(L_, E, S, steps):
    """Pools up to 4096 slots keep the slot table in LDS, larger ones read it from global
    memory; the two cases at that edge wrap their pool (about 8000 fills) and evict."""
    cfg = synth.CONFIGS["zipf_decode"].with_(L=L_, steps=steps, T=16, S=S, E=E)
    tr = synth.trace(cfg)
    g = GpuLookup(cfg.L, cfg.E, cfg.S, cfg.T, cfg.k)
    o = LruOracle(cfg.L, cfg.E, cfg.S)
    r = np.random.default_rng(1)
    for s in range(cfg.steps):
        for l in range(cfg.L):
            nt = int(r.integers(0, cfg.T + 1))
            a = g(l, tr[s, l], 1 << 16, n_tok=nt)
            b = o.lookup(l, tr[s, l], 1 << 16, n_tok=nt)
            assert np.array_equal(a["slots"], b["slots"])
            assert a["fills"] == b["fills"] and a["host"] == b["host"]
        _compare_state(g, o)
    if S >= 4096:
        assert o.stats[4] > 0                  # the pool wrapped: evictions happened


def test_lookup_invalid_ids_and_masks():
    g = GpuLookup(2, 8, 3, 3, 2)
    o = LruOracle(2, 8, 3)
    ids = np.array([[0, -1], [9, 3], [-7, 5]], dtype=np.int32)     # -1 masked, 9 and -7 invalid
    for layer in (1, 0, 1):
        a = g(layer, ids, 1 << 16)
        b = o.lookup(layer, ids, 1 << 16)
        assert np.array_equal(a["slots"], b["slots"])
        assert a["fills"] == b["fills"] and a["host"] == b["host"]
        _compare_state(g, o)
    assert o.stats[6] == 6


def test_route_signed_zero_and_inf_ties():
    """-0 and +0 are equal logits (the lower id wins); -inf logits rank last."""
    lg = np.array([[0.0, -0.0, -0.0, 0.0, -np.inf, 1.0, -1.0, -np.inf],
                   [-0.0, -np.inf, 0.0, -np.inf, -0.0, -np.inf, -np.inf, -np.inf]], np.float32)
    for k in (3, 6, 8):
        ids, w = _route_gpu(lg, k, 1)
        rid, rw = route(lg, k, 1)
        assert np.array_equal(ids, rid), k
        assert np.max(np.abs(w - rw)) < 2e-6


@pytest.mark.parametrize("cname,T,S,steps", [("qwen_decode", 1, 600, 12), ("zipf_decode", 16, 512, 6),
                                              ("tiny", 4, 4, 32)])
def test_route_lookup_fused_equals_separate(cname, T, S, steps):
    """moe_route_lookup (one launch) against moe_route + slot_cache_lookup_evict on a
    second cache: ids, gates, slots, fill/host lists and the whole cache state bit for
    bit after every call; with a device valid count below T on the batched trace."""
    from expert_cache_offloaded_amd import moe_route, moe_route_lookup, slot_cache_lookup_evict
    from expert_cache_offloaded_amd.runtime import CacheState
    cfg = synth.CONFIGS[cname].with_(steps=steps, T=T, S=S, L=min(synth.CONFIGS[cname].L, 6))
    tr = synth.trace(cfg)
    i32 = dict(dtype=torch.int32, device="cuda")
    sides = []
    for _ in range(2):
        cs = CacheState(cfg.L, cfg.E, cfg.S)
        cs.reset()
        sides.append(dict(cs=cs, ids=torch.empty((T, cfg.k), **i32),
                          w=torch.empty((T, cfg.k), dtype=torch.float32, device="cuda"),
                          slots=torch.empty((T, cfg.k), **i32), ff=torch.empty(T * cfg.k, **i32),
                          fs=torch.empty(T * cfg.k, **i32), nf=torch.empty(1, **i32),
                          hf=torch.empty(T * cfg.k, **i32), nh=torch.empty(1, **i32)))
    ntok = torch.empty(1, **i32)
    r = np.random.default_rng(3)
    for s in range(cfg.steps):
        lgs = synth.step_logits(cfg, tr[s], s)
        for l in range(cfg.L):
            lg = torch.from_numpy(np.ascontiguousarray(lgs[l])).cuda()
            nt = None
            if T > 1 and s % 2:
                ntok.fill_(int(r.integers(0, T + 1)))
                nt = ntok
            a, b = sides
            frac = (1 << 16) if cname != "tiny" else (1 << 15)
            moe_route_lookup(lg, cfg.renorm, a["ids"], a["w"], a["cs"].desc, l, nt, frac, 1, 1, a["slots"],
                             a["ff"], a["fs"], a["nf"], a["hf"], a["nh"])
            moe_route(lg, cfg.k, cfg.renorm, b["ids"], b["w"])
            slot_cache_lookup_evict(b["cs"].desc, l, b["ids"], nt, frac, 1, 1, b["slots"], b["ff"], b["fs"],
                                    b["nf"], b["hf"], b["nh"])
            torch.cuda.synchronize()
            for key in ("ids", "w", "slots", "nf", "nh"):
                assert torch.equal(a[key], b[key]), (s, l, key)
            nf, nh = int(a["nf"].item()), int(a["nh"].item())
            assert torch.equal(a["ff"][:nf], b["ff"][:nf]) and torch.equal(a["fs"][:nf], b["fs"][:nf])
            assert torch.equal(a["hf"][:nh], b["hf"][:nh])
            sa, sb = a["cs"].state(), b["cs"].state()
            for key in sa:
                assert np.array_equal(sa[key], sb[key]), (s, l, key)


def _set_state(g, o, id_of, stamp, clock):
    """The same cache state on the device tables and the oracle."""
    L_, E, S = o.L, o.E, o.S
    slot_of = np.full(L_ * E, -1, dtype=np.int64)
    for sl, f in enumerate(id_of):
        if f >= 0:
            slot_of[f] = sl
    o.slot_of, o.id_of = slot_of.copy(), np.asarray(id_of, dtype=np.int64).copy()
    o.stamp, o.clock = np.asarray(stamp, dtype=np.int64).copy(), int(clock)
    o.stats = np.zeros(8, dtype=np.int64)
    t = g.cs.t
    t["slot_of"].copy_(torch.from_numpy(slot_of.astype(np.int32)))
    t["id_of"].copy_(torch.from_numpy(np.asarray(id_of, dtype=np.int32)))
    t["stamp"].copy_(torch.from_numpy(np.asarray(stamp, dtype=np.int64)))
    t["clock"].fill_(int(clock))
    t["stats"].zero_()


@pytest.mark.parametrize("clock,edge", [(1 << 32, 2), (1 << 32, 1), ((1 << 33) + 10, 1), ((1 << 40) + 3, 5)])
@pytest.mark.parametrize("S", [8, 4097])
def test_lookup_victims_at_large_clock(clock, edge, S):
    """Victim order when stamps lie up to 2^32 and more calls behind the clock: with every
    slot occupied and the oldest stamp clock - 2^32 + 2, the ages just fit 32 bits (a tie at
    the oldest included); at clock - 2^32 + 1 and beyond they do not (the exact rounds).
    A small pool and one above the fast path's size; tables bit-exact after every call."""
    L_, E, k = 2, 16, 2
    g = GpuLookup(L_, E, S, 1, k)
    o = LruOracle(L_, E, S)
    rng = np.random.default_rng(clock % 9973 + S + edge)
    id_of = np.full(S, -1, dtype=np.int64)
    stamp = np.zeros(S, dtype=np.int64)
    id_of[:8] = [0, 1, 2, 3, 16, 17, 18, 19]
    base = clock - (1 << 32)
    stamp[:8] = [base + edge, base + edge + 2, base + edge, clock - 5, clock - 7, clock - 7, clock - 3,
                 base + edge + 1]
    if S > 8:                                    # more resident experts, recent stamps
        extra = rng.permutation(np.arange(20, L_ * E))
        id_of[8:8 + len(extra)] = extra
        stamp[8:8 + len(extra)] = clock - rng.integers(1, 50, len(extra))
    _set_state(g, o, id_of, stamp, clock)
    for step in range(12):
        layer = step % L_
        ids = rng.choice(E, k, replace=False).astype(np.int32)[None, :]
        a = g(layer, ids, 1 << 16)
        b = o.lookup(layer, ids, 1 << 16)
        assert np.array_equal(a["slots"], b["slots"]), step
        assert a["fills"] == b["fills"] and a["host"] == b["host"], step
        _compare_state(g, o)
