"""GPU parity: fills, moe_experts_decode, hybrid split/merge and whole decode steps."""
import zlib

import numpy as np
import pytest
import torch

import synth
from oracle import LruOracle, decode_layer, hybrid_partials
from gpu_helpers import (assert_bf16_close, device_banks, empty_device_banks, pinned_banks, rel_l2,
                         t_of)

pytestmark = pytest.mark.gpu


def _desc(cfg, t):
    from expert_cache_offloaded_amd import make_banks
    return make_banks(cfg.fmt, cfg.H, cfg.I, t)


def _resident_case(cfg, T, n_slots, host_frac, seed, shared=False, layer=1, nt=None):
    """Routes of one layer call with their experts placed at random slots of a device pool.

    A fraction of the routes is marked host-side (slot -1).  Unused slots hold other
    experts so a wrong slot read cannot go unnoticed.
    """
    r = np.random.default_rng(seed)
    ids = np.stack([r.choice(cfg.E, cfg.k, replace=False) for _ in range(T)]).astype(np.int32)
    w = r.random((T, cfg.k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    flats = sorted({layer * cfg.E + int(e) for e in ids.ravel()})
    assert len(flats) <= n_slots
    slot_perm = r.permutation(n_slots)
    slot_of = {f: int(slot_perm[i]) for i, f in enumerate(flats)}
    fillers = [f for f in range(cfg.n_flat) if f not in slot_of][: n_slots - len(flats)]
    entry_flat = [None] * n_slots
    for f, s in slot_of.items():
        entry_flat[s] = f
    for s in range(n_slots):
        if entry_flat[s] is None:
            entry_flat[s] = fillers.pop()
    banks = synth.host_pool(cfg, entry_flat)               # entry s = expert entry_flat[s]
    slots = np.array([[slot_of[layer * cfg.E + int(e)] for e in row] for row in ids], dtype=np.int32)
    slots[r.random(slots.shape) < host_frac] = -1
    x = synth.activations(cfg, seed, T=T)
    sh = synth.shared_pool(cfg) if shared else None
    index_of = {f: i for i, f in enumerate(entry_flat)}.__getitem__
    y_gpu_ref, _, _, _ = hybrid_partials(x, ids, slots, w, banks, layer, cfg.E, cfg.fmt, cfg.H, cfg.I,
                                         n_tok=nt, index_of=index_of)
    if sh is not None:
        from oracle import bf16_to_f64, expert_ffn, expert_matrices
        wg, wu, wd = expert_matrices(sh, layer, cfg.fmt, cfg.H, cfg.I)
        n = T if nt is None else nt
        y_gpu_ref[:n] += expert_ffn(wg, wu, wd, bf16_to_f64(x[:n]))
    return dict(ids=ids, w=w, slots=slots, x=x, banks=banks, shared=sh, ref=y_gpu_ref, layer=layer)


def _run_decode(cfg, case, nt=None):
    from expert_cache_offloaded_amd import decode_ws_bytes, finish_bf16, moe_experts_decode
    T = case["ids"].shape[0]
    pool_t = device_banks(case["banks"])
    pool = _desc(cfg, pool_t)
    sh = None
    if case["shared"] is not None:
        sh_t = {k: t_of(v[case["layer"]:case["layer"] + 1]).cuda() for k, v in case["shared"].items()}
        sh = _desc(cfg, sh_t)
    x = t_of(case["x"]).cuda()
    slots = torch.from_numpy(case["slots"]).cuda()
    w = torch.from_numpy(case["w"]).cuda()
    ws = torch.zeros(decode_ws_bytes(T, cfg.k, cfg.H, cfg.I) // 4, dtype=torch.float32, device="cuda")
    y = torch.full((T, cfg.H), 7.0, dtype=torch.float32, device="cuda")    # overwritten
    ntt = None
    if nt is not None:
        ntt = torch.tensor([nt], dtype=torch.int32, device="cuda")
    yb = torch.empty((T, cfg.H), dtype=torch.int16, device="cuda")
    moe_experts_decode(x, slots, w, ntt, pool, sh, ws, y, accumulate=0, y_bf16=yb)
    # a second call accumulating on top doubles the result; the separate rounding pass
    # gives the same bf16 bits as the fused one
    y2 = y.clone()
    moe_experts_decode(x, slots, w, ntt, pool, sh, ws, y2, accumulate=1)
    yb2 = torch.empty_like(yb)
    finish_bf16(y, ntt, yb2)
    torch.cuda.synchronize()
    assert torch.equal(yb, yb2)
    assert torch.allclose(y2, 2 * y, rtol=1e-6, atol=1e-6)
    return y.cpu().numpy(), yb


CASES = [
    # name, config, T, slots, host fraction, shared, shape overrides
    ("tiny-bf16", "tiny", 4, 8, 0.25, False, {}),
    ("qwen-mxfp4-bs1", "qwen_decode", 1, 24, 0.0, True, {}),
    ("qwen-mxfp4-bs1-split", "qwen_decode", 1, 24, 0.4, True, {}),
    ("zipf-mxfp4-bs4", "zipf_decode", 4, 40, 0.1, False, {}),
    ("zipf-mxfp4-bs16", "zipf_decode", 16, 130, 0.1, False, {}),
    ("dsv4-mxfp4-bs1", "dsv4_hybrid", 1, 8, 0.3, False, {}),
    # bf16 weights past the tiny shape: two 16-B chunks per lane in gate_up and down rows
    # of 128 chunks (64 lanes x 2), then four chunks per lane in gate_up
    ("bf16-h1024-i1024-bs3", "tiny", 3, 20, 0.2, True, dict(E=16, k=4, H=1024, I=1024)),
    ("bf16-h2048-i512-bs1", "tiny", 1, 12, 0.0, False, dict(E=12, k=3, H=2048, I=512)),
]


@pytest.mark.parametrize("name,cname,T,n_slots,hf,shared,shape", CASES)
def test_decode_matches_oracle(name, cname, T, n_slots, hf, shared, shape):
    cfg = synth.CONFIGS[cname].with_(L=2, **shape)
    case = _resident_case(cfg, T, n_slots, hf, seed=zlib.crc32(name.encode()) % 1000, shared=shared)
    y, yb = _run_decode(cfg, case)
    assert rel_l2(y, case["ref"]) <= 1e-4, name              # fp32 partial (diagnostic bar)
    assert_bf16_close(yb, case["ref"], name)                  # bf16 output bar


def test_decode_max_routes_heavy_sharing():
    """1024 routes (64 tokens x 16) over 32 experts: every unit is routed by ~32 tokens
    spread over all sixteen 64-route groups, and a fifth of the routes are host-side."""
    cfg = synth.CONFIGS["zipf_decode"].with_(L=2, E=32, k=16, H=256, I=128)
    case = _resident_case(cfg, 64, 40, 0.2, seed=11, shared=True)
    assert len(np.unique(case["slots"][case["slots"] >= 0])) <= 32
    y, yb = _run_decode(cfg, case)
    assert rel_l2(y, case["ref"]) <= 1e-4
    assert_bf16_close(yb, case["ref"], "max-routes")


def test_decode_valid_count_and_empty():
    cfg = synth.CONFIGS["zipf_decode"].with_(L=2)
    for nt in (0, 5, 16):
        case = _resident_case(cfg, 16, 130, 0.0, seed=7, nt=nt)
        y, yb = _run_decode(cfg, case, nt=nt)
        assert np.all(y[nt:] == 0)
        if nt:
            assert rel_l2(y[:nt], case["ref"][:nt]) <= 1e-4
            assert_bf16_close(yb[:nt], case["ref"][:nt])
        assert torch.all(yb[nt:] == 0)


def test_fill_copies_every_bank():
    from expert_cache_offloaded_amd import fill_slots
    for cname in ("tiny", "qwen_decode"):
        cfg = synth.CONFIGS[cname].with_(L=1, E=24) if cname == "qwen_decode" else synth.CONFIGS[cname]
        host_np = synth.host_pool(cfg)
        host_t = pinned_banks(cfg, host_np)
        host = _desc(cfg, host_t)
        S = 6
        pool_t = empty_device_banks(cfg, S)
        for v in pool_t.values():
            v.fill_(0)
        pool = _desc(cfg, pool_t)
        flats = [3, 0, cfg.n_flat - 1, 5]
        slots = [4, 1, 0, 5]
        n = 3                                   # the 4th entry is beyond n_fill and must not move
        ff = torch.tensor(flats, dtype=torch.int32, device="cuda")
        fs = torch.tensor(slots, dtype=torch.int32, device="cuda")
        nf = torch.tensor([n], dtype=torch.int32, device="cuda")
        fill_slots(host, pool, ff, fs, nf)
        torch.cuda.synchronize()
        for name, arr in pool_t.items():
            got = arr.cpu()
            for i in range(4):
                want = t_of(host_np[name][flats[i]]) if i < n else torch.zeros_like(got[slots[i]])
                assert torch.equal(got[slots[i]], want), (cname, name, i)
            for s in (2, 3):
                assert torch.all(got[s] == 0)


def _step_oracle(cfg, o, layer, ids, w, x, banks, frac, shared=None):
    res = o.lookup(layer, ids, frac, 1, 1)
    y = decode_layer(x, ids, w, banks, layer, cfg.E, cfg.fmt, cfg.H, cfg.I, shared=shared)
    return res, y


@pytest.mark.parametrize("frac,fill_mode", [(1 << 16, "copy"), (1 << 15, "copy"), (1 << 16, "through"),
                                            (1 << 15, "through"), (1 << 15, "split"), (1 << 16, "fused"),
                                            (1 << 15, "fused")])
def test_tiny_trace_end_to_end(frac, fill_mode):
    """The tiny config through route -> lookup -> split -> fill -> experts -> merge, every step
    (4 slots for up to 8 unique experts: overflow misses run on the host branch)."""
    from expert_cache_offloaded_amd import HostPool
    from expert_cache_offloaded_amd.runtime import BankSet, CacheState, DecodeBuffers, DecodeLayer
    from oracle import route
    cfg = synth.CONFIGS["tiny"]
    tr = synth.trace(cfg)
    host_np = synth.host_pool(cfg)
    host = BankSet(pinned_banks(cfg, host_np), cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(empty_device_banks(cfg, cfg.S), cfg.H, cfg.I, cfg.fmt)
    cs = CacheState(cfg.L, cfg.E, cfg.S)
    cs.reset()
    hp = HostPool(2)
    dl = DecodeLayer(cs, host, pool, None, DecodeBuffers(cfg.T, cfg.k, cfg.H, cfg.I), frac_q16=frac,
                     hybrid=True, host_pool=hp, fill_mode=fill_mode)
    o = LruOracle(cfg.L, cfg.E, cfg.S)
    x_dev = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    for s in range(cfg.steps):
        lg = synth.step_logits(cfg, tr[s], s)[0]
        x = synth.activations(cfg, s)
        x_dev.copy_(t_of(x))
        y = dl(0, torch.from_numpy(lg).cuda(), x_dev)
        torch.cuda.synchronize()
        ids, w = route(lg, cfg.k)
        res, yref = _step_oracle(cfg, o, 0, ids, w, x, host_np, frac)
        assert np.array_equal(dl.b.slots.cpu().numpy(), res["slots"]), s
        assert_bf16_close(y, yref, "step %d" % s)
    st = cs.state()
    assert np.array_equal(st["stats"], o.stats) and np.array_equal(st["slot_of"], o.slot_of)
    # every slot equals its host bank (a fill never corrupts a resident expert)
    for sl in range(cfg.S):
        f = int(st["id_of"][sl])
        if f >= 0:
            for name, arr in pool.t.items():
                assert torch.equal(arr[sl].cpu(), t_of(host_np[name][f]))
    hp.close()


@pytest.mark.parametrize("ratio,p,fill_mode", [(1.5, 0.5, "copy"), (2.0, 0.5, "copy"), (1.5, 0.9, "copy"),
                                               (3.0, 0.9, "copy"), (2.0, 0.9, "fused")])
def test_dsv4_shaped_hybrid_steps(ratio, p, fill_mode):
    """DeepSeek-V4-Flash expert shapes (H 4096, I 2048, MXFP4, top-6) on a reduced pool of
    E=16 experts x 3 layers, split by q* with B_H/B_P = ratio; y against the unsplit layer
    (fills copied first, or carried by the gate_up launch)."""
    from expert_cache_offloaded_amd import HostPool, fetch_fraction_q16
    from expert_cache_offloaded_amd.runtime import BankSet, CacheState, DecodeBuffers, DecodeLayer
    from oracle import route
    cfg = synth.CONFIGS["dsv4_hybrid"].with_(L=3, E=16, S=10, steps=2, p=p)
    tr = synth.trace(cfg)
    host_np = synth.host_pool(cfg)
    host = BankSet(pinned_banks(cfg, host_np), cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(empty_device_banks(cfg, cfg.S), cfg.H, cfg.I, cfg.fmt)
    cs = CacheState(cfg.L, cfg.E, cfg.S)
    cs.reset()
    frac = fetch_fraction_q16(1.0, ratio)
    hp = HostPool(4)
    dl = DecodeLayer(cs, host, pool, None, DecodeBuffers(1, cfg.k, cfg.H, cfg.I), frac_q16=frac,
                     hybrid=True, host_pool=hp, fill_mode=fill_mode)
    o = LruOracle(cfg.L, cfg.E, cfg.S)
    x_dev = torch.empty((1, cfg.H), dtype=torch.int16, device="cuda")
    for s in range(cfg.steps):
        lgs = synth.step_logits(cfg, tr[s], s)
        for l in range(cfg.L):
            x = synth.activations(cfg, s, l)
            x_dev.copy_(t_of(x))
            y = dl(l, torch.from_numpy(lgs[l]).cuda(), x_dev)
            torch.cuda.synchronize()
            ids, w = route(lgs[l], cfg.k)
            res = o.lookup(l, ids, frac, 1, 1)
            assert np.array_equal(dl.b.slots.cpu().numpy(), res["slots"])
            n_host = int(dl.b.n_host.item())
            assert n_host == len(res["host"])
            # the two partials (their sum is the unsplit layer, pinned in the oracle tests)
            yg, yh, _, _ = hybrid_partials(x, ids, res["slots"], w, host_np, l, cfg.E, cfg.fmt, cfg.H, cfg.I)
            assert_bf16_close(y, yg + yh, "step %d layer %d" % (s, l))
            assert rel_l2(dl.b.y_acc.cpu().numpy(), yg) <= 1e-4
            if n_host:
                assert rel_l2(dl.b.y_host.cpu().numpy(), yh) <= 1e-4
    assert o.stats[3] > 0          # some misses did run on the host
    hp.close()


def test_hybrid_step_in_a_graph():
    """The hybrid split and merge enqueue kernels only (the host branch is served from the
    stage by the worker pool's dispatcher): a captured 3-layer step, replayed with new
    routes and activations, matches the oracle on every replay, and no merge wait runs out."""
    from expert_cache_offloaded_amd import HostPool
    from expert_cache_offloaded_amd.runtime import BankSet, CacheState, DecodeBuffers, DecodeLayer
    from oracle import route
    cfg = synth.CONFIGS["dsv4_hybrid"].with_(L=3, E=16, S=10, steps=6, p=0.5)
    tr = synth.trace(cfg)
    host_np = synth.host_pool(cfg)
    host = BankSet(pinned_banks(cfg, host_np), cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(empty_device_banks(cfg, cfg.S), cfg.H, cfg.I, cfg.fmt)
    cs = CacheState(cfg.L, cfg.E, cfg.S)
    cs.reset()
    frac = 1 << 15
    hp = HostPool(4)
    layers = [DecodeLayer(cs, host, pool, None, DecodeBuffers(1, cfg.k, cfg.H, cfg.I), frac_q16=frac,
                          hybrid=True, host_pool=hp) for _ in range(cfg.L)]
    lg_buf = torch.empty((cfg.L, 1, cfg.E), dtype=torch.float32, device="cuda")
    x_buf = torch.empty((cfg.L, 1, cfg.H), dtype=torch.int16, device="cuda")
    o = LruOracle(cfg.L, cfg.E, cfg.S)
    steps = []

    def load(s):
        lgs = synth.step_logits(cfg, tr[s], s)
        xs = [synth.activations(cfg, s, l) for l in range(cfg.L)]
        lg_buf.copy_(torch.from_numpy(lgs))
        x_buf.copy_(torch.from_numpy(np.stack(xs).view(np.int16)))
        steps.append((lgs, xs))

    def run():
        for l in range(cfg.L):
            layers[l](l, lg_buf[l], x_buf[l])

    def check():
        torch.cuda.synchronize()
        lgs, xs = steps[-1]
        for l in range(cfg.L):
            ids, w = route(lgs[l], cfg.k)
            res = o.lookup(l, ids, frac, 1, 1)
            assert np.array_equal(layers[l].b.slots.cpu().numpy(), res["slots"])
            yg, yh, _, _ = hybrid_partials(xs[l], ids, res["slots"], w, host_np, l, cfg.E, cfg.fmt, cfg.H, cfg.I)
            assert_bf16_close(layers[l].b.y, yg + yh, "replay %d layer %d" % (len(steps) - 1, l))

    load(0)
    run()                                   # eager first step (also the capture's warm-up)
    check()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for s in range(1, cfg.steps):
        load(s)
        g.replay()
        check()
    assert o.stats[3] > 0                   # some misses ran on the host during the replays
    assert all(dl.stage.errors() == 0 for dl in layers)
    del g
    for dl in layers:
        dl.stage.close()
    hp.close()


def test_hybrid_stage_must_be_coherent():
    """A stage of ordinary pinned memory is refused: its GPU and host stores need not be
    visible to each other while a kernel runs."""
    from expert_cache_offloaded_amd import _lib as L
    from expert_cache_offloaded_amd import HostPool, make_banks
    cfg = synth.CONFIGS["tiny"]
    host_np = synth.host_pool(cfg)
    host = make_banks(cfg.fmt, cfg.H, cfg.I, pinned_banks(cfg, host_np))
    T, k = 1, cfg.k
    i32 = dict(dtype=torch.int32, device="cuda")
    x = torch.zeros((T, cfg.H), dtype=torch.int16, device="cuda")
    ids, slots = torch.zeros((T, k), **i32), torch.full((T, k), -1, **i32)
    w = torch.full((T, k), 0.5, dtype=torch.float32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    stage = torch.zeros(L.hybrid_stage_bytes(T, k, cfg.H), dtype=torch.uint8, pin_memory=True)
    hp = HostPool(2)
    hy = L.make_hybrid(x, ids, slots, w, 0, cfg.E, None, host, hp, stage, torch.empty((T, k), **f32),
                       torch.empty((T, k), **i32), torch.zeros((T, cfg.H), **f32), torch.zeros((T, cfg.H), **f32),
                       torch.empty((T, cfg.H), dtype=torch.int16, device="cuda"))
    with pytest.raises(RuntimeError, match="mc_hybrid_stage_alloc"):
        L.hybrid_split_merge(hy, L.MC_SPLIT_SUBMIT)
    hp.close()


@pytest.mark.parametrize("cname,T,steps,fmt", [("qwen_decode", 1, 4, None), ("zipf_decode", 4, 3, None),
                                               ("dsv4_hybrid", 1, 2, None), ("qwen_decode", 1, 3, "bf16")])
def test_fill_through_equals_fill_then_decode(cname, T, steps, fmt):
    """Fill-through (the expert pass reads filled experts from the host and writes their
    slots), the split form (gate_up fills through while the down banks are copied on a
    side stream) and the fused form (gate_up fills through, the down banks copied by
    workgroups of the same launch) against the separate fill copy followed by the expert
    pass: outputs, slots and every resident pool byte identical after each layer call;
    outputs against the oracle."""
    from expert_cache_offloaded_amd.runtime import BankSet, CacheState, DecodeBuffers, DecodeLayer
    from oracle import route
    # S >= T*k keeps every miss fillable (no overflow to the host set)
    cfg = synth.CONFIGS[cname].with_(L=3, E=32, S=max(14, T * 8 + 6), steps=steps, T=T)
    if fmt is not None:            # bf16 rows of H = 2048: the widest one-token gate_up rows
        cfg = cfg.with_(fmt=fmt)
    tr = synth.trace(cfg)
    host_np = synth.host_pool(cfg)
    host = BankSet(pinned_banks(cfg, host_np), cfg.H, cfg.I, cfg.fmt)
    sh_np = synth.shared_pool(cfg) if cfg.shared else None
    shared = (BankSet({k: t_of(v).cuda() for k, v in sh_np.items()}, cfg.H, cfg.I, cfg.fmt)
              if sh_np is not None else None)
    runs = []
    for mode in ("through", "split", "fused", "copy"):
        pool = BankSet(empty_device_banks(cfg, cfg.S), cfg.H, cfg.I, cfg.fmt)
        cs = CacheState(cfg.L, cfg.E, cfg.S)
        cs.reset()
        dl = DecodeLayer(cs, host, pool, shared, DecodeBuffers(T, cfg.k, cfg.H, cfg.I),
                         frac_q16=1 << 16, renorm=cfg.renorm, fill_mode=mode)
        runs.append((pool, cs, dl))
    x_dev = torch.empty((T, cfg.H), dtype=torch.int16, device="cuda")
    n_fills = 0
    for s in range(cfg.steps):
        lgs = synth.step_logits(cfg, tr[s], s)
        for l in range(cfg.L):
            x = synth.activations(cfg, s, l, T=T)
            x_dev.copy_(t_of(x))
            lg = torch.from_numpy(lgs[l]).cuda()
            ys = [dl(l, lg, x_dev).clone() for _, _, dl in runs]
            torch.cuda.synchronize()
            n_fills += int(runs[0][2].b.n_fill.item())
            id_of = runs[0][1].t["id_of"].cpu().numpy()
            res = torch.from_numpy(np.nonzero(id_of >= 0)[0]).cuda()
            for other in runs[1:]:
                assert torch.equal(ys[0], ys[runs.index(other)]), (s, l)
                assert torch.equal(runs[0][2].b.slots, other[2].b.slots)
                # resident slots hold identical bytes (free slots are uninitialised memory)
                assert np.array_equal(id_of, other[1].t["id_of"].cpu().numpy())
                for name in runs[0][0].t:
                    assert torch.equal(runs[0][0].t[name][res], other[0].t[name][res]), (s, l, name)
            if l == 0:
                ids, w = route(lgs[l], cfg.k)
                yref = decode_layer(x, ids, w, host_np, l, cfg.E, cfg.fmt, cfg.H, cfg.I, shared=sh_np)
                assert_bf16_close(ys[0], yref, "step %d" % s)
    assert n_fills > 0
    st = runs[0][1].state()
    for sl in range(cfg.S):
        f = int(st["id_of"][sl])
        if f >= 0:
            for name, arr in runs[0][0].t.items():
                assert torch.equal(arr[sl].cpu(), t_of(host_np[name][f]))


def test_resize_pool_sweeps_in_one_run():
    """Elastic resize ([jjl357] "7.2"): one process walks a batched Zipf trace (bs 4,
    6 layers) through pools of 64, 160 and 96 slots, resizing at safe points.  Each
    segment starts cold and equals a fresh oracle LRU of that size bit for bit (slots,
    tables, stats); outputs against the oracle on the segment's first and last steps."""
    from expert_cache_offloaded_amd.runtime import (BankSet, CacheState, DecodeBuffers, DecodeLayer,
                                                   alloc_banks, resize_pool)
    from oracle import route
    cfg = synth.CONFIGS["zipf_decode"].with_(L=6, E=64, T=4, steps=9)
    tr = synth.trace(cfg)
    host_np = synth.host_pool(cfg)
    host = BankSet(pinned_banks(cfg, host_np), cfg.H, cfg.I, cfg.fmt)
    sizes = [64, 160, 96]
    pool = BankSet(alloc_banks(sizes[0], cfg.H, cfg.I, cfg.fmt, device="cuda"), cfg.H, cfg.I, cfg.fmt)
    cache = CacheState(cfg.L, cfg.E, sizes[0])
    cache.reset()
    layers = [DecodeLayer(cache, host, pool, None, DecodeBuffers(cfg.T, cfg.k, cfg.H, cfg.I), renorm=cfg.renorm)
              for _ in range(cfg.L)]
    x_dev = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    seg = cfg.steps // len(sizes)
    for i, S in enumerate(sizes):
        if i:
            cache, pool = resize_pool(layers, S)
        o = LruOracle(cfg.L, cfg.E, S)
        for s in range(i * seg, (i + 1) * seg):
            lgs = synth.step_logits(cfg, tr[s], s)
            for l in range(cfg.L):
                x = synth.activations(cfg, s, l)
                x_dev.copy_(t_of(x))
                y = layers[l](l, torch.from_numpy(lgs[l]).cuda(), x_dev)
                torch.cuda.synchronize()
                ids, w = route(lgs[l], cfg.k)
                res = o.lookup(l, ids, 1 << 16, 1, 1)
                assert np.array_equal(layers[l].b.slots.cpu().numpy(), res["slots"]), (S, s, l)
                if s in (i * seg, (i + 1) * seg - 1) and l % 3 == 0:
                    ref = decode_layer(x, ids, w, host_np, l, cfg.E, cfg.fmt, cfg.H, cfg.I)
                    assert_bf16_close(y, ref, "S %d step %d layer %d" % (S, s, l))
        st = cache.state()
        assert np.array_equal(st["stats"], o.stats) and np.array_equal(st["slot_of"], o.slot_of)
        assert np.array_equal(st["id_of"], o.id_of) and np.array_equal(st["stamp"], o.stamp)
        assert o.stats[2] > 0
