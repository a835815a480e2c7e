"""GPU parity on the configurations' own settings: the DeepSeek-V4-Flash-shaped cache
(43 layers x 256 experts, 1500 slots) under every fetch fraction and locality of its
runs, a captured batched step replayed with a device valid count that changes between
replays ([jjl357] "8.2": fixed shapes, device-side valid counts), and a decode layer whose
misses all run on the CPU (no fill at all)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_bf16_close, empty_device_banks, pinned_banks, rel_l2, t_of
from oracle import LruOracle, decode_layer, hybrid_partials, route
from test_gpu_route_lookup import GpuLookup, _compare_state

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ratio", [1.5, 2.0, 3.0])
@pytest.mark.parametrize("p", [0.5, 0.9])
def test_lookup_dsv4_cache_config(ratio, p):
    """43 x 256 experts over 1500 slots, fetched fraction f = 1/ratio (B_H/B_P = ratio),
    min_fill 1: every call's slots, fill list and host list bit-exact, the whole state
    (slot_of, id_of, stamps, clock, stats) after every step of 43 calls."""
    from expert_cache_offloaded_amd import fetch_fraction_q16
    # at locality 0.5 about one fill per call at f = 1/3: 44 steps wrap the 1500 slots
    cfg = synth.CONFIGS["dsv4_hybrid"].with_(p=p, steps=44 if p == 0.5 else 16)
    tr = synth.trace(cfg)
    frac = fetch_fraction_q16(1.0, ratio)
    g = GpuLookup(cfg.L, cfg.E, cfg.S, 1, cfg.k)
    o = LruOracle(cfg.L, cfg.E, cfg.S)
    calls = 0
    for s in range(cfg.steps):
        for l in range(cfg.L):
            a = g(l, tr[s, l], frac, 1, 1)
            b = o.lookup(l, tr[s, l], frac, 1, 1)
            assert np.array_equal(a["slots"], b["slots"]), (s, l)
            assert a["fills"] == b["fills"] and a["host"] == b["host"], (s, l)
            calls += 1
        _compare_state(g, o)
    assert calls >= 64
    assert o.stats[3] > 0                        # misses ran on the host
    if p == 0.5:
        assert o.stats[4] > 0                    # the pool wrapped: evictions happened


def test_batched_step_graph_with_changing_valid_count():
    """A batched Zipf step (T = 16 capacity, 4 layers of the batched configuration's shape)
    captured once and replayed with the device valid count set to 16, 5, 0, 11, 1, 16 and
    new routes and activations: on every replay the cache state equals the oracle's, the
    outputs of the valid tokens match, and the rows beyond the count are zero."""
    from expert_cache_offloaded_amd.runtime import BankSet, CacheState, DecodeBuffers, DecodeLayer
    cfg = synth.CONFIGS["zipf_decode"].with_(L=4, T=16, S=320, steps=7)
    tr = synth.trace(cfg)
    host_np = synth.host_pool(cfg)
    host = BankSet(pinned_banks(cfg, host_np), cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(empty_device_banks(cfg, cfg.S), cfg.H, cfg.I, cfg.fmt)
    cs = CacheState(cfg.L, cfg.E, cfg.S)
    cs.reset()
    layers = [DecodeLayer(cs, host, pool, None, DecodeBuffers(cfg.T, cfg.k, cfg.H, cfg.I))
              for _ in range(cfg.L)]
    lg_buf = torch.empty((cfg.L, cfg.T, cfg.E), dtype=torch.float32, device="cuda")
    x_buf = torch.empty((cfg.L, cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    n_tok = torch.full((1,), cfg.T, dtype=torch.int32, device="cuda")
    o = LruOracle(cfg.L, cfg.E, cfg.S)
    counts = [16, 16, 5, 0, 11, 1, 16]

    def load(s):
        lgs = synth.step_logits(cfg, tr[s], s)
        xs = np.stack([synth.activations(cfg, s, l) for l in range(cfg.L)])
        lg_buf.copy_(torch.from_numpy(lgs))
        x_buf.copy_(torch.from_numpy(xs.view(np.int16)))
        n_tok.fill_(counts[s])
        return lgs, xs

    def run():
        for l in range(cfg.L):
            layers[l](l, lg_buf[l], x_buf[l], n_tok=n_tok)

    def check(s, lgs, xs):
        torch.cuda.synchronize()
        nt = counts[s]
        for l in range(cfg.L):
            ids, w = route(lgs[l], cfg.k)
            res = o.lookup(l, ids, 1 << 16, 1, 1, n_tok=nt)
            assert np.array_equal(layers[l].b.slots.cpu().numpy(), res["slots"]), (s, l)
            ref = decode_layer(xs[l], ids, w, host_np, l, cfg.E, cfg.fmt, cfg.H, cfg.I, n_tok=nt)
            y = layers[l].b.y
            if nt:
                assert_bf16_close(y[:nt], ref[:nt], "replay %d layer %d" % (s, l))
            assert torch.all(y[nt:] == 0)
        st = cs.state()
        for key in ("slot_of", "id_of", "stamp"):
            assert np.array_equal(st[key], getattr(o, key))
        assert np.array_equal(st["stats"], o.stats) and int(st["clock"][0]) == o.clock

    lgs, xs = load(0)
    run()                                        # eager first step (the capture's warm-up)
    check(0, lgs, xs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for s in range(1, cfg.steps):
        lgs, xs = load(s)
        g.replay()
        check(s, lgs, xs)
    assert o.stats[4] > 0                        # fills evicted residents during the replays
    del g


def test_every_miss_on_the_cpu():
    """The pure-CPU expert path ([jjl357] "8.5"): fixed-cap mode with cap 0 and no minimum
    fill gives q = 0, so every miss is computed on the host and nothing is ever filled; the
    layer still equals the unsplit definition."""
    from expert_cache_offloaded_amd import HostPool
    from expert_cache_offloaded_amd.runtime import BankSet, CacheState, DecodeBuffers, DecodeLayer
    cfg = synth.CONFIGS["qwen_decode"].with_(L=3, E=32, S=16, steps=3)
    tr = synth.trace(cfg)
    host_np = synth.host_pool(cfg)
    sh_np = synth.shared_pool(cfg)
    host = BankSet(pinned_banks(cfg, host_np), cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(empty_device_banks(cfg, cfg.S), cfg.H, cfg.I, cfg.fmt)
    shared = BankSet({k: t_of(v).cuda() for k, v in sh_np.items()}, cfg.H, cfg.I, cfg.fmt)
    cs = CacheState(cfg.L, cfg.E, cfg.S)
    cs.reset()
    hp = HostPool(4)
    dl = DecodeLayer(cs, host, pool, shared, DecodeBuffers(1, cfg.k, cfg.H, cfg.I), frac_q16=0,
                     fixed_cap=0, min_fill=0, hybrid=True, host_pool=hp)
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
            res = o.lookup(l, ids, 0, 0, 0)
            assert np.array_equal(dl.b.slots.cpu().numpy(), res["slots"])
            assert np.all(res["slots"] == -1)                # nothing is ever resident
            ref = decode_layer(x, ids, w, host_np, l, cfg.E, cfg.fmt, cfg.H, cfg.I, shared=sh_np)
            assert_bf16_close(y, ref, "step %d layer %d" % (s, l))
            yg, yh, _, _ = hybrid_partials(x, ids, res["slots"], w, host_np, l, cfg.E, cfg.fmt, cfg.H, cfg.I)
            assert rel_l2(dl.b.y_host.cpu().numpy(), yh) <= 1e-4
    st = cs.state()
    assert int(st["stats"][2]) == 0 and int(st["stats"][4]) == 0     # no fill, no eviction
    assert int(st["stats"][3]) == int(st["stats"][1]) > 0             # every miss on the host
    dl.stage.close()
    hp.close()
