"""GPU parity at full size, in the launch configuration bench.py times: the Qwen3.6-shaped
decode (40 MoE layers, E=256 top-8 + one shared expert, H 2048, I 512, MXFP4, bs 1, an LRU
pool of 600 of the 10 240 slots, locality 0.8), one captured hipGraph per 40-layer step,
replayed with each step's logits and activations copied in; the fills carried by the gate_up
launch (the default) and copied by their own kernel first.

After every replay: every layer's slot rewrite and the whole cache state (slot_of, id_of,
stamp, clock, stats) against the oracle LRU, bit for bit, and the bf16 outputs of four
layers (a different four each step; the float64 oracle takes about a second per layer)
against the oracle's unsplit layer."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_bf16_close
from oracle import LruOracle, decode_layer

pytestmark = pytest.mark.gpu


def _pinned_pool(cfg):
    from expert_cache_offloaded_amd.runtime import alloc_banks
    banks = alloc_banks(cfg.n_flat, cfg.H, cfg.I, cfg.fmt, pin=True)
    views = {k: v.numpy() for k, v in banks.items()}

    def one(f):
        for k, a in synth.expert_weights(cfg, f).items():
            views[k][f] = a
    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(one, range(cfg.n_flat)))
    return banks, views


@pytest.fixture(scope="module")
def qwen_host():
    """The Qwen-shaped host banks (10 240 experts, 17 GB pinned), built once for the module."""
    cfg = synth.CONFIGS["qwen_decode"]
    host_t, host_np = _pinned_pool(cfg)
    yield cfg, host_t, host_np
    del host_t, host_np


@pytest.mark.parametrize("fill_mode", ["fused", "copy"])
def test_qwen_shaped_decode_graph_full_size(qwen_host, fill_mode):
    from expert_cache_offloaded_amd.runtime import BankSet, CacheState, DecodeBuffers, DecodeLayer, alloc_banks
    from oracle import route
    cfg, host_t, host_np = qwen_host
    steps = 8                  # 320 experts at step 0, ~64 new per step: the 600 slots wrap
    tr = synth.trace(cfg, steps=steps)
    logits = np.stack([synth.step_logits(cfg, tr[s], s) for s in range(steps)])          # [S, L, 1, E]
    xs = np.stack([np.stack([synth.activations(cfg, s, l) for l in range(cfg.L)]) for s in range(steps)])
    host = BankSet(host_t, cfg.H, cfg.I, cfg.fmt)
    sh_np = synth.shared_pool(cfg)
    shared = BankSet({k: torch.from_numpy(v).cuda() for k, v in sh_np.items()}, cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(alloc_banks(cfg.S, cfg.H, cfg.I, cfg.fmt, device="cuda"), cfg.H, cfg.I, cfg.fmt)
    cache = CacheState(cfg.L, cfg.E, cfg.S)
    cache.reset()
    layers = [DecodeLayer(cache, host, pool, shared, DecodeBuffers(1, cfg.k, cfg.H, cfg.I),
                          frac_q16=1 << 16, renorm=cfg.renorm, fill_mode=fill_mode) for _ in range(cfg.L)]
    logits_buf = torch.from_numpy(logits[0]).cuda()
    x_buf = torch.from_numpy(xs[0].view(np.int16)).cuda()

    def step():
        for l in range(cfg.L):
            layers[l](l, logits_buf[l], x_buf[l])

    o = LruOracle(cfg.L, cfg.E, cfg.S)

    def check(s):
        torch.cuda.synchronize()
        sampled = {(s * 7 + 10 * j) % cfg.L for j in range(4)}
        for l in range(cfg.L):
            ids, w = route(logits[s, l], cfg.k)
            res = o.lookup(l, ids, 1 << 16, 1, 1)
            assert np.array_equal(layers[l].b.slots.cpu().numpy(), res["slots"]), (s, l)
            if l in sampled:
                y_ref = decode_layer(xs[s, l], ids, w, host_np, l, cfg.E, cfg.fmt, cfg.H, cfg.I, shared=sh_np)
                assert_bf16_close(layers[l].b.y, y_ref, "step %d layer %d" % (s, l))
        st = cache.state()
        assert np.array_equal(st["slot_of"], o.slot_of) and np.array_equal(st["id_of"], o.id_of)
        assert np.array_equal(st["stamp"], o.stamp) and int(st["clock"][0]) == o.clock
        assert np.array_equal(st["stats"], o.stats), s

    # step 0 eagerly (also the capture's warm-up), then capture; the capture itself does
    # not run the kernels, so the cache advances only on replays
    step()
    check(0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for s in range(1, steps):
        logits_buf.copy_(torch.from_numpy(logits[s]))
        x_buf.copy_(torch.from_numpy(xs[s].view(np.int16)))
        g.replay()
        check(s)
    assert o.stats[2] > 0 and o.stats[4] > 0    # fills and evictions happened during the replays
    # every resident slot holds its host expert's bytes
    st = cache.state()
    res = np.nonzero(st["id_of"] >= 0)[0]
    sample = res[:: max(1, len(res) // 24)]
    for sl in sample:
        f = int(st["id_of"][sl])
        for name, arr in pool.t.items():
            assert torch.equal(arr[int(sl)].cpu(), torch.from_numpy(host_np[name][f])), (sl, name)
