"""GPU parity: prefill token sort, grouped GEMM layer, and the whole-layer double buffer."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_bf16_close, bf16_bits_to_f64, device_banks, pinned_banks, t_of
from oracle import bf16_to_f64, expert_ffn, expert_matrices, prefill_per_token, route, sort_routes

pytestmark = pytest.mark.gpu


def _sort_gpu(ids, E, n_tok=None):
    from expert_cache_offloaded_amd import _lib as L
    T, k = ids.shape
    d = torch.from_numpy(ids).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(E * 16 + (E + 1) * 4 + 256, dtype=torch.uint8, device="cuda")
    nt = None if n_tok is None else torch.tensor([n_tok], dtype=torch.int32, device="cuda")
    L.prefill_sort_routes(d, nt, E, ws, counts, offsets, perm)
    torch.cuda.synchronize()
    return counts.cpu().numpy(), offsets.cpu().numpy(), perm.cpu().numpy()


@pytest.mark.parametrize("T,k,E,n_tok", [(300, 6, 16, None), (301, 2, 8, 77), (8192, 6, 256, None),
                                         (5, 3, 1024, None), (64, 4, 32, 0)])
def test_sort_routes_bit_exact(T, k, E, n_tok):
    r = np.random.default_rng(T + E)
    ids = r.integers(0, E, size=(T, k)).astype(np.int32)
    ids[r.random(ids.shape) < 0.02] = -1
    ids[r.random(ids.shape) < 0.01] = E + 3          # invalid ids are left out
    c, o, p = _sort_gpu(ids, E, n_tok)
    rc, ro, rp = sort_routes(ids, E, n_tok)
    assert np.array_equal(c, rc) and np.array_equal(o, ro)
    assert np.array_equal(p[:ro[-1]], rp)


def _layer(cfg, E, layer=0, seed_shift=0):
    flats = [layer * cfg.E + e for e in range(E)]
    return synth.host_pool(cfg, flats)


def _run_prefill(cfg, x_bits, ids, w, banks_dev, E, n_tok=None):
    from expert_cache_offloaded_amd import _lib as L
    T, k = ids.shape
    buf = L.make_banks(cfg.fmt, cfg.H, cfg.I, banks_dev)
    ws = torch.empty(L.prefill_ws_bytes(T, k, E, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    y = torch.full((T, cfg.H), 0x7F7F, dtype=torch.int16, device="cuda")
    nt = None if n_tok is None else torch.tensor([n_tok], dtype=torch.int32, device="cuda")
    L.moe_experts_prefill(t_of(x_bits).cuda(), torch.from_numpy(ids).cuda(),
                          torch.from_numpy(w.astype(np.float32)).cuda(), nt, E, buf, ws, y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T,E,k,H,I,n_tok", [(200, 8, 2, 256, 128, None), (333, 16, 6, 512, 256, None),
                                             (97, 8, 3, 256, 256, 41), (1, 4, 2, 256, 128, None),
                                             # k at and past the combine's batched-read limit (8)
                                             (150, 16, 8, 256, 128, None), (90, 16, 10, 256, 128, 70)])
def test_prefill_small_layers(T, E, k, H, I, n_tok):
    cfg = synth.CONFIGS["prefill"].with_(L=1, E=E, k=k, H=H, I=I, T=T)
    banks = _layer(cfg, E)
    x = synth.activations(cfg, 0)
    lg = synth.uniform_logits(cfg)
    ids, w = route(lg, k)
    y = _run_prefill(cfg, x, ids, w.astype(np.float32), device_banks(banks), E, n_tok)
    n = T if n_tok is None else n_tok
    ref = prefill_per_token(x, ids, w.astype(np.float32).astype(np.float64), banks, E, cfg.fmt, H, I,
                            tokens=range(n))
    assert_bf16_close(y[:n], ref, "prefill T=%d E=%d" % (T, E))
    assert torch.all(y[n:] == 0)


def test_prefill_full_layer_sampled_and_deterministic():
    """The 8192-token, 256-expert, H 4096 / I 2048 MXFP4 layer: sampled tokens against the
    per-token definition; two runs bit-identical."""
    cfg = synth.CONFIGS["prefill"]
    E = cfg.E
    banks = _layer(cfg, E)
    dev = device_banks(banks)
    x = synth.activations(cfg, 0)
    lg = synth.uniform_logits(cfg)
    ids, w = route(lg, cfg.k)
    w32 = w.astype(np.float32)
    y1 = _run_prefill(cfg, x, ids, w32, dev, E)
    y2 = _run_prefill(cfg, x, ids, w32, dev, E)
    assert torch.equal(y1, y2)
    # every expert is routed (uniform routing over 8192 tokens)
    assert len(np.unique(ids)) == E
    sample = [0, 1, 4095, 8191, 3333, 777]
    cache = {}
    x64 = bf16_to_f64(x)
    ref = np.zeros((len(sample), cfg.H))
    for n, t in enumerate(sample):
        for j in range(cfg.k):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = expert_matrices(banks, e, cfg.fmt, cfg.H, cfg.I)
            wg, wu, wd = cache[e]
            ref[n] += float(w32[t, j]) * expert_ffn(wg, wu, wd, x64[t:t + 1])[0]
    got = y1[sample]
    assert_bf16_close(got, ref, "full-size prefill sample")


def test_double_buffer_equals_serialized():
    """Layers stream host -> HBM into two layer buffers on a copy stream while the
    previous layer computes; the outputs equal a serialized run bit for bit."""
    from expert_cache_offloaded_amd import _lib as L
    from expert_cache_offloaded_amd.runtime import alloc_banks
    cfg = synth.CONFIGS["prefill"].with_(L=3, E=16, k=4, H=512, I=256, T=512)
    host_np = synth.host_pool(cfg)
    host_t = pinned_banks(cfg, host_np)
    host = L.make_banks(cfg.fmt, cfg.H, cfg.I, host_t)
    bufs_t = [alloc_banks(cfg.E, cfg.H, cfg.I, cfg.fmt, device="cuda") for _ in range(2)]
    bufs = [L.make_banks(cfg.fmt, cfg.H, cfg.I, b) for b in bufs_t]
    x = t_of(synth.activations(cfg, 0)).cuda()
    routes = []
    for l in range(cfg.L):
        ids, w = route(synth.uniform_logits(cfg, layer=l), cfg.k)
        routes.append((torch.from_numpy(ids).cuda(), torch.from_numpy(w.astype(np.float32)).cuda()))
    ws = torch.empty(L.prefill_ws_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    comp = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    ys = [torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda") for _ in range(cfg.L)]
    # pipelined
    done = [torch.cuda.Event() for _ in range(2)]
    free = [torch.cuda.Event() for _ in range(2)]
    with torch.cuda.stream(copy):
        for name in bufs_t[0]:
            bufs_t[0][name].copy_(host_t[name][0:cfg.E], non_blocking=True)
        done[0].record(copy)
    for l in range(cfg.L):
        b = l % 2
        comp.wait_event(done[b])
        nxt = None
        if l + 1 < cfg.L:
            copy.wait_event(free[1 - b])
            nxt = L.make_prefetch(host, (l + 1) * cfg.E, bufs[1 - b], copy)
        L.moe_experts_prefill(x, routes[l][0], routes[l][1], None, cfg.E, bufs[b], ws, ys[l], nxt)
        if nxt is not None:
            done[1 - b].record(copy)
        free[b].record(comp)
    torch.cuda.synchronize()
    # serialized: copy, wait, compute
    for l in range(cfg.L):
        for name in bufs_t[0]:
            bufs_t[0][name].copy_(host_t[name][l * cfg.E:(l + 1) * cfg.E])
        y = torch.empty_like(ys[l])
        L.moe_experts_prefill(x, routes[l][0], routes[l][1], None, cfg.E, bufs[0], ws, y)
        torch.cuda.synchronize()
        assert torch.equal(y, ys[l]), l
        # and against the oracle on a few tokens
        ids = routes[l][0].cpu().numpy()
        w = routes[l][1].cpu().numpy().astype(np.float64)
        layer_np = {k: v[l * cfg.E:(l + 1) * cfg.E] for k, v in host_np.items()}
        ref = prefill_per_token(synth.activations(cfg, 0), ids, w, layer_np, cfg.E, cfg.fmt, cfg.H, cfg.I,
                                tokens=range(16))
        assert_bf16_close(y[:16], ref, "layer %d" % l)


@pytest.mark.parametrize("S", [32, 40, 24])
def test_prefill_runner_buffers_become_decode_cache(S):
    """Prefill over the decode slot pool ([jjl357] "4.3"): with S >= 2E the two layer
    buffers are pool slots (double buffer), with E <= S < 2E one buffer (no overlap).
    Outputs equal a standalone resident prefill bit for bit; afterwards the experts left
    in the buffers are the cache's residents (tables equal the oracle's install, slot
    bytes equal host truth) and a decode call on the last layer hits them all."""
    from expert_cache_offloaded_amd import _lib as L
    from expert_cache_offloaded_amd.runtime import (BankSet, CacheState, DecodeBuffers, DecodeLayer,
                                                   PrefillRunner, alloc_banks)
    from oracle import LruOracle, decode_layer
    cfg = synth.CONFIGS["prefill"].with_(L=3, E=16, k=4, H=512, I=256, T=512)
    host_np = synth.host_pool(cfg)
    host = BankSet(pinned_banks(cfg, host_np), cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(alloc_banks(S, cfg.H, cfg.I, cfg.fmt, device="cuda"), cfg.H, cfg.I, cfg.fmt)
    cache = CacheState(cfg.L, cfg.E, S)
    x = t_of(synth.activations(cfg, 0)).cuda()
    logits = [torch.from_numpy(synth.uniform_logits(cfg, layer=l)).cuda() for l in range(cfg.L)]
    ys = [torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda") for _ in range(cfg.L)]
    runner = PrefillRunner(cache, host, pool, cfg.T, cfg.k)
    assert runner.double == (S >= 2 * cfg.E)
    flats = runner.run(logits, x, ys)
    torch.cuda.synchronize()
    # outputs: a standalone prefill of each layer from its own resident buffer
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.prefill_ws_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    for l in range(cfg.L):
        buf = L.make_banks(cfg.fmt, cfg.H, cfg.I,
                           device_banks({k: v[l * cfg.E:(l + 1) * cfg.E] for k, v in host_np.items()}))
        L.moe_route(logits[l], cfg.k, 1, ids, w)
        y = torch.empty_like(ys[l])
        L.moe_experts_prefill(x, ids, w, None, cfg.E, buf, ws, y)
        torch.cuda.synchronize()
        assert torch.equal(y, ys[l]), l
    # the cache after prefill: the last one or two layers, installed where they sit
    last = [cfg.L - 1] if S < 2 * cfg.E else [cfg.L - 2, cfg.L - 1]
    want = []
    for b in range(len(last)):
        layer = [l for l in last if l % 2 == b][0] if len(last) == 2 else last[0]
        want.extend(range(layer * cfg.E, (layer + 1) * cfg.E))
    assert flats == want
    o = LruOracle(cfg.L, cfg.E, S)
    o.install(want)
    st = cache.state()
    assert np.array_equal(st["slot_of"], o.slot_of) and np.array_equal(st["id_of"], o.id_of)
    assert np.array_equal(st["stats"], o.stats)
    for sl, f in enumerate(want):
        for name, arr in pool.t.items():
            assert torch.equal(arr[sl].cpu(), t_of(host_np[name][f])), (sl, name)
    # decode on the last layer: every route hits the adopted experts
    dl = DecodeLayer(cache, host, pool, None, DecodeBuffers(1, cfg.k, cfg.H, cfg.I))
    lg = torch.from_numpy(synth.uniform_logits(cfg.with_(T=1), layer=cfg.L - 1)).cuda()
    xd = t_of(synth.activations(cfg, 1, T=1)).cuda()
    yd = dl(cfg.L - 1, lg, xd)
    torch.cuda.synchronize()
    st = cache.state()
    assert int(st["stats"][1]) == 0 and int(st["stats"][0]) == cfg.k      # hits only
    from oracle import route
    rid, rw = route(lg.cpu().numpy(), cfg.k)
    ref = decode_layer(synth.activations(cfg, 1, T=1), rid, rw, host_np, cfg.L - 1, cfg.E, cfg.fmt, cfg.H, cfg.I)
    assert_bf16_close(yd, ref, "decode after prefill")


def test_prefill_runner_needs_one_layer_of_slots():
    from expert_cache_offloaded_amd.runtime import BankSet, CacheState, PrefillRunner, alloc_banks
    cfg = synth.CONFIGS["prefill"].with_(L=2, E=16, k=4, H=512, I=256, T=64)
    host = BankSet(pinned_banks(cfg, synth.host_pool(cfg)), cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(alloc_banks(8, cfg.H, cfg.I, cfg.fmt, device="cuda"), cfg.H, cfg.I, cfg.fmt)
    with pytest.raises(ValueError):
        PrefillRunner(CacheState(cfg.L, cfg.E, 8), host, pool, cfg.T, cfg.k)
