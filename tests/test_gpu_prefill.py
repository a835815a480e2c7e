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


def _expected_residents(route_ids, E, S):
    """Where the on-demand runner leaves each layer's routed experts: ascending expert
    order, groups of G = S // 2 alternating between slots [0, G) and [G, 2G), each
    layer's last group in the second half (one slot, one buffer, when S = 1)."""
    G, nb = (S // 2, 2) if S >= 2 else (1, 1)
    held = [[] for _ in range(nb)]
    for l, ids in enumerate(route_ids):
        routed = np.unique(ids[ids >= 0])
        groups = [routed[i:i + G] for i in range(0, len(routed), G)]
        h0 = len(groups) % 2 if nb == 2 else 0
        for g, grp in enumerate(groups):
            held[(h0 + g) % nb] = [l * E + int(e) for e in grp]
    flats = []
    for h in held:
        flats.extend(h + [-1] * (G - len(h)))
    while flats and flats[-1] == -1:
        flats.pop()
    return flats


@pytest.mark.parametrize("S,T", [(32, 512), (40, 512), (24, 512), (8, 512), (5, 512), (1, 64), (6, 3),
                                 (16, 5), (24, 3)])
def test_prefill_runner_buffers_become_decode_cache(S, T):
    """Prefill over the decode slot pool ([jjl357] "4.3", "4.4"): with S >= 2E the two
    layer buffers are pool slots (double buffer); with S < 2E — also S < E — each layer
    loads only its routed experts on demand, in groups that ping-pong between two halves
    of the pool.  Outputs equal a standalone resident prefill bit for bit and the oracle
    on sampled tokens; afterwards the experts left in the buffers are the cache's
    residents (tables equal the oracle's install, slot bytes equal host truth), and a
    decode call on the last layer gives the oracle's lookup and output."""
    from expert_cache_offloaded_amd import _lib as L
    from expert_cache_offloaded_amd.runtime import (BankSet, CacheState, DecodeBuffers, DecodeLayer,
                                                   PrefillRunner, alloc_banks)
    from oracle import LruOracle, decode_layer, route
    cfg = synth.CONFIGS["prefill"].with_(L=3, E=16, k=4, H=512, I=256, T=T)
    host_np = synth.host_pool(cfg)
    host = BankSet(pinned_banks(cfg, host_np), cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(alloc_banks(S, cfg.H, cfg.I, cfg.fmt, device="cuda"), cfg.H, cfg.I, cfg.fmt)
    cache = CacheState(cfg.L, cfg.E, S)
    x_np = synth.activations(cfg, 0)
    x = t_of(x_np).cuda()
    logits_np = [synth.uniform_logits(cfg, layer=l) for l in range(cfg.L)]
    logits = [torch.from_numpy(a).cuda() for a in logits_np]
    ys = [torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda") for _ in range(cfg.L)]
    runner = PrefillRunner(cache, host, pool, cfg.T, cfg.k)
    assert runner.double == (S >= 2 * cfg.E)
    flats = runner.run(logits, x, ys)
    torch.cuda.synchronize()
    print("S=%d T=%d groups per layer %s" % (S, T, [len(g) for g in runner.groups]), flush=True)
    # outputs: a standalone prefill of each layer from its own resident buffer
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.prefill_ws_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    route_ids = []
    for l in range(cfg.L):
        buf = L.make_banks(cfg.fmt, cfg.H, cfg.I,
                           device_banks({k: v[l * cfg.E:(l + 1) * cfg.E] for k, v in host_np.items()}))
        L.moe_route(logits[l], cfg.k, 1, ids, w)
        y = torch.empty_like(ys[l])
        L.moe_experts_prefill(x, ids, w, None, cfg.E, buf, ws, y)
        torch.cuda.synchronize()
        assert torch.equal(y, ys[l]), l
        rid, rw = route(logits_np[l], cfg.k)
        assert np.array_equal(ids.cpu().numpy(), rid)
        route_ids.append(rid)
        layer_np = {k: v[l * cfg.E:(l + 1) * cfg.E] for k, v in host_np.items()}
        tok = range(min(cfg.T, 16))
        ref = prefill_per_token(x_np, rid, rw, layer_np, cfg.E, cfg.fmt, cfg.H, cfg.I, tokens=tok)
        assert_bf16_close(ys[l][:len(tok)], ref, "layer %d" % l)
    # the cache after prefill
    if S >= 2 * cfg.E:
        want = []
        for b in range(2):
            layer = [l for l in (cfg.L - 2, cfg.L - 1) if l % 2 == b][0]
            want.extend(range(layer * cfg.E, (layer + 1) * cfg.E))
    else:
        want = _expected_residents(route_ids, cfg.E, S)
        assert len(runner.groups) == cfg.L
        for l, groups in enumerate(runner.groups):      # only routed experts were loaded
            assert np.array_equal(np.concatenate(groups) if groups else np.zeros(0), np.unique(route_ids[l]))
    assert flats == want
    o = LruOracle(cfg.L, cfg.E, S)
    o.install(want)
    st = cache.state()
    assert np.array_equal(st["slot_of"], o.slot_of) and np.array_equal(st["id_of"], o.id_of)
    assert np.array_equal(st["stats"], o.stats)
    for sl, f in enumerate(want):
        if f < 0:
            continue
        for name, arr in pool.t.items():
            assert torch.equal(arr[sl].cpu(), t_of(host_np[name][f])), (sl, name)
    if S < cfg.k:
        return                      # offload decode needs k slots
    # decode on the last layer: lookup and output as the oracle's
    dl = DecodeLayer(cache, host, pool, None, DecodeBuffers(1, cfg.k, cfg.H, cfg.I))
    lg_np = synth.uniform_logits(cfg.with_(T=1), layer=cfg.L - 1)
    xd_np = synth.activations(cfg, 1, T=1)
    yd = dl(cfg.L - 1, torch.from_numpy(lg_np).cuda(), t_of(xd_np).cuda())
    torch.cuda.synchronize()
    rid, rw = route(lg_np, cfg.k)
    o.lookup(cfg.L - 1, rid, 1 << 16)
    st = cache.state()
    assert np.array_equal(st["slot_of"], o.slot_of) and np.array_equal(st["stats"], o.stats)
    if S >= 2 * cfg.E:
        assert int(st["stats"][1]) == 0 and int(st["stats"][0]) == cfg.k      # hits only
    ref = decode_layer(xd_np, rid, rw, host_np, cfg.L - 1, cfg.E, cfg.fmt, cfg.H, cfg.I)
    assert_bf16_close(yd, ref, "decode after prefill")


def test_prefill_part_steps_match_whole_layer():
    """moe_experts_prefill_part: the sort's route counts equal the oracle's; the experts
    step run over any partition of the routed experts — here three parts of a shuffled
    order, each in a buffer of its own in arbitrary entry order — then one combine gives
    the whole-layer call's output bit for bit."""
    from expert_cache_offloaded_amd import _lib as L
    from oracle import route
    cfg = synth.CONFIGS["prefill"].with_(L=1, E=16, k=4, H=512, I=256, T=300)
    host_np = synth.host_pool(cfg)
    x = t_of(synth.activations(cfg, 0)).cuda()
    lg = synth.uniform_logits(cfg, layer=0)
    rid, rw = route(lg, cfg.k)
    ids = torch.from_numpy(rid).cuda()
    w = torch.from_numpy(rw.astype(np.float32)).cuda()
    ws = torch.empty(L.prefill_ws_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    whole = L.make_banks(cfg.fmt, cfg.H, cfg.I, device_banks(host_np))
    y0 = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    L.moe_experts_prefill(x, ids, w, None, cfg.E, whole, ws, y0)
    counts = torch.full((cfg.E,), -7, dtype=torch.int32, device="cuda")
    L.moe_experts_prefill_part(x, ids, w, None, cfg.E, whole, None, L.PF_SORT, ws, counts=counts)
    want_counts = np.bincount(rid.ravel(), minlength=cfg.E)
    assert np.array_equal(counts.cpu().numpy(), want_counts)
    rng = np.random.default_rng(5)
    order = rng.permutation(cfg.E)
    parts = [order[:5], order[5:6], order[6:]]
    keep = []
    for p in parts:
        perm = rng.permutation(len(p))           # entry j of the part buffer holds expert p[perm[j]]
        ex = p[perm]
        buf_np = {k: np.ascontiguousarray(v[ex]) for k, v in host_np.items()}
        t = device_banks(buf_np)
        keep.append(t)
        eo = np.full(cfg.E, -1, dtype=np.int32)
        eo[ex] = np.arange(len(ex), dtype=np.int32)
        eo_t = torch.from_numpy(eo).cuda()
        keep.append(eo_t)
        L.moe_experts_prefill_part(x, ids, w, None, cfg.E, L.make_banks(cfg.fmt, cfg.H, cfg.I, t), eo_t,
                                   L.PF_EXPERTS, ws)
    y1 = torch.empty_like(y0)
    L.moe_experts_prefill_part(x, ids, w, None, cfg.E, whole, None, L.PF_COMBINE, ws, y=y1)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_prefill_part_rejects_bad_steps():
    from expert_cache_offloaded_amd import _lib as L
    cfg = synth.CONFIGS["prefill"].with_(L=1, E=16, k=4, H=512, I=256, T=8)
    host_np = synth.host_pool(cfg)
    whole = L.make_banks(cfg.fmt, cfg.H, cfg.I, device_banks(host_np))
    ids = torch.zeros((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.zeros((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    x = torch.zeros((cfg.T, cfg.H), dtype=torch.int16, device="cuda")
    ws = torch.empty(L.prefill_ws_bytes(cfg.T, cfg.k, cfg.E, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    with pytest.raises(L.McError):
        L.moe_experts_prefill_part(x, ids, w, None, cfg.E, whole, None, 0, ws)
    with pytest.raises(L.McError):
        L.moe_experts_prefill_part(x, ids, w, None, cfg.E, whole, None, 8, ws)
    with pytest.raises(L.McError):             # experts without entry_of
        L.moe_experts_prefill_part(x, ids, w, None, cfg.E, whole, None, L.PF_EXPERTS, ws)
