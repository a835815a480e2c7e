"""Pins for the oracle's routing, expert FFN, combine and prefill grouping (CPU only)."""
import math

import numpy as np
import pytest

import synth
from oracle import (bf16_to_f64, decode_layer, expert_ffn, expert_ffn_loops, expert_matrices, hybrid_partials,
                    prefill_grouped, prefill_per_token, route, sort_routes)


def _small_cfg(fmt="mxfp4", **kw):
    base = dict(name="t", L=2, E=8, k=3, H=64, I=64, fmt=fmt, T=5, steps=4, S=6, seed=11)
    base.update(kw)
    return synth.Config(**base)


def test_ffn_matmul_equals_loops():
    cfg = _small_cfg(H=32, I=64)
    banks = synth.host_pool(cfg, flats=[3])
    wg, wu, wd = expert_matrices(banks, 0, cfg.fmt, cfg.H, cfg.I)
    x = np.random.default_rng(1).standard_normal((2, cfg.H))
    y = expert_ffn(wg, wu, wd, x)
    for t in range(2):
        y_loop = expert_ffn_loops(wg, wu, wd, x[t])
        assert np.max(np.abs(y[t] - y_loop)) <= 1e-12 * max(1.0, np.max(np.abs(y_loop)))


def test_ffn_zero_gate_and_hand_value():
    wg = np.zeros((4, 3)); wu = np.ones((4, 3)); wd = np.ones((3, 4))
    assert np.all(expert_ffn(wg, wu, wd, np.ones((1, 3))) == 0.0)
    # H = I = 1: y = wd * silu(wg x) * (wu x) with wg=1, wu=2, wd=3, x=0.5
    y = expert_ffn(np.array([[1.0]]), np.array([[2.0]]), np.array([[3.0]]), np.array([[0.5]]))
    silu = 0.5 / (1.0 + math.exp(-0.5))
    assert abs(y[0, 0] - 3.0 * silu * 1.0) < 1e-15


def test_route_brute_force_and_ties():
    r = np.random.default_rng(2)
    lg = r.standard_normal((50, 16)).astype(np.float32)
    lg[::7, 3] = lg[::7, 9]            # exact ties between ids 3 and 9
    lg[1] = 0.5                          # a fully tied row
    for k in (1, 2, 5, 16):
        ids, _ = route(lg, k)
        for t in range(lg.shape[0]):
            # rank of e = number of experts that beat it (higher logit, or equal logit and lower id)
            ranks = []
            for e in range(16):
                beat = sum(1 for o in range(16)
                           if lg[t, o] > lg[t, e] or (lg[t, o] == lg[t, e] and o < e))
                ranks.append(beat)
            want = [e for r_ in range(k) for e in range(16) if ranks[e] == r_]
            assert list(ids[t]) == want
    ids, _ = route(lg[1:2], 4)
    assert list(ids[0]) == [0, 1, 2, 3]


def test_route_gates_hand_values():
    lg = np.array([[0.0, math.log(3.0), -50.0]], dtype=np.float32)
    ids, w = route(lg, 2, renorm=1)
    assert list(ids[0]) == [1, 0]
    l3 = float(np.float32(math.log(3.0)))
    assert abs(w[0, 0] - math.exp(l3) / (math.exp(l3) + 1.0)) < 1e-15
    assert abs(w[0, 0] - 0.75) < 1e-7 and abs(w[0, 1] - 0.25) < 1e-7
    ids, w = route(lg, 2, renorm=0)
    tot = math.exp(l3) + 1.0 + math.exp(-50.0)
    assert abs(w[0, 0] - math.exp(l3) / tot) < 1e-15
    assert abs(w[0, 1] - 1.0 / tot) < 1e-15


def test_trace_logits_reproduce_trace_sets():
    for name in ("tiny", "zipf_decode"):
        cfg = synth.CONFIGS[name].with_(L=2, steps=6, T=3)
        tr = synth.trace(cfg)
        for s in range(cfg.steps):
            lg = synth.step_logits(cfg, tr[s], s)
            for l in range(cfg.L):
                ids, _ = route(lg[l], cfg.k)
                for t in range(cfg.T):
                    assert set(ids[t]) == set(tr[s, l, t])
                    assert len(set(tr[s, l, t])) == cfg.k


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_hybrid_partials_sum_to_unsplit(fmt):
    cfg = _small_cfg(fmt)
    banks = synth.host_pool(cfg)
    shared = synth.shared_pool(cfg)
    r = np.random.default_rng(5)
    x = synth.activations(cfg, 0)
    ids = np.stack([r.choice(cfg.E, cfg.k, replace=False) for _ in range(cfg.T)]).astype(np.int32)
    ids[2, 1] = -1
    w = r.random((cfg.T, cfg.k))
    slots = np.where(r.random((cfg.T, cfg.k)) < 0.5, 0, -1).astype(np.int32)
    layer = 1
    y_gpu, y_host, gpu_w, host_ids = hybrid_partials(x, ids, slots, w, banks, layer, cfg.E, fmt, cfg.H, cfg.I)
    y = decode_layer(x, ids, w, banks, layer, cfg.E, fmt, cfg.H, cfg.I)
    assert np.max(np.abs(y_gpu + y_host - y)) <= 1e-12 * np.linalg.norm(y)
    # complementary masks: each valid route is on exactly one side
    for t in range(cfg.T):
        for j in range(cfg.k):
            if ids[t, j] < 0:
                assert gpu_w[t, j] == 0 and host_ids[t, j] == -1
            else:
                assert (slots[t, j] >= 0) == (gpu_w[t, j] == w[t, j]) == (host_ids[t, j] == -1)
    # shared expert adds one weight-1 FFN
    y_sh = decode_layer(x, ids, w, banks, layer, cfg.E, fmt, cfg.H, cfg.I, shared=shared)
    wg, wu, wd = expert_matrices(shared, layer, fmt, cfg.H, cfg.I)
    assert np.allclose(y_sh - y, expert_ffn(wg, wu, wd, bf16_to_f64(x)), rtol=0, atol=1e-12)


def test_sort_routes_brute_force():
    r = np.random.default_rng(7)
    ids = r.integers(0, 9, size=(40, 3)).astype(np.int32)
    ids[5, 0] = -1
    counts, offsets, perm = sort_routes(ids, 9)
    want = []
    for e in range(9):
        for t in range(40):
            for j in range(3):
                if ids[t, j] == e:
                    want.append(t * 3 + j)
    assert list(perm) == want
    assert list(counts) == [int(np.sum(ids == e)) for e in range(9)]
    assert offsets[0] == 0 and offsets[-1] == len(want)
    counts, offsets, perm = sort_routes(ids, 9, n_tok=10)
    assert offsets[-1] == int(np.sum((ids[:10] >= 0)))


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_prefill_grouped_equals_per_token(fmt):
    cfg = _small_cfg(fmt, T=40, E=6, k=2)
    banks = synth.host_pool(cfg, flats=range(cfg.E))
    x = synth.activations(cfg, 0)
    lg = synth.uniform_logits(cfg)
    ids, w = route(lg, cfg.k)
    y_g = prefill_grouped(x, ids, w, banks, cfg.E, fmt, cfg.H, cfg.I)
    y_t = prefill_per_token(x, ids, w, banks, cfg.E, fmt, cfg.H, cfg.I)
    assert np.max(np.abs(y_g - y_t)) <= 1e-12 * np.max(np.abs(y_t))


def _per_route_sum(x_bits, ids, w, banks, layer, E, fmt, H, I, n_tok=None, keep=None):
    """y_t = sum_j w_tj Expert_{layer*E + ids_tj}(x_t), one route at a time, each expert
    evaluated by the explicit-loop FFN ([jjl357] "1.1": the gate-weighted sum of the
    selected experts' outputs)."""
    x = bf16_to_f64(x_bits)
    T, k = ids.shape
    n_tok = T if n_tok is None else n_tok
    y = np.zeros((T, H))
    for t in range(n_tok):
        for j in range(k):
            e = int(ids[t, j])
            if e < 0 or (keep is not None and not keep[t, j]):
                continue
            wg, wu, wd = expert_matrices(banks, layer * E + e, fmt, H, I)
            y[t] += float(w[t, j]) * expert_ffn_loops(wg, wu, wd, x[t])
    return y


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
@pytest.mark.parametrize("n_tok", [None, 3])
@pytest.mark.parametrize("with_shared", [False, True])
def test_decode_layer_equals_per_route_definition(fmt, n_tok, with_shared):
    cfg = _small_cfg(fmt, H=32, I=32, E=6, k=3, T=5)
    banks = synth.host_pool(cfg)
    shared = synth.shared_pool(cfg) if with_shared else None
    r = np.random.default_rng(17)
    x = synth.activations(cfg, 1)
    # several tokens share experts, so a per-expert grouping has to scatter to the right rows
    ids = np.stack([r.choice(cfg.E, cfg.k, replace=False) for _ in range(cfg.T)]).astype(np.int32)
    ids[1] = ids[0][::-1]
    ids[3, 2] = -1
    w = r.random((cfg.T, cfg.k)) + 0.1
    for layer in (0, 1):
        want = _per_route_sum(x, ids, w, banks, layer, cfg.E, fmt, cfg.H, cfg.I, n_tok=n_tok)
        if with_shared:
            wg, wu, wd = expert_matrices(shared, layer, fmt, cfg.H, cfg.I)
            xs = bf16_to_f64(x)
            for t in range(cfg.T if n_tok is None else n_tok):
                want[t] += expert_ffn_loops(wg, wu, wd, xs[t])
        got = decode_layer(x, ids, w, banks, layer, cfg.E, fmt, cfg.H, cfg.I, shared=shared, n_tok=n_tok)
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))
        if n_tok is not None:
            assert np.all(got[n_tok:] == 0.0)
        # the split: the GPU partial is the per-route sum over resident routes, the host
        # partial the sum over the others
        slots = np.where(r.random((cfg.T, cfg.k)) < 0.5, 2, -1).astype(np.int32)
        y_gpu, y_host, _, _ = hybrid_partials(x, ids, slots, w, banks, layer, cfg.E, fmt, cfg.H, cfg.I,
                                              n_tok=n_tok)
        want_gpu = _per_route_sum(x, ids, w, banks, layer, cfg.E, fmt, cfg.H, cfg.I, n_tok, keep=slots >= 0)
        want_host = _per_route_sum(x, ids, w, banks, layer, cfg.E, fmt, cfg.H, cfg.I, n_tok, keep=slots < 0)
        tol = 1e-12 * max(1.0, np.max(np.abs(want)))
        assert np.max(np.abs(y_gpu - want_gpu)) <= tol
        assert np.max(np.abs(y_host - want_host)) <= tol


def _bf16_bits(vals):
    """bf16 bit patterns of values that bf16 holds exactly."""
    a = np.asarray(vals, dtype=np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_to_f64(bits), a.astype(np.float64))
    return bits


def test_decode_layer_hand_built_two_layers():
    """Two layers of two experts, H = 2, I = 1, every weight a small exact binary
    fraction and different per (layer, expert): the output is evaluated by hand from
    y_t = sum_j w_tj * wd * silu(wg . x_t) * (wu . x_t)."""
    L_, E, H, I = 2, 2, 2, 1
    # (wg0, wg1, wu0, wu1, wd0, wd1) per flat id l*E + e
    params = {0: (0.5, -1.0, 1.0, 0.25, 2.0, -0.5),
              1: (1.0, 0.5, -0.5, 1.0, 1.0, 3.0),
              2: (-0.25, 2.0, 0.75, -1.0, -1.0, 0.5),
              3: (1.5, 1.0, 0.5, 0.5, 0.25, -2.0)}
    gu = np.zeros((L_ * E, 2 * I, H), dtype=np.uint16)
    dn = np.zeros((L_ * E, H, I), dtype=np.uint16)
    for f, (g0, g1, u0, u1, d0, d1) in params.items():
        gu[f] = _bf16_bits([[g0, g1], [u0, u1]])
        dn[f] = _bf16_bits([[d0], [d1]])
    banks = {"gate_up": gu, "down": dn}
    x_vals = [[1.0, 2.0], [-0.5, 0.25]]
    x = _bf16_bits(x_vals)
    ids = np.array([[1, 0], [0, -1]], dtype=np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.125]])

    def by_hand(layer):
        y = np.zeros((2, H))
        for t in range(2):
            for j in range(2):
                e = int(ids[t, j])
                if e < 0:
                    continue
                g0, g1, u0, u1, d0, d1 = params[layer * E + e]
                xa, xb = x_vals[t]
                g = g0 * xa + g1 * xb
                u = u0 * xa + u1 * xb
                h = g / (1.0 + math.exp(-g)) * u
                y[t, 0] += w[t, j] * d0 * h
                y[t, 1] += w[t, j] * d1 * h
        return y

    for layer in range(L_):
        got = decode_layer(x, ids, w, banks, layer, E, "bf16", H, I)
        assert np.max(np.abs(got - by_hand(layer))) <= 1e-14
    assert np.max(np.abs(by_hand(0) - by_hand(1))) > 0.1       # the layers really differ
