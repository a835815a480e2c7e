"""Routing, expert FFN and the gated combine (oracle side; test infrastructure only).

Pages:
  [jjl357] "1.1 Dense LLM 与 MoE LLM 的区别": the router picks the top-k experts of
           a token and the layer output is the gate-weighted sum of their outputs.
  [jjl357] "6.2 每个 miss 有两条精确执行路径" and "6.9": the GPU and CPU partials
           use the router's own ids and gates and are added; nothing is dropped.
  [wanger] "代码全链路 / 2. 每步 decode": GPU routes get gate 0 on the host side's
           complement and host routes are marked -1 on the GPU side; the partial
           outputs are summed.
  [juhe]   "为什么可以直接相加": y = y_gpu + y_cpu; shared experts always run and
           stay GPU-resident.
The expert FFN form (SwiGLU, no biases) is not spelled out by the pages; the
reading used is y = W_down (silu(W_gate x) * (W_up x)), silu(z) = z / (1 + e^-z).

Parity pins (tests/test_oracle_moe.py): the matmul FFN against an explicit
triple-loop FFN, W_gate = 0 => y = 0, a one-hot FFN against hand-evaluated
silu, routing against a brute-force full sort and hand-computed softmaxes,
trace logits reproducing their id sets, the hybrid split summing to the
unsplit layer, and the grouped prefill against the per-token definition.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .formats import bf16_to_f64, expert_matrices


def _silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):          # exp(-z) -> inf for z << 0 gives the limit -0
        return z / (1.0 + np.exp(-z))


def expert_ffn(wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, x: np.ndarray) -> np.ndarray:
    """SwiGLU expert on rows of x: [n, H] -> [n, H] (float64)."""
    g = x @ wg.T
    u = x @ wu.T
    h = _silu(g) * u
    return h @ wd.T


def expert_ffn_loops(wg, wu, wd, x_row):
    """The same expert for one token, written as explicit loops (pin for ``expert_ffn``)."""
    I, H = wg.shape
    h = [0.0] * I
    for i in range(I):
        g = 0.0
        u = 0.0
        for c in range(H):
            g += float(wg[i, c]) * float(x_row[c])
            u += float(wu[i, c]) * float(x_row[c])
        h[i] = (g / (1.0 + np.exp(-g))) * u
    y = [0.0] * H
    for r in range(H):
        acc = 0.0
        for i in range(I):
            acc += float(wd[r, i]) * h[i]
        y[r] = acc
    return np.array(y)


def route(logits: np.ndarray, k: int, renorm: int = 1):
    """Top-k routing [jjl357] "1.1": ids [T, k] int32 and gates [T, k] float64.

    Order: logit descending, ties to the lower expert id; comparisons on the raw
    fp32 logits.  renorm=1: softmax over the k selected logits; renorm=0: the
    selected experts' probabilities under the softmax over all E logits.
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t]))   # last key is primary
        sel = order[:k]
        ids[t] = sel
        l64 = lg[t].astype(np.float64)
        if renorm:
            z = np.exp(l64[sel] - l64[sel].max())
            w[t] = z / z.sum()
        else:
            z = np.exp(l64 - l64.max())
            w[t] = z[sel] / z.sum()
    return ids, w


def _x64(x_bits: np.ndarray) -> np.ndarray:
    return bf16_to_f64(x_bits)


def _accumulate(y, x, routes_by_flat, banks, fmt, H, I, index_of):
    for flat, lst in routes_by_flat.items():
        wg, wu, wd = expert_matrices(banks, index_of(flat), fmt, H, I)
        toks = np.array([t for t, _ in lst])
        gates = np.array([g for _, g in lst])
        out = expert_ffn(wg, wu, wd, x[toks])
        np.add.at(y, toks, gates[:, None] * out)


def decode_layer(x_bits, ids, w, banks, layer: int, E: int, fmt: str, H: int, I: int,
                 shared: Optional[dict] = None, n_tok: Optional[int] = None,
                 index_of=None) -> np.ndarray:
    """Unsplit MoE layer output y [T, H] (float64) from host truth.

    y_t = sum_j w_tj Expert_{layer, ids_tj}(x_t)  (+ Expert_shared(x_t) with weight 1).
    Experts are read by flat id layer*E + e from the host banks (``index_of`` maps a
    flat id to a bank entry; identity by default).  Routes with id -1 and tokens at
    or beyond ``n_tok`` contribute nothing.
    """
    index_of = index_of or (lambda f: f)
    x = _x64(x_bits)
    T = x.shape[0]
    n_tok = T if n_tok is None else n_tok
    y = np.zeros((T, H))
    by_flat = {}
    for t in range(n_tok):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if e < 0:
                continue
            by_flat.setdefault(layer * E + e, []).append((t, float(w[t, j])))
    _accumulate(y, x, by_flat, banks, fmt, H, I, index_of)
    if shared is not None:
        wg, wu, wd = expert_matrices(shared, layer, fmt, H, I)
        y[:n_tok] += expert_ffn(wg, wu, wd, x[:n_tok])
    return y


def hybrid_partials(x_bits, ids_raw, slots, w, banks, layer: int, E: int, fmt: str, H: int, I: int,
                    n_tok: Optional[int] = None, index_of=None):
    """Split of one decode layer into its two partial outputs ([wanger] "代码全链路").

    A route (t, j) goes to the GPU partial when its slot is >= 0 and to the host
    partial when its slot is -1 and its raw id is valid.  Both partials read the
    expert from host truth by flat id.  Returns (y_gpu, y_host, gpu_w, host_ids)
    where gpu_w is w with host routes zeroed and host_ids is the raw id with GPU
    routes set to -1 — the two complementary masks.
    """
    index_of = index_of or (lambda f: f)
    x = _x64(x_bits)
    T, k = ids_raw.shape
    n_tok = T if n_tok is None else n_tok
    y_gpu = np.zeros((T, H))
    y_host = np.zeros((T, H))
    gpu_w = np.zeros((T, k))
    host_ids = np.full((T, k), -1, dtype=np.int32)
    on_gpu, on_host = {}, {}
    for t in range(n_tok):
        for j in range(k):
            e = int(ids_raw[t, j])
            if e < 0:
                continue
            flat = layer * E + e
            if slots[t, j] >= 0:
                gpu_w[t, j] = w[t, j]
                on_gpu.setdefault(flat, []).append((t, float(w[t, j])))
            else:
                host_ids[t, j] = e
                on_host.setdefault(flat, []).append((t, float(w[t, j])))
    _accumulate(y_gpu, x, on_gpu, banks, fmt, H, I, index_of)
    _accumulate(y_host, x, on_host, banks, fmt, H, I, index_of)
    return y_gpu, y_host, gpu_w, host_ids


def sort_routes(ids: np.ndarray, E: int, n_tok: Optional[int] = None):
    """Stable grouping of the routes of a prefill chunk by expert.

    Route r = t*k + j.  Returns counts [E], offsets [E+1] (exclusive prefix sum) and
    perm [n_valid]: the route indices of expert 0 in (t, j) order, then expert 1, ...
    Routes with id outside [0, E) and tokens at or beyond n_tok are left out.
    """
    T, k = ids.shape
    n_tok = T if n_tok is None else n_tok
    flat_ids = ids[:n_tok].reshape(-1).astype(np.int64)
    r = np.arange(flat_ids.size)
    ok = (flat_ids >= 0) & (flat_ids < E)
    counts = np.bincount(flat_ids[ok], minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat_ids[ok], kind="stable")
    perm = r[ok][order].astype(np.int32)
    return counts, offsets, perm


def prefill_per_token(x_bits, ids, w, banks, E: int, fmt: str, H: int, I: int,
                      tokens=None, index_of=None) -> np.ndarray:
    """Prefill layer output by the per-token definition, optionally for a token subset.

    ``banks`` holds the layer's E experts (entry e = expert e).  Returns [len(tokens), H].
    """
    index_of = index_of or (lambda e: e)
    x = _x64(x_bits)
    tokens = range(x.shape[0]) if tokens is None else tokens
    tokens = list(tokens)
    out = np.zeros((len(tokens), H))
    for n, t in enumerate(tokens):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if e < 0:
                continue
            wg, wu, wd = expert_matrices(banks, index_of(e), fmt, H, I)
            out[n] += float(w[t, j]) * expert_ffn(wg, wu, wd, x[t:t + 1])[0]
    return out


def prefill_grouped(x_bits, ids, w, banks, E: int, fmt: str, H: int, I: int,
                    experts=None, index_of=None) -> np.ndarray:
    """Prefill layer output computed per expert: gather its tokens, run the expert on
    the group, scatter-add the gated outputs ([jjl357] "6.8": grouped execution).

    ``experts`` restricts the sum to a subset of experts (for bounded samples).
    """
    index_of = index_of or (lambda e: e)
    x = _x64(x_bits)
    T = x.shape[0]
    y = np.zeros((T, H))
    counts, offsets, perm = sort_routes(ids, E)
    k = ids.shape[1]
    experts = range(E) if experts is None else experts
    for e in experts:
        rs = perm[offsets[e]:offsets[e + 1]]
        if rs.size == 0:
            continue
        toks = rs // k
        gates = w.reshape(-1)[rs].astype(np.float64)
        wg, wu, wd = expert_matrices(banks, index_of(e), fmt, H, I)
        out = expert_ffn(wg, wu, wd, x[toks])
        np.add.at(y, toks, gates[:, None] * out)
    return y
