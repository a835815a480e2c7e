"""Seeded synthetic inputs shared by the tests, the oracle and the benchmark.

This module only *makes inputs*: expert weight codes, activations, routing
traces and router logits.  It holds none of the MoE layer's arithmetic — no
MXFP4 decode, no routing, no cache logic, no expert FFN.  Both the CPU oracle
(``oracle/``) and the HIP path consume what it returns; neither side's code is
imported here.

Workload shapes follow the FreeToken pages:
  * Qwen3.6-35B-A3B-shaped decode: 40 MoE layers, 256 routed experts, top-8,
    one shared expert, hidden 2048, expert intermediate 512 (jjl357 blog,
    "9.2 模型"; juhe.plus article, slot-pool example "40 层 × 每层 256 个专家").
  * DeepSeek-V4-Flash-shaped decode: 43 MoE layers, 256 experts, top-6,
    native MXFP4 experts (jjl357 blog, "1.2 一个具体例子").
  * Prefill: 8192-token chunks (jjl357 blog, "4.2 双缓冲时间线").
  * Routing locality p = probability that a token keeps the previous token's
    expert (Qiita article, "5. デコード側の答え その1").
Weight values, activations and the exact trace recipe are not given by the
pages; the recipe used here is stated next to each generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    name: str
    L: int                 # MoE layers
    E: int                 # routed experts per layer
    k: int                 # top-k
    H: int                 # hidden size
    I: int                 # expert intermediate size
    fmt: str               # "bf16" | "mxfp4"
    T: int                 # tokens per decode step (batch size) / prefill tokens
    steps: int             # decode steps in the trace
    S: int                 # slots in the cross-layer cache
    seed: int
    routing: str = "locality"   # "locality" | "zipf" | "uniform"
    p: float = 0.8              # routing locality
    zipf_s: float = 1.1
    shared: bool = False        # one always-on shared expert per layer
    renorm: int = 1             # gates: softmax over the k selected logits

    @property
    def n_flat(self) -> int:
        return self.L * self.E

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS: Dict[str, Config] = {
    # tiny correctness layer: 1 layer, E=8, top-2, H=64, I=128, bf16, 4 tokens x 64 steps, 4 slots
    "tiny": Config("tiny", L=1, E=8, k=2, H=64, I=128, fmt="bf16", T=4, steps=64, S=4,
                   seed=0, routing="locality", p=0.7),
    # Qwen3.6-35B-A3B-shaped decode
    "qwen_decode": Config("qwen_decode", L=40, E=256, k=8, H=2048, I=512, fmt="mxfp4", T=1,
                          steps=2048, S=600, seed=2, routing="locality", p=0.8, shared=True),
    # DeepSeek-V4-Flash-shaped hybrid decode (p in {0.5, 0.9} is set per run)
    "dsv4_hybrid": Config("dsv4_hybrid", L=43, E=256, k=6, H=4096, I=2048, fmt="mxfp4", T=1,
                          steps=1024, S=1500, seed=3, routing="locality", p=0.5),
    # prefill: one layer shape, 8192 tokens, uniform routing
    "prefill": Config("prefill", L=4, E=256, k=6, H=4096, I=2048, fmt="mxfp4", T=8192,
                      steps=1, S=512, seed=4, routing="uniform"),
    # batched decode with Zipf skew (T in {1,4,16}, S swept 256..4096 per run)
    "zipf_decode": Config("zipf_decode", L=40, E=256, k=8, H=2048, I=512, fmt="mxfp4", T=1,
                          steps=1024, S=1024, seed=5, routing="zipf", zipf_s=1.1),
}


def expert_bytes(H: int, I: int, fmt: str) -> int:
    """Bytes of one complete expert (all banks)."""
    if fmt == "bf16":
        return 3 * H * I * 2
    return 3 * H * I // 2 + 3 * H * I // 32


def bank_shapes(H: int, I: int, fmt: str) -> Dict[str, Tuple[Tuple[int, ...], np.dtype]]:
    """Per-expert bank shapes of the expert layout (flat id / slot is the leading dim).

    gate_up rows [0, I) are the gate projection, rows [I, 2I) the up projection;
    the contraction axis is the last one.  MXFP4: byte j of a row packs element 2j
    in its low nibble and element 2j+1 in its high nibble; one e8m0 scale byte per
    32 consecutive elements of a row.
    """
    if fmt == "bf16":
        return {"gate_up": ((2 * I, H), np.dtype(np.uint16)),
                "down": ((H, I), np.dtype(np.uint16))}
    return {"gate_up": ((2 * I, H // 2), np.dtype(np.uint8)),
            "gate_up_scale": ((2 * I, H // 32), np.dtype(np.uint8)),
            "down": ((H, I // 2), np.dtype(np.uint8)),
            "down_scale": ((H, I // 32), np.dtype(np.uint8))}


# ----------------------------------------------------------------------------
# bf16 bit patterns (generation side: rounding fp32 samples into bf16 inputs)
# ----------------------------------------------------------------------------


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 samples to bf16 (round-to-nearest-even) and return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


# ----------------------------------------------------------------------------
# expert weights
# ----------------------------------------------------------------------------

# MXFP4 code sampling.  The pages do not give weight statistics; the codes are
# drawn from a fixed distribution so the decoded weights have std ~0.02 (the
# same spread as the bf16 layers' N(0, 0.02)).  Magnitude code counts (out of 16)
# for e2m1 codes 0..7; sign bits are fair coins.
_MAG_COUNTS = np.array([1, 3, 2, 2, 3, 2, 2, 1])
# shared-exponent draws: X - 127 in {-8, -7, -6} with counts (out of 256)
_EXP_COUNTS = {-8: 48, -7: 160, -6: 48}


def _mag_pair_table() -> np.ndarray:
    mags = np.repeat(np.arange(8, dtype=np.uint8), _MAG_COUNTS)          # 16 entries
    lo = np.tile(mags, 16)
    hi = np.repeat(mags, 16)
    return (lo | (hi << 4)).astype(np.uint8)                              # 256 entries


def _exp_table() -> np.ndarray:
    vals = []
    for e, c in _EXP_COUNTS.items():
        vals += [127 + e] * c
    return np.array(vals, dtype=np.uint8)


_MAG_TABLE = _mag_pair_table()
_EXP_TABLE = _exp_table()
assert _MAG_TABLE.size == 256 and _EXP_TABLE.size == 256


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(x) for x in key]))


def _mxfp4_codes(rng: np.random.Generator, rows: int, cols: int) -> Tuple[np.ndarray, np.ndarray]:
    n = rows * cols // 2
    mag = _MAG_TABLE[rng.integers(0, 256, size=n, dtype=np.uint8)]
    sign = rng.integers(0, 256, size=n, dtype=np.uint8) & np.uint8(0x88)
    codes = (mag | sign).reshape(rows, cols // 2)
    scales = _EXP_TABLE[rng.integers(0, 256, size=rows * cols // 32, dtype=np.uint8)]
    return codes, scales.reshape(rows, cols // 32)


def _bf16_matrix(rng: np.random.Generator, rows: int, cols: int, std: float = 0.02) -> np.ndarray:
    return to_bf16_bits(rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std))


# weight key tags: routed experts use tag 1, shared experts tag 2
_TAG_ROUTED, _TAG_SHARED, _TAG_X, _TAG_TRACE, _TAG_LOGIT = 1, 2, 3, 4, 5


def expert_weights(cfg: Config, flat: int, tag: int = _TAG_ROUTED) -> Dict[str, np.ndarray]:
    """All banks of one routed expert, flat id = layer * E + expert.

    Seeded from (config seed, tag, flat id, bank), so any expert can be made on its
    own and any subset of the pool reproduced exactly.
    """
    H, I = cfg.H, cfg.I
    if cfg.fmt == "bf16":
        return {"gate_up": _bf16_matrix(_rng(cfg.seed, tag, flat, 0), 2 * I, H),
                "down": _bf16_matrix(_rng(cfg.seed, tag, flat, 1), H, I)}
    gu, gus = _mxfp4_codes(_rng(cfg.seed, tag, flat, 0), 2 * I, H)
    dn, dns = _mxfp4_codes(_rng(cfg.seed, tag, flat, 1), H, I)
    return {"gate_up": gu, "gate_up_scale": gus, "down": dn, "down_scale": dns}


def exponent_variant(cfg: Config, flat: int, gu_bases: Sequence[int], dn_bases: Sequence[int],
                     spread: int = 2, tag: int = _TAG_ROUTED) -> Dict[str, np.ndarray]:
    """An MXFP4 expert whose block exponents sit at chosen places of the e8m0 range
    (inputs for tests of the format's edges, not a workload).  The codes are those of
    ``expert_weights``; row r of the gate_up bank takes the base exponent
    gu_bases[r % len(gu_bases)], row r of the down bank dn_bases[r % len(dn_bases)], and
    each 32-element block of a row gets X - 127 = base - d with d uniform in [0, spread]
    (seeded), X clamped to [0, 254]."""
    if cfg.fmt != "mxfp4":
        raise ValueError("exponent_variant needs MXFP4 experts")
    w = expert_weights(cfg, flat, tag)
    r = _rng(cfg.seed, tag, flat, 7)
    for name, bases in (("gate_up_scale", gu_bases), ("down_scale", dn_bases)):
        rows, blocks = w[name].shape
        base = np.array([bases[i % len(bases)] for i in range(rows)], dtype=np.int64)[:, None]
        x = 127 + base - r.integers(0, spread + 1, size=(rows, blocks))
        w[name] = np.clip(x, 0, 254).astype(np.uint8)
    return w


def shared_weights(cfg: Config, layer: int) -> Dict[str, np.ndarray]:
    """The always-on shared expert of one layer (same format and shape as a routed one)."""
    return expert_weights(cfg, layer, tag=_TAG_SHARED)


def alloc_banks(cfg: Config, n: int, empty=np.empty) -> Dict[str, np.ndarray]:
    """Allocate n experts' worth of banks (``empty`` may allocate pinned memory)."""
    return {name: empty((n,) + shp, dtype=dt) for name, (shp, dt) in bank_shapes(cfg.H, cfg.I, cfg.fmt).items()}


def fill_banks(cfg: Config, banks: Dict[str, np.ndarray], flats: Iterable[int], first: int = 0,
               tag: int = _TAG_ROUTED) -> None:
    """Write experts ``flats`` into consecutive entries of ``banks`` starting at ``first``."""
    for i, f in enumerate(flats):
        w = expert_weights(cfg, int(f), tag)
        for name, arr in w.items():
            banks[name][first + i] = arr


def host_pool(cfg: Config, flats: Optional[Sequence[int]] = None, empty=np.empty) -> Dict[str, np.ndarray]:
    """The host-side expert pool indexed by flat id (all L*E experts unless ``flats``)."""
    flats = range(cfg.n_flat) if flats is None else flats
    flats = list(flats)
    b = alloc_banks(cfg, len(flats), empty)
    fill_banks(cfg, b, flats)
    return b


def shared_pool(cfg: Config, empty=np.empty) -> Dict[str, np.ndarray]:
    b = alloc_banks(cfg, cfg.L, empty)
    fill_banks(cfg, b, range(cfg.L), tag=_TAG_SHARED)
    return b


# ----------------------------------------------------------------------------
# activations
# ----------------------------------------------------------------------------


def activations(cfg: Config, step: int, layer: int = 0, T: Optional[int] = None) -> np.ndarray:
    """x ~ N(0, 1) rounded to bf16; returned as uint16 bits [T, H]."""
    T = cfg.T if T is None else T
    r = _rng(cfg.seed, _TAG_X, step, layer)
    return to_bf16_bits(r.standard_normal((T, cfg.H), dtype=np.float32))


# ----------------------------------------------------------------------------
# routing traces
# ----------------------------------------------------------------------------


def locality_stream(E: int, k: int, steps: int, p: float, rng: np.random.Generator) -> np.ndarray:
    """One token stream of k distinct expert ids per step with locality p.

    Each step keeps each of the k positions with probability p; a replaced position
    takes an id uniform over the experts not currently in the set, so the set stays
    distinct (a reading of the Qiita article's locality parameter, which lets a
    replacement collide).
    """
    cur = rng.choice(E, size=k, replace=False).astype(np.int64)
    out = np.empty((steps, k), dtype=np.int32)
    for s in range(steps):
        if s > 0:
            u = rng.random(k)
            for j in range(k):
                if u[j] > p:
                    free = np.setdiff1d(np.arange(E), cur, assume_unique=False)
                    cur[j] = free[rng.integers(0, free.size)]
        out[s] = cur
    return out


def zipf_stream(E: int, k: int, steps: int, s_exp: float, perm: np.ndarray,
                rng: np.random.Generator) -> np.ndarray:
    """k distinct ids per step drawn without replacement from P(rank r) ~ r^-s."""
    w = np.arange(1, E + 1, dtype=np.float64) ** (-s_exp)
    pr = w / w.sum()
    out = np.empty((steps, k), dtype=np.int32)
    for s in range(steps):
        ranks = rng.choice(E, size=k, replace=False, p=pr)
        out[s] = perm[ranks]
    return out


def trace(cfg: Config, steps: Optional[int] = None, T: Optional[int] = None) -> np.ndarray:
    """Routing trace ids [steps, L, T, k] (int32, expert-in-layer ids, distinct per token)."""
    steps = cfg.steps if steps is None else steps
    T = cfg.T if T is None else T
    out = np.empty((steps, cfg.L, T, cfg.k), dtype=np.int32)
    for l in range(cfg.L):
        if cfg.routing == "zipf":
            perm = _rng(cfg.seed, _TAG_TRACE, l, 1 << 20).permutation(cfg.E).astype(np.int32)
        for t in range(T):
            r = _rng(cfg.seed, _TAG_TRACE, l, t)
            if cfg.routing == "locality":
                out[:, l, t] = locality_stream(cfg.E, cfg.k, steps, cfg.p, r)
            elif cfg.routing == "zipf":
                out[:, l, t] = zipf_stream(cfg.E, cfg.k, steps, cfg.zipf_s, perm, r)
            else:
                for s in range(steps):
                    out[s, l, t] = r.choice(cfg.E, size=cfg.k, replace=False)
    return out


def logits_for(ids: np.ndarray, E: int, rng: np.random.Generator) -> np.ndarray:
    """Router logits [..., E] (fp32) whose top-k set is exactly ``ids`` [..., k].

    Unselected experts get N(0, 1) clipped to [-4, 4]; selected ones get
    4.5 + 3*U(0, 1), so they always rank above every unselected expert.
    """
    lead = ids.shape[:-1]
    lg = np.clip(rng.standard_normal(lead + (E,)), -4.0, 4.0).astype(np.float32)
    hi = (4.5 + 3.0 * rng.random(ids.shape)).astype(np.float32)
    np.put_along_axis(lg, ids.astype(np.int64), hi, axis=-1)
    return lg


def step_logits(cfg: Config, ids_step: np.ndarray, step: int) -> np.ndarray:
    """Logits [L, T, E] for one decode step of a trace (ids_step [L, T, k])."""
    return logits_for(ids_step, cfg.E, _rng(cfg.seed, _TAG_LOGIT, step))


def uniform_logits(cfg: Config, T: Optional[int] = None, layer: int = 0) -> np.ndarray:
    """Prefill router logits: i.i.d. N(0, 1) per (token, expert), fp32 [T, E]."""
    T = cfg.T if T is None else T
    return _rng(cfg.seed, _TAG_LOGIT, 1 << 30, layer).standard_normal((T, cfg.E), dtype=np.float32)


def drifting_working_set(E: int, K: int, steps: int, locality: float, seed: int) -> np.ndarray:
    """Routing trace of the Qiita article's simulation ("5. デコード側の答え その1"),
    generated here from its description: K positions start on K distinct ids; at
    every step each position independently takes a fresh id, uniform over all E
    experts (so two positions may coincide), with probability 1 - locality, and
    keeps its id otherwise.  All random draws of the run are made up front from
    this module's seeded streams (not the article's generator sequence), so the
    article's printed miss rates are matched statistically, not digit for digit.
    Returns int32 [steps, K].
    """
    g = _rng(seed, _TAG_TRACE, E, K)
    start = g.permutation(E)[:K]
    redraw = g.random((steps, K)) >= locality          # position takes a fresh id this step
    fresh = g.integers(0, E, size=(steps, K))
    # the id a position holds at step s is the fresh id of its latest redraw at or
    # before s, or its starting id if it was never redrawn
    step_idx = np.where(redraw, np.arange(steps)[:, None], -1)
    last = np.maximum.accumulate(step_idx, axis=0)
    held = np.where(last >= 0, fresh[np.maximum(last, 0), np.arange(K)[None, :]], start[None, :])
    return held.astype(np.int32)
