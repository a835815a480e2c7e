"""Cross-layer LRU slot cache and the fetch/host split (oracle side; test infrastructure only).

Pages:
  [jjl357] "3. FreeToken Overview": one expert cache shared by all MoE layers; a slot
           holds one whole (layer, expert).
  [jjl357] "6.1 全局 LRU 专家缓存": per step, hits H, unique misses M, m = |M|; an
           expert shared by several tokens is loaded/run once; recency updates on
           every real access.
  [jjl357] "6.2": M = F (filled, then resident) disjoint-union C (host-computed; no
           change to residency).
  [jjl357] "6.4"-"6.5": T_fill = qS/B_P, T_cpu = (m-q)S/(B_H-B_P), B_R = max(B_H-B_P, 0),
           q* = m B_P / B_H;  "6.5" closing paragraph: integer q, at least one fill,
           B_H <= B_P sends every miss to the GPU.
  [jjl357] "6.7": dedup + residency, at most q LRU victims, chosen misses filled, the
           rest become host tasks, hits + fills run on the GPU.
  [jjl357] "8.2 把控制流表示成数据": the kernel dedups, checks residency, derives q,
           picks victims and rewrites ids to slot or a host flag.
  [juhe]   "生成阶段：专家缓存到底怎么工作": slot_for_id / id_of_slot = layer*E+expert /
           usage[slot] = current_step.
  [wanger] "3. ensure_experts_hybrid 内核": the Q16 split — lo = floor(m f), pick lo or
           lo+1 by the smaller max(F(1-f), (m-F)f); then phase 2 allocates that many
           slots by LRU and phase 3 rewrites ids.
  [wanger] "实测版本": f = p_ov / (p_ov + c_ov) from concurrently measured bandwidths;
           with full contention it reduces to pcie_bw / cpu_bw.  No profile -> fixed
           fetch cap of 1.
  [qiita]  "8. 四捨五入で27%損をした話": latency model, brute-force optimum over q.

Readings where the pages leave a step open (each also listed with the design notes):
  * clock: +1 per lookup call (one layer call), global across layers; every access
    in a call shares that stamp.
  * victims: slots not hit in this call (stamp < clock), ordered by (stamp, slot);
    empty slots have stamp 0 so they go first.
  * which misses are filled: the first q unique misses in ascending flat id,
    paired in order with the victims.
  * more misses than evictable slots: the overflow goes to the host set.
  * q: the Q16 rule, then at least one fill when m >= 1 (min_fill), then capped by
    the evictable slots and by the list capacity.

Parity pins (tests/test_oracle_cache.py): a second LRU written as a recency list
with linear scans, bit-identical on small traces; reuse-distance invariants; the
Qiita replay's printed miss rate; the pages' worked q values (Fig. 2, RTX 4060
Laptop, RTX 5090 Desktop and the 27.6 % rounding loss); exact-rational brute
force of the latency model; the overlap form reducing to B_P / B_H.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Optional

import numpy as np

STAT_HITS, STAT_MISSES, STAT_FILLS, STAT_HOST, STAT_EVICT, STAT_CALLS, STAT_ERR = range(7)
Q16 = 1 << 16


# ----------------------------------------------------------------------------
# split count
# ----------------------------------------------------------------------------


def split_count(m: int, frac_q16: int, fixed_cap: int = 1, min_fill: int = 1) -> int:
    """Number of unique misses to fill (q) before the evictable/capacity caps.

    frac_q16 = 0 selects the fixed cap (the no-profile default of [wanger]).  Otherwise
    f = frac_q16 / 2^16 and q is the integer neighbour of m f minimising the slower
    branch, max(F (1-f), (m-F) f), ties to the smaller F ([wanger] "3.").  With
    min_fill, at least one fill when m >= 1 ([jjl357] "6.5").
    """
    if m <= 0:
        return 0
    if frac_q16 == 0:
        q = min(m, fixed_cap)
    else:
        f = int(frac_q16)
        lo = (m * f) >> 16

        def cost(F):
            return max(F * (Q16 - f), (m - F) * f)

        q = lo if cost(lo) <= cost(lo + 1) else lo + 1
        q = min(q, m)
    if min_fill and m >= 1:
        q = max(q, 1)
    return q


def fetch_fraction(b_p: float, b_h: float, p_ov: float = 0.0, c_ov: float = 0.0) -> Fraction:
    """Fetched fraction of the misses, exact rational.

    With overlap measurements (p_ov > 0): f = p_ov / (p_ov + c_ov) ([wanger] "实测版本").
    Otherwise f = B_P / B_H ([jjl357] "6.5"), and f = 1 when B_H <= B_P (no residual
    host bandwidth, [jjl357] "6.4"/"6.5").
    """
    if p_ov > 0:
        P, C = Fraction(p_ov), Fraction(c_ov)
        return P / (P + C)
    P, B = Fraction(b_p), Fraction(b_h)
    if B <= P:
        return Fraction(1)
    return P / B


def fetch_fraction_q16(b_p: float, b_h: float, p_ov: float = 0.0, c_ov: float = 0.0) -> int:
    """Q16 form of ``fetch_fraction``: round half up, clamped to [1, 65536].

    With no usable measurement (p_ov <= 0 and B_P <= 0) it returns 0, the fixed-cap
    mode ([wanger] "1. 启动时": no profile -> a fixed fetch cap).
    """
    if p_ov <= 0 and b_p <= 0:
        return 0
    f = fetch_fraction(b_p, b_h, p_ov, c_ov)
    v = (f * Q16 + Fraction(1, 2)).__floor__()
    return int(min(max(v, 1), Q16))


def recommend_backend(cpu_gbs: float, pcie_gbs: float, threshold: float = 2.0) -> str:
    """Backend choice of the bandwidth profile ([wanger] "第一层带宽比：选后端"): the
    ratio of the host expert kernel's bandwidth to the link's decides; above the
    threshold (2.0 on that page) the CPU branch is worth having ("hybrid"), otherwise
    every miss goes over the link ("offload")."""
    ratio = Fraction(cpu_gbs) / Fraction(pcie_gbs) if pcie_gbs > 0 else None
    if ratio is None:
        return "hybrid" if cpu_gbs > 0 else "offload"
    return "hybrid" if ratio > Fraction(threshold) else "offload"


def miss_latency(q: int, m: int, b_p, b_h):
    """Exposed miss time of the Qiita latency model (S cancels): exact rational or inf.

    Fill q experts at B_P while the host computes m - q at the residual B_H - B_P;
    the two run concurrently, so the slower one is exposed.
    """
    P, B = Fraction(b_p), Fraction(b_h)
    t_fill = Fraction(q) / P
    if q == m:
        return t_fill
    resid = B - P
    if resid <= 0:
        return float("inf")
    return max(t_fill, Fraction(m - q) / resid)


def best_q_bruteforce(m: int, b_p, b_h, q_min: int = 1) -> int:
    """Exhaustive optimum of ``miss_latency`` over q in [q_min, m], ties to the smaller q."""
    best, best_t = None, None
    for q in range(q_min, m + 1):
        t = miss_latency(q, m, b_p, b_h)
        if best is None or t < best_t:
            best, best_t = q, t
    return best


# ----------------------------------------------------------------------------
# LRU slot cache
# ----------------------------------------------------------------------------


class LruOracle:
    """Cross-layer LRU over S slots holding (layer, expert) pairs, flat id = layer*E + e.

    State mirrors the library's device tables: slot_of [L*E] (-1 = absent),
    id_of [S] (-1 = empty), stamp [S] (0 = never used), clock, stats [8]
    (hits, misses, fills, host, evictions, calls, err, reserved).
    """

    def __init__(self, L: int, E: int, S: int):
        self.L, self.E, self.S = L, E, S
        self.slot_of = np.full(L * E, -1, dtype=np.int64)
        self.id_of = np.full(S, -1, dtype=np.int64)
        self.stamp = np.zeros(S, dtype=np.int64)
        self.clock = 0
        self.stats = np.zeros(8, dtype=np.int64)

    def install(self, flats) -> None:
        """A fixed placement made ahead of lookups: flats[i] becomes resident in slot i.
        The install is one clock tick: its slots are stamped with it, so they are more
        recent than the empty slots (stamp 0) and older than anything a later lookup
        touches.  Id -1 leaves slot i empty.  Slots that are
        occupied, other ids out of range and repeated ids are skipped and counted as
        errors (as the device call does)."""
        self.clock += 1
        for i, f in enumerate(flats):
            f = int(f)
            if i >= self.S:
                break
            if f == -1:
                continue
            if self.id_of[i] != -1 or f < 0 or f >= self.L * self.E or self.slot_of[f] != -1:
                self.stats[STAT_ERR] += 1
                continue
            self.slot_of[f] = i
            self.id_of[i] = f
            self.stamp[i] = self.clock

    def lookup(self, layer: int, ids: np.ndarray, frac_q16: int, fixed_cap: int = 1,
               min_fill: int = 1, kcap: Optional[int] = None, n_tok: Optional[int] = None) -> dict:
        """One layer call: dedup, hits, split, LRU victims, fills, rewrite."""
        ids = np.asarray(ids)
        T, k = ids.shape
        n_tok = T if n_tok is None else n_tok
        kcap = T * k if kcap is None else kcap
        self.clock += 1
        clock = self.clock

        # 1. unique flat ids of the valid routes (id -1 = masked route; other
        #    out-of-range ids count as errors and are treated as absent)
        U = set()
        for t in range(n_tok):
            for j in range(k):
                e = int(ids[t, j])
                if e == -1:
                    continue
                if e < 0 or e >= self.E:
                    self.stats[STAT_ERR] += 1
                    continue
                U.add(layer * self.E + e)
        U = sorted(U)

        # 2. hits are stamped with this call's clock
        hits = [f for f in U if self.slot_of[f] >= 0]
        for f in hits:
            self.stamp[self.slot_of[f]] = clock
        misses = [f for f in U if self.slot_of[f] < 0]
        m = len(misses)

        # 3. split count, capped by evictable slots and list capacity
        evictable = [s for s in range(self.S) if self.stamp[s] < clock]
        q = split_count(m, frac_q16, fixed_cap, min_fill)
        q = min(q, len(evictable), kcap)

        # 4. victims: smallest (stamp, slot) among the evictable slots
        victims = sorted(evictable, key=lambda s: (int(self.stamp[s]), s))[:q]
        fills = []
        for f, s in zip(misses[:q], victims):
            old = int(self.id_of[s])
            if old >= 0:
                self.slot_of[old] = -1
                self.stats[STAT_EVICT] += 1
            self.slot_of[f] = s
            self.id_of[s] = f
            self.stamp[s] = clock
            fills.append((f, s))
        host = misses[q:]

        # 5. rewrite each route to its slot, or -1 (host-computed / masked / invalid)
        slots = np.full((T, k), -1, dtype=np.int32)
        for t in range(n_tok):
            for j in range(k):
                e = int(ids[t, j])
                if 0 <= e < self.E:
                    slots[t, j] = self.slot_of[layer * self.E + e]

        self.stats[STAT_HITS] += len(hits)
        self.stats[STAT_MISSES] += m
        self.stats[STAT_FILLS] += q
        self.stats[STAT_HOST] += m - q
        self.stats[STAT_CALLS] += 1
        return {"slots": slots, "fills": fills, "host": host, "hits": hits, "m": m, "q": q}

    def state(self) -> dict:
        return {"slot_of": self.slot_of.copy(), "id_of": self.id_of.copy(),
                "stamp": self.stamp.copy(), "clock": self.clock, "stats": self.stats.copy()}


def lru_bruteforce(calls, S: int, frac_q16: int = Q16, fixed_cap: int = 1, min_fill: int = 1):
    """Second, independent LRU: a recency list of slots with linear scans.

    ``calls`` is a list of sorted-unique flat-id lists (one per layer call).  The list
    runs from least to most recently used; slots touched in one call move to the
    back in slot order.  Returns per-call (fills [(flat, slot)], host [flat], hits)
    and the final slot contents.
    """
    order = list(range(S))
    content = [None] * S
    out = []
    for U in calls:
        where = {content[s]: s for s in range(S) if content[s] is not None}
        hit_slots = [where[f] for f in U if f in where]
        misses = [f for f in U if f not in where]
        q = split_count(len(misses), frac_q16, fixed_cap, min_fill)
        free = [s for s in order if s not in hit_slots]
        q = min(q, len(free))
        victims = free[:q]
        fills = []
        for f, s in zip(misses[:q], victims):
            content[s] = f
            fills.append((f, s))
        touched = set(hit_slots) | set(victims)
        order = [s for s in order if s not in touched] + sorted(touched)
        out.append({"fills": fills, "host": misses[q:], "hits": sorted(U[i] for i in range(len(U)) if U[i] in where)})
    return out, content


def static_resident_set(warm_steps, cap: int) -> list:
    """Static (prefill-time) placement as [qiita] "5. デコード側の答え その1" defines it: the
    cap most frequent ids over the warm-up steps, fixed from then on.  Each step's routed
    ids count once per occurrence; equal counts keep the order in which the ids first
    appear (the behaviour of the page's frequency count).  Returns the ids in rank order."""
    counts = {}
    order = []
    for step in warm_steps:
        for e in np.asarray(step).ravel().tolist():
            if e not in counts:
                counts[e] = 0
                order.append(e)
            counts[e] += 1
    ranked = sorted(order, key=lambda e: (-counts[e], order.index(e)))
    return ranked[:cap]


def static_miss_counts(trace, resident) -> tuple:
    """(misses, accesses) of a fixed placement over a trace: per step the unique routed
    ids are the accesses, and those outside the placement miss ([qiita] "5.")."""
    res = set(int(e) for e in resident)
    miss = acc = 0
    for step in trace:
        u = set(int(e) for e in np.asarray(step).ravel().tolist())
        acc += len(u)
        miss += sum(1 for e in u if e not in res)
    return miss, acc
