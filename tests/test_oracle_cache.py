"""Pins for the oracle's LRU slot cache and fetch/host split (CPU only)."""
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import (LruOracle, best_q_bruteforce, fetch_fraction_q16, lru_bruteforce, miss_latency,
                    split_count)
from oracle.cache import STAT_ERR, STAT_EVICT, STAT_FILLS, STAT_HITS, STAT_HOST, STAT_MISSES, fetch_fraction

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- split count

@pytest.mark.parametrize("row", _rows("split_worked.txt"))
def test_split_worked_values(row):
    m, bp, bh, q = int(row[0]), float(row[1]), float(row[2]), int(row[3])
    assert split_count(m, fetch_fraction_q16(bp, bh), min_fill=1) == q
    # the closed form's neighbourhood: q is floor or ceil of m B_P / B_H, or m
    qstar = Fraction(m) * Fraction(bp) / Fraction(bh)
    assert q in {qstar.__floor__(), qstar.__ceil__(), m}
    assert best_q_bruteforce(m, bp, bh) == q


@pytest.mark.parametrize("row", _rows("rounding_loss.txt"))
def test_rounding_loss(row):
    m, bp, bh, q_round, loss = int(row[0]), float(row[1]), float(row[2]), int(row[3]), float(row[4])
    assert round(m * bp / bh) == q_round
    best = best_q_bruteforce(m, bp, bh)
    got = miss_latency(q_round, m, bp, bh) / miss_latency(best, m, bp, bh) - 1
    assert round(float(got) * 100, 1) == loss


def test_split_equals_exact_bruteforce_except_near_ties():
    near_tie = []
    for m in (4, 8, 16, 32):
        for i in range(1, 100):
            bp, bh = Fraction(i, 100), Fraction(1)
            f = fetch_fraction(bp, bh)
            q16 = fetch_fraction_q16(bp, bh)
            q = split_count(m, q16, min_fill=1)
            best = best_q_bruteforce(m, bp, bh)
            if q != best:
                # the Q16 rounding of f may only flip a choice within 2^-16 of a tie f = j/(m+1)
                j = round(f * (m + 1))
                assert abs(f - Fraction(j, m + 1)) <= Fraction(1, 1 << 16), (m, i, q, best)
                near_tie.append((m, i))
    # the enumeration is small and fixed
    assert len(near_tie) <= 8, near_tie


def test_split_special_cases():
    assert split_count(0, 12345) == 0
    assert split_count(5, 1 << 16, min_fill=0) == 5          # offload: every miss is filled
    assert split_count(5, 0, fixed_cap=1) == 1                 # no profile: fixed cap of one
    assert split_count(5, 0, fixed_cap=9) == 5
    assert split_count(3, 1, min_fill=0) == 0                  # f ~ 0: everything on the host
    assert split_count(3, 1, min_fill=1) == 1                  # ... but at least one fill
    # B_H <= B_P: no residual host bandwidth, all misses fetched
    assert fetch_fraction_q16(50.0, 40.0) == 1 << 16
    assert split_count(7, fetch_fraction_q16(50.0, 50.0)) == 7


def test_overlap_form_reduces_to_ratio():
    for bp, bh in [(11.8, 47.5), (52.7, 77.3), (25.1, 63.2), (51.5, 178.0), (49.0, 53.8)]:
        P, B = Fraction(bp), Fraction(bh)
        assert fetch_fraction(0, 0, p_ov=P, c_ov=B - P) == P / B
        assert fetch_fraction_q16(bp, bh, p_ov=bp, c_ov=float(B - P)) == fetch_fraction_q16(bp, bh)


def test_q_is_neighbour_of_closed_form():
    for m in range(1, 40):
        for q16 in range(1, 1 << 16, 997):
            q = split_count(m, q16, min_fill=0)
            qstar = Fraction(m * q16, 1 << 16)
            assert q in (qstar.__floor__(), qstar.__ceil__())


# ---------------------------------------------------------------- LRU

def _random_calls(rng, n_calls, L, E, k, T):
    calls = []
    for _ in range(n_calls):
        layer = int(rng.integers(0, L))
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        calls.append((layer, ids))
    return calls


@pytest.mark.parametrize("S,frac,cap", [(1, 1 << 16, 1), (3, 1 << 16, 1), (4, 32768, 1),
                                        (7, 21845, 1), (5, 0, 1), (5, 0, 2), (12, 1 << 16, 1)])
def test_lru_matches_bruteforce(S, frac, cap):
    rng = np.random.default_rng(S * 1000 + frac + cap)
    L, E, k, T = 3, 5, 2, 2
    calls = _random_calls(rng, 300, L, E, k, T)
    lru = LruOracle(L, E, S)
    uniq = []
    res = []
    for layer, ids in calls:
        res.append(lru.lookup(layer, ids, frac, fixed_cap=cap, min_fill=1))
        uniq.append(sorted({layer * E + int(e) for e in ids.ravel()}))
    bf, content = lru_bruteforce(uniq, S, frac, cap, 1)
    for a, b in zip(res, bf):
        assert a["fills"] == b["fills"]
        assert a["host"] == b["host"]
        assert a["hits"] == b["hits"]
    assert [int(x) if x >= 0 else None for x in lru.id_of] == content
    # table consistency
    for s in range(S):
        f = int(lru.id_of[s])
        if f >= 0:
            assert lru.slot_of[f] == s
    assert np.sum(lru.slot_of >= 0) == np.sum(lru.id_of >= 0)


def test_lru_rewrite_and_stats():
    lru = LruOracle(1, 8, 4)
    ids = np.array([[0, 1], [1, 2], [3, 4], [-1, 5]], dtype=np.int32)
    r = lru.lookup(0, ids, 1 << 16)
    # 6 unique misses, 4 slots: the first 4 by flat id are filled into slots 0..3
    assert r["fills"] == [(0, 0), (1, 1), (2, 2), (3, 3)]
    assert r["host"] == [4, 5]
    assert r["slots"].tolist() == [[0, 1], [1, 2], [3, -1], [-1, -1]]
    st = lru.stats
    assert (st[STAT_HITS], st[STAT_MISSES], st[STAT_FILLS], st[STAT_HOST], st[STAT_EVICT]) == (0, 6, 4, 2, 0)
    # next call: 1 and 3 hit; misses 6, 7 evict the LRU of slots {0, 2} (stamp 1, slot order)
    r = lru.lookup(0, np.array([[1, 6], [3, 7]], np.int32), 1 << 16)
    assert r["hits"] == [1, 3] and r["fills"] == [(6, 0), (7, 2)]
    assert lru.stats[STAT_EVICT] == 2 and lru.slot_of[0] == -1 and lru.slot_of[2] == -1
    # masked rows beyond n_tok
    r = lru.lookup(0, np.array([[1, 6], [5, 4]], np.int32), 1 << 16, n_tok=1)
    assert r["m"] == 0 and r["slots"][1].tolist() == [-1, -1]


def test_install_then_lookup_hand_worked():
    """A fixed placement (installed before any lookup): id -1 leaves its slot empty and
    is no error; a duplicate, an id out of range and an occupied slot are errors and
    skipped.  The install is a clock tick of its own: its experts are more recent than
    the empty slots, which a miss takes first, and older than anything a lookup
    touches."""
    lru = LruOracle(2, 4, 5)           # flat ids 0..7
    lru.install([5, -1, 2, 5, 99])
    assert lru.id_of.tolist() == [5, -1, 2, -1, -1]
    assert lru.slot_of.tolist() == [-1, -1, 2, -1, -1, 0, -1, -1]
    assert lru.stats[STAT_ERR] == 2     # the second 5 and 99
    lru.install([7])                    # slot 0 is occupied
    assert lru.stats[STAT_ERR] == 3 and lru.slot_of[7] == -1
    # layer 1 call: expert 1 (flat 5) hits; 0, 2, 3 (flats 4, 6, 7) fill the empty slots
    r = lru.lookup(1, np.array([[1, 0], [2, 3]], np.int32), 1 << 16)
    assert r["hits"] == [5]
    assert r["fills"] == [(4, 1), (6, 3), (7, 4)]
    assert r["slots"].tolist() == [[0, 1], [3, 4]]
    # layer 0 call: expert 2 (flat 2, installed) hits; expert 0 (flat 0) must evict the
    # least recent resident: flat 2 was just refreshed, the other four carry the first
    # call's stamp, and the tie goes to the lowest slot (0, flat 5)
    r = lru.lookup(0, np.array([[2, 0]], np.int32), 1 << 16)
    assert r["hits"] == [2] and r["fills"] == [(0, 0)]
    assert lru.stats[STAT_EVICT] == 1 and lru.slot_of[5] == -1


def test_lru_reuse_distance_invariants():
    """Offload mode: D distinct keys between two accesses of a key x, S_c the key set
    of x's previous call.  |S_c| + D <= S => hit;  D >= S => miss (no overflow here)."""
    rng = np.random.default_rng(3)
    L, E, k, S = 4, 16, 3, 10
    lru = LruOracle(L, E, S)
    history = []          # list of sets of flat ids per call
    last = {}
    n_checked = 0
    for c in range(2000):
        layer = int(rng.integers(0, L))
        ids = rng.choice(E, (1, k), replace=False).astype(np.int32)
        keys = sorted({layer * E + int(e) for e in ids.ravel()})
        r = lru.lookup(layer, ids, 1 << 16)
        hits = set(r["hits"])
        for x in keys:
            if x in last:
                cp = last[x]
                D = len(set().union(*history[cp + 1:c])) if c > cp + 1 else 0
                if len(history[cp]) + D <= S:
                    assert x in hits
                    n_checked += 1
                if D >= S:
                    assert x not in hits
                    n_checked += 1
        for x in keys:
            last[x] = c
        history.append(set(keys))
    assert n_checked > 1000


def test_lru_compulsory_misses_only_when_pool_is_large():
    cfg = synth.CONFIGS["tiny"].with_(L=2, steps=30)
    tr = synth.trace(cfg)
    S = cfg.L * cfg.E
    lru = LruOracle(cfg.L, cfg.E, S)
    for s in range(cfg.steps):
        for l in range(cfg.L):
            lru.lookup(l, tr[s, l], 1 << 16)
    distinct = len({l * cfg.E + int(e) for s in range(cfg.steps) for l in range(cfg.L) for e in tr[s, l].ravel()})
    assert lru.stats[STAT_MISSES] == distinct and lru.stats[STAT_EVICT] == 0


@pytest.mark.parametrize("row", _rows("lru_replay.txt"))
def test_qiita_replay_miss_rate(row):
    E, K, steps, seed = int(row[0]), int(row[1]), int(row[2]), int(row[3])
    locality, slots, rate, tol = float(row[4]), int(row[5]), float(row[6]), float(row[7])
    tr = synth.drifting_working_set(E, K, steps, locality, seed)
    lru = LruOracle(1, E, slots)
    accesses = 0
    for s in range(steps):
        accesses += len(np.unique(tr[s]))
        lru.lookup(0, tr[s][None, :], 1 << 16)
    got = 100.0 * lru.stats[STAT_MISSES] / accesses
    assert abs(got - rate) <= tol, got


def test_recommend_backend_pages_machines():
    """[wanger] "第一层带宽比": hybrid iff the host kernel's bandwidth exceeds 2.0x the link's.
    Pinned by the pages' machines ([jjl357] "9.1 测试硬件" bandwidths): the RTX 4060 Laptop
    (B_P 11.8, B_H 47.5 GB/s) is the case whose misses largely run on the CPU branch
    ([jjl357] "12. Cross-Hardware Results": its low B_P/B_H sends more misses to the CPU); the RTX 5090 Desktop
    (49.0 / 53.8) fetches every miss over the link (q = m, [qiita] "8.")."""
    from oracle import recommend_backend
    assert recommend_backend(47.5, 11.8) == "hybrid"
    assert recommend_backend(53.8, 49.0) == "offload"
    # the threshold itself is not enough: strictly greater
    assert recommend_backend(2.0, 1.0) == "offload"
    assert recommend_backend(2.0000001, 1.0) == "hybrid"
    assert recommend_backend(3.0, 1.0, threshold=3.0) == "offload"
    assert recommend_backend(1.0, 0.0) == "hybrid"


def test_static_placement_definition():
    """Hand-evaluated cases of the static placement rule: counts over the warm-up window,
    ties in order of first appearance."""
    from oracle import static_miss_counts, static_resident_set
    assert static_resident_set([[1, 2, 3], [2, 3, 4], [3]], 2) == [3, 2]
    assert static_resident_set([[5, 6], [6, 5]], 1) == [5]
    assert static_resident_set([[7, 7, 1]], 2) == [7, 1]          # repeated ids count twice
    assert static_miss_counts([[1, 2, 2], [3, 1]], [1]) == (2, 4)  # accesses are unique per step


def test_static_placement_qiita_replay():
    """The page's printed static miss rate on its own trace (golden file)."""
    from oracle import static_miss_counts, static_resident_set
    path = os.path.join(os.path.dirname(__file__), "golden", "static_replay.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    for E, K, steps, seed, loc, slots, warm, pct, tol in rows:
        tr = synth.drifting_working_set(int(E), int(K), int(steps), float(loc), int(seed))
        res = static_resident_set(tr[: int(warm)], int(slots))
        miss, acc = static_miss_counts(tr, res)
        assert abs(100.0 * miss / acc - float(pct)) <= float(tol)
