"""The C ABI library loads and exports what include/mc.h declares; host-side
argument validation (no GPU work is enqueued by these calls)."""
import ctypes as C
import os
import re

import pytest

from oracle import fetch_fraction_q16 as oracle_q16

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "mc.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", src))
    skip = {"if", "for", "while", "return", "sizeof", "defined"}
    return sorted(n for n in names if n not in skip and (n.startswith("mc_") or n.startswith("moe_")
                                                       or n in ("slot_cache_lookup_evict", "hybrid_split_merge")))


def test_header_declares_the_hot_path():
    names = _declared()
    for n in ("moe_route", "slot_cache_lookup_evict", "moe_experts_decode", "hybrid_split_merge",
              "mc_fill_slots"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from expert_cache_offloaded_amd import _lib
    lib = _lib.lib()
    for n in _declared():
        assert hasattr(lib, n), n
    # and the binding covers every declared entry point
    assert set(_declared()) <= set(_lib.declared_symbols())


def test_abi_version():
    from expert_cache_offloaded_amd import abi_version
    assert abi_version() == 1


@pytest.mark.parametrize("bp,bh,pov,cov", [(11.8, 47.5, 0, 0), (52.7, 77.3, 0, 0), (49.0, 53.8, 0, 0),
                                           (1.0, 4.0, 0, 0), (50.0, 40.0, 0, 0), (0, 0, 0, 0),
                                           (0, 0, 30.0, 10.0), (0, 0, 12.5, 0.0), (1e-9, 1.0, 0, 0)])
def test_fetch_fraction_matches_oracle(bp, bh, pov, cov):
    from expert_cache_offloaded_amd import fetch_fraction_q16
    assert fetch_fraction_q16(bp, bh, pov, cov) == oracle_q16(bp, bh, pov, cov)


def test_validation_errors_do_not_need_a_gpu():
    from expert_cache_offloaded_amd import _lib as L
    lib = L.lib()
    ids = (C.c_int32 * 8)()
    w = (C.c_float * 8)()
    lg = (C.c_float * 64)()
    # k = 0, k > E, E too large, renorm out of range
    assert lib.moe_route(lg, 4, 16, 0, 1, ids, w, None) == L.MC_EINVAL
    assert lib.moe_route(lg, 4, 2, 3, 1, ids, w, None) == L.MC_EINVAL
    assert lib.moe_route(lg, 1, 4096, 2, 1, ids, w, None) == L.MC_EINVAL
    assert lib.moe_route(lg, 4, 16, 2, 7, ids, w, None) == L.MC_EINVAL
    assert "renorm" in L.last_error()
    # empty batch: nothing to do
    assert lib.moe_route(lg, 0, 16, 2, 1, ids, w, None) == L.MC_OK
    # cache checks
    c = L.Cache()
    c.L, c.E, c.S = 2, 8, 4
    assert lib.slot_cache_lookup_evict(C.byref(c), 0, ids, 4, 2, None, 65536, 1, 1, ids, ids, ids, ids,
                                       ids, ids, 8, None) == L.MC_EINVAL        # NULL tables
    buf = (C.c_int64 * 64)()
    c.slot_of = c.id_of = c.stamp = c.clock = c.stats = C.cast(buf, C.c_void_p)
    assert lib.slot_cache_lookup_evict(C.byref(c), 2, ids, 4, 2, None, 65536, 1, 1, ids, ids, ids, ids,
                                       ids, ids, 8, None) == L.MC_EINVAL        # layer out of range
    assert lib.slot_cache_lookup_evict(C.byref(c), 0, ids, 4, 2, None, 65537, 1, 1, ids, ids, ids, ids,
                                       ids, ids, 8, None) == L.MC_EINVAL        # frac > 1
    assert lib.slot_cache_lookup_evict(C.byref(c), 0, ids, 4, 2, None, 65536, 1, 1, ids, ids, ids, ids,
                                       ids, ids, 7, None) == L.MC_EINVAL        # kcap < T*k
    assert "kcap" in L.last_error()
    # bank checks
    b = L.Banks()
    b.fmt, b.H, b.I, b.n = L.MC_MXFP4, 100, 64, 4
    assert lib.moe_experts_decode(ids, ids, w, 1, 2, None, C.byref(b), None, ids, 0, w, 0, None, None, None) == L.MC_EINVAL
    assert "multiples of 64" in L.last_error()
    b.H = 64
    assert lib.moe_experts_decode(ids, ids, w, 1, 2, None, C.byref(b), None, ids, 0, w, 0, None, None, None) == L.MC_EINVAL
    # fill lists longer than the fill grid's entry dimension
    big = (C.c_uint8 * 64)()
    addr = (C.addressof(big) + 15) // 16 * 16
    fb = L.Banks()
    fb.fmt, fb.H, fb.I, fb.n = L.MC_MXFP4, 64, 64, 4
    fb.gate_up = fb.gate_up_scale = fb.down = fb.down_scale = addr
    assert lib.mc_fill_slots(C.byref(fb), C.byref(fb), ids, ids, ids, 65536, None) == L.MC_EINVAL
    assert "kcap" in L.last_error()
    assert lib.mc_fill_slots(C.byref(fb), C.byref(fb), ids, ids, ids, -1, None) == L.MC_EINVAL
    # a fill list of an unknown mode is refused before any device work
    ws_n = lib.moe_experts_decode_ws_bytes(1, 2, 64, 64)
    ws = (C.c_uint8 * (ws_n + 16))()
    ws_addr = (C.addressof(ws) + 15) // 16 * 16
    fl = L.FillList()
    fl.host = C.pointer(fb)
    fl.fill_flat = fl.fill_slot = fl.n_fill = C.cast(ids, C.c_void_p)
    fl.kcap, fl.mode = 2, 7
    assert lib.moe_experts_decode(addr, ids, w, 1, 2, None, C.byref(fb), None, ws_addr, ws_n, w, 0, None, None,
                                  C.byref(fl)) == L.MC_EINVAL
    assert "fill mode" in L.last_error()
    assert lib.mc_host_pool_create(0, None) is None


def test_host_pool_lifecycle():
    from expert_cache_offloaded_amd import HostPool
    for n in (1, 2, 5):
        p = HostPool(n)
        p.close()


@pytest.mark.parametrize("cpu,pcie,thr", [(47.5, 11.8, 2.0), (53.8, 49.0, 2.0), (2.0, 1.0, 2.0),
                                          (2.0000001, 1.0, 2.0), (30.0, 10.0, 3.0), (31.0, 10.0, 3.0),
                                          (1.0, 0.0, 2.0), (0.0, 5.0, 2.0)])
def test_recommend_backend_matches_oracle(cpu, pcie, thr):
    from expert_cache_offloaded_amd import recommend_backend
    from oracle import recommend_backend as ref
    assert recommend_backend(cpu, pcie, thr) == ref(cpu, pcie, thr)


def test_bw_profile_store_roundtrip(tmp_path):
    from expert_cache_offloaded_amd.runtime import load_fetch_fraction, save_bw_profile
    p = str(tmp_path / "bw.json")
    assert load_fetch_fraction(p, "mxfp4", "gfx950") == 0            # no profile: fixed cap
    save_bw_profile(p, {"frac_q16": 20000, "pcie_gbs": 50.0}, "mxfp4", "gfx950")
    save_bw_profile(p, {"frac_q16": 65536}, "bf16", "gfx950")
    assert load_fetch_fraction(p, "mxfp4", "gfx950") == 20000
    assert load_fetch_fraction(p, "bf16", "gfx950") == 65536
    assert load_fetch_fraction(p, "mxfp4", "other") == 0


def test_static_placement_matches_oracle():
    import numpy as np
    import synth
    from expert_cache_offloaded_amd.runtime import static_placement
    from oracle import static_resident_set
    tr = synth.drifting_working_set(256, 8, 600, 0.95, 20260825)
    for cap in (1, 8, 64, 200):
        assert static_placement(tr[:512], cap).tolist() == static_resident_set(tr[:512], cap)
    r = np.random.default_rng(4)
    for _ in range(20):
        w = r.integers(0, 40, size=(r.integers(1, 30), 6))
        assert static_placement(w, 10).tolist() == static_resident_set(w, 10)


def test_host_forget_needs_no_gpu():
    """mc_host_forget drops remembered host translations; with none remembered for an
    address it drops nothing, and NULL is refused."""
    from expert_cache_offloaded_amd import _lib
    buf = C.create_string_buffer(64)
    assert _lib.host_forget(C.addressof(buf), 64) == 0
    with pytest.raises(_lib.McError):
        _lib.host_forget(0, 0)


def test_noalloc_rejects_oversized_calls_without_a_gpu():
    """moe_experts_decode_noalloc checks the workspace a call needs against its scratch
    array before anything is enqueued: a call beyond it fails with MC_ENOMEM."""
    from expert_cache_offloaded_amd import _lib
    lib = _lib.lib()
    assert lib.moe_experts_decode_noalloc_max_bytes() == 4 << 20
    buf = C.create_string_buffer(4096 + 16)
    base = (C.addressof(buf) + 15) & ~15
    b = _lib.Banks()
    b.fmt, b.H, b.I, b.n = _lib.MC_MXFP4, 4096, 2048, 1
    b.gate_up = b.gate_up_scale = b.down = b.down_scale = base
    need = lib.moe_experts_decode_ws_bytes(64, 16, 4096, 2048)
    assert need > 4 << 20
    rc = lib.moe_experts_decode_noalloc(base, base, base, 64, 16, None, C.byref(b), None, base, 0, None,
                                        None, None)
    assert rc == _lib.MC_ENOMEM
    assert "scratch array" in _lib.last_error()


def test_host_pool_pins_physical_cores_by_default():
    """[jjl357] "8.3": the workers are pinned to physical cores.  With no CPU list the pool's
    threads take distinct CPUs of this process's affinity set, one per physical core before
    any second hardware thread, leaving one CPU to the rest of the process (threads beyond
    the others stay unpinned); an explicit list is taken as given, -1 leaving a thread free."""
    import os
    from expert_cache_offloaded_amd import HostPool
    allowed = sorted(os.sched_getaffinity(0))

    def core_of(c):
        try:
            with open("/sys/devices/system/cpu/cpu%d/topology/core_id" % c) as f:
                core = int(f.read())
            with open("/sys/devices/system/cpu/cpu%d/topology/physical_package_id" % c) as f:
                return (int(f.read()), core)
        except OSError:
            return (0, 100000 + c)

    n_cores = len({core_of(c) for c in allowed})
    n = min(4, len(allowed))
    p = HostPool(n)
    cpus = p.cpus()
    p.close()
    pinned = [c for c in cpus if c >= 0]
    assert len(cpus) == n and len(pinned) == min(n, len(allowed) - 1)
    assert all(c in allowed for c in pinned) and len(set(pinned)) == len(pinned)
    assert len(set(allowed) - set(pinned)) >= 1               # one CPU left to the process
    if len(pinned) < n_cores:
        assert len({core_of(c) for c in pinned}) == len(pinned)   # distinct physical cores
    # as many threads as allowed CPUs: every CPU but one pinned, the last thread free
    p = HostPool(len(allowed))
    cpus = p.cpus()
    p.close()
    assert cpus[-1] == -1 and len({c for c in cpus if c >= 0}) == len(allowed) - 1
    p = HostPool(2, [allowed[0], -1])
    assert p.cpus() == [allowed[0], -1]
    p.close()
