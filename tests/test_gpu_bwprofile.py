"""GPU: the start-up bandwidth profile (fill kernel vs host expert kernel, alone and overlapped)."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import empty_device_banks, pinned_banks, t_of
from oracle import fetch_fraction_q16, recommend_backend

pytestmark = pytest.mark.gpu


def test_bandwidth_profile_qwen_shaped():
    from expert_cache_offloaded_amd import HostPool, bandwidth_profile
    from expert_cache_offloaded_amd import _lib as L
    cfg = synth.CONFIGS["qwen_decode"].with_(L=1, E=24)
    host_np = synth.host_pool(cfg)
    host_t = pinned_banks(cfg, host_np)
    pool_t = empty_device_banks(cfg, 8)
    host, pool = L.make_banks(cfg.fmt, cfg.H, cfg.I, host_t), L.make_banks(cfg.fmt, cfg.H, cfg.I, pool_t)
    hp = HostPool(4)
    prof = bandwidth_profile(host, pool, hp, 6, seconds=0.4)
    hp.close()
    torch.cuda.synchronize()
    print(prof)
    assert prof["expert_bytes"] == synth.expert_bytes(cfg.H, cfg.I, cfg.fmt)
    for key in ("pcie_gbs", "cpu_gbs", "pcie_ov_gbs", "cpu_ov_gbs"):
        assert 0.05 < prof[key] < 1000.0, key
    # the fraction and the backend follow the page's rules from the measured rates
    ref = fetch_fraction_q16(prof["pcie_gbs"], prof["cpu_gbs"], prof["pcie_ov_gbs"], prof["cpu_ov_gbs"])
    assert abs(int(prof["frac_q16"]) - ref) <= 1
    assert prof["backend"] == recommend_backend(prof["cpu_gbs"], prof["pcie_gbs"], 2.0)
    # each call moves on to the next 6 of the 24 host entries (the window is the whole
    # pool here): the last call left entries off .. off+5 in slots 0..5, one off for all
    got = {name: arr.cpu() for name, arr in pool_t.items()}
    offs = [o for o in range(0, 24, 6) if torch.equal(got["gate_up"][0], t_of(host_np["gate_up"][o]))]
    assert len(offs) == 1, offs
    for name in got:
        for i in range(6):
            assert torch.equal(got[name][i], t_of(host_np[name][offs[0] + i])), (name, i)


def test_bandwidth_profile_rejects_bad_arguments():
    from expert_cache_offloaded_amd import McError, bandwidth_profile
    from expert_cache_offloaded_amd import _lib as L
    cfg = synth.CONFIGS["tiny"]
    host_t = pinned_banks(cfg, synth.host_pool(cfg))
    pool_t = empty_device_banks(cfg, 2)
    host, pool = L.make_banks(cfg.fmt, cfg.H, cfg.I, host_t), L.make_banks(cfg.fmt, cfg.H, cfg.I, pool_t)
    with pytest.raises(McError):
        bandwidth_profile(host, pool, None, 3, seconds=0.1)      # more experts than pool slots
    with pytest.raises(McError):
        bandwidth_profile(host, pool, None, 2, seconds=0.0)
