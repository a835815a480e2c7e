"""The library's host expert kernel (C++, runs on the CPU) against the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import decode_layer


def _banks_desc(cfg, banks):
    from expert_cache_offloaded_amd import make_banks
    t = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16) if v.dtype == np.uint16 else
                             np.ascontiguousarray(v)) for k, v in banks.items()}
    return make_banks(cfg.fmt, cfg.H, cfg.I, t), t


@pytest.mark.parametrize("fmt,H,I,T,k,threads", [("bf16", 64, 128, 4, 2, 1), ("mxfp4", 64, 64, 5, 3, 3),
                                                 ("mxfp4", 2048, 512, 1, 8, 4), ("bf16", 256, 192, 3, 4, 2),
                                                 ("mxfp4", 4096, 2048, 2, 2, 8)])
def test_host_experts_match_oracle(fmt, H, I, T, k, threads):
    from expert_cache_offloaded_amd import HostPool, host_experts
    cfg = synth.Config("t", L=2, E=8, k=k, H=H, I=I, fmt=fmt, T=T, steps=1, S=4, seed=21)
    flats = list(range(cfg.n_flat))
    banks = synth.host_pool(cfg, flats)
    desc, keep = _banks_desc(cfg, banks)
    r = np.random.default_rng(3)
    x = synth.activations(cfg, 0)
    ids = np.stack([r.choice(cfg.E, k, replace=False) for _ in range(T)]).astype(np.int32)
    if T > 1:
        ids[1, 0] = -1                     # a route marked as GPU-side
    w = r.random((T, k)).astype(np.float32)
    layer = 1
    y = torch.zeros((T, H), dtype=torch.float32)
    pool = HostPool(threads) if threads > 1 else None
    host_experts(pool, torch.from_numpy(x.view(np.int16)), torch.from_numpy(ids), torch.from_numpy(w),
                 layer, cfg.E, desc, y)
    ref = decode_layer(x, ids, w.astype(np.float64), banks, layer, cfg.E, fmt, H, I)
    err = np.linalg.norm(y.numpy() - ref) / np.linalg.norm(ref)
    assert err <= 1e-5, err
    # thread count does not change the bits
    if pool is not None:
        y1 = torch.zeros_like(y)
        host_experts(None, torch.from_numpy(x.view(np.int16)), torch.from_numpy(ids), torch.from_numpy(w),
                     layer, cfg.E, desc, y1)
        assert torch.equal(y, y1)
        pool.close()
