"""GPU parity at the edges of the MXFP4 format ([jjl357] "6.9": native MXFP4 expert blocks
are consumed bit-exactly): block exponents spread over the e8m0 range, from X = 0
(2^-127, a subnormal scale) to X - 127 = +60, including both sides of the fp16 range the
prefill down GEMM dequantises into ([-23, 13]).  Outputs are compared per group of
hidden rows that share a down-row exponent base, so tiny groups are not hidden by large
ones."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import bf16_bits_to_f64, device_banks, rel_l2, t_of
from oracle import decode_layer, prefill_per_token, route

pytestmark = pytest.mark.gpu

# (gate_up row bases, down row bases): X - 127 of the blocks (each block up to 2 below)
CASES = {
    # down rows on both sides of fp16's exact range, gate_up ordinary
    "fp16-edges": ([-7], [-26, -24, -23, -7, 13, 14, 17]),
    # tiny down scales, down to X = 0 (2^-127), against large h
    "tiny-down": ([40], [-125, -118, -110]),
    # large down scales against small h
    "large-down": ([-40], [60, 45]),
    # large gate_up scales
    "large-gate_up": ([22, 28], [-30]),
}


def _banks(cfg, flats, gu, dn):
    b = synth.alloc_banks(cfg, len(flats))
    for i, f in enumerate(flats):
        for name, arr in synth.exponent_variant(cfg, f, gu, dn).items():
            b[name][i] = arr
    return b


def _groups(H, dn):
    return [np.arange(g, H, len(dn)) for g in range(len(dn))]


def _check_groups(got, ref, dn, bar, what):
    for g, rows in enumerate(_groups(ref.shape[-1], dn)):
        a, b = got[..., rows], ref[..., rows]
        assert np.all(np.isfinite(a)), "%s group %d: non-finite output" % (what, dn[g])
        assert np.linalg.norm(b) > 0, "%s group %d: the reference is zero" % (what, dn[g])
        r = rel_l2(a, b)
        assert r <= bar, "%s down base %d: rel_l2 %.3g" % (what, dn[g], r)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("T", [1, 4])
def test_decode_e8m0_range(name, T):
    """Both decode paths (one token: dot products in fp32; several: bf16 MFMA with h split
    into two bf16 halves) against the oracle, per down-exponent group."""
    from expert_cache_offloaded_amd import _lib as L
    gu, dn = CASES[name]
    cfg = synth.CONFIGS["zipf_decode"].with_(L=1, E=16, k=4, T=T)
    r = np.random.default_rng(len(name) * 7 + T)
    ids = np.stack([r.choice(cfg.E, cfg.k, replace=False) for _ in range(T)]).astype(np.int32)
    w = r.random((T, cfg.k)).astype(np.float32)
    banks = _banks(cfg, range(cfg.E), gu, dn)
    keep = device_banks(banks)
    pool = L.make_banks(cfg.fmt, cfg.H, cfg.I, keep)
    x = synth.activations(cfg, 3, T=T)
    ws = torch.zeros(L.decode_ws_bytes(T, cfg.k, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    y = torch.zeros((T, cfg.H), dtype=torch.float32, device="cuda")
    L.moe_experts_decode(t_of(x).cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), None,
                         pool, None, ws, y, accumulate=0)
    torch.cuda.synchronize()
    ref = decode_layer(x, ids, w.astype(np.float64), banks, 0, cfg.E, cfg.fmt, cfg.H, cfg.I)
    _check_groups(y.cpu().numpy().astype(np.float64), ref, dn, 1e-4, "decode %s T=%d" % (name, T))


def _prefill(cfg, x, ids, w, banks):
    from expert_cache_offloaded_amd import _lib as L
    T, k = ids.shape
    keep = device_banks(banks)
    buf = L.make_banks(cfg.fmt, cfg.H, cfg.I, keep)
    ws = torch.empty(L.prefill_ws_bytes(T, k, cfg.E, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    y = torch.zeros((T, cfg.H), dtype=torch.int16, device="cuda")
    L.moe_experts_prefill(t_of(x).cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), None,
                          cfg.E, buf, ws, y)
    rc, status = L.prefill_status(ws)
    return y, rc, status


def test_prefill_down_rows_outside_fp16_range_are_exact():
    """W_down rows with blocks on both sides of fp16's exact range (and X = 0 blocks inside
    rows whose largest block is ordinary): the layer equals the oracle per group, and the
    call reports no status bit."""
    from expert_cache_offloaded_amd import _lib as L
    dn = [-30, -26, -24, -23, -7, 13, 14, 20]
    cfg = synth.CONFIGS["prefill"].with_(L=1, E=8, k=2, H=256, I=128, T=96)
    banks = _banks(cfg, range(cfg.E), [-7], dn)
    # a few X = 0 blocks inside ordinary rows (their share is far below fp32 rounding)
    banks["down_scale"][:, 4::len(dn), 1] = 0
    x = synth.activations(cfg, 5)
    ids, w = route(synth.uniform_logits(cfg), cfg.k)
    w32 = w.astype(np.float32)
    y, rc, status = _prefill(cfg, x, ids, w32, banks)
    assert rc == L.MC_OK and status == 0
    ref = prefill_per_token(x, ids, w32.astype(np.float64), banks, cfg.E, cfg.fmt, cfg.H, cfg.I)
    _check_groups(bf16_bits_to_f64(y), ref, dn, 2e-3, "prefill fp16 edges")


def test_prefill_reports_h_beyond_fp16():
    """gate_up scales that drive h = silu(g) * u past 65504: the status word says so and the
    status call returns MC_EDEVICE; an ordinary layer on the same workspace clears it."""
    from expert_cache_offloaded_amd import _lib as L
    cfg = synth.CONFIGS["prefill"].with_(L=1, E=8, k=2, H=256, I=128, T=64)
    x = synth.activations(cfg, 6)
    ids, w = route(synth.uniform_logits(cfg), cfg.k)
    w32 = w.astype(np.float32)
    _, rc, status = _prefill(cfg, x, ids, w32, _banks(cfg, range(cfg.E), [16], [-7]))
    assert rc == L.MC_EDEVICE and status & 1
    _, rc, status = _prefill(cfg, x, ids, w32, _banks(cfg, range(cfg.E), [-7], [-7]))
    assert rc == L.MC_OK and status == 0
