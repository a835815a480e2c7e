"""Helpers shared by the GPU tests: move synth inputs into torch device/pinned memory."""
import numpy as np
import torch

import synth


def t_of(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a)


def pinned_banks(cfg, banks_np):
    out = {}
    for k, v in banks_np.items():
        src = t_of(v)
        dst = torch.empty(src.shape, dtype=src.dtype, pin_memory=True)
        dst.copy_(src)
        out[k] = dst
    return out


def device_banks(banks_np, device="cuda"):
    return {k: t_of(v).to(device) for k, v in banks_np.items()}


def empty_device_banks(cfg, n, device="cuda"):
    from expert_cache_offloaded_amd.runtime import alloc_banks
    return alloc_banks(n, cfg.H, cfg.I, cfg.fmt, device=device)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def bf16_bits_to_f64(t: torch.Tensor) -> np.ndarray:
    from oracle import bf16_to_f64
    return bf16_to_f64(t.cpu().numpy().view(np.uint16))


def assert_bf16_close(y_bits: torch.Tensor, ref: np.ndarray, what=""):
    """The output bar: rel-L2 <= 2e-3 and max-abs <= 1e-2 against the fp64 oracle."""
    y = bf16_bits_to_f64(y_bits)
    r = rel_l2(y, ref)
    m = float(np.max(np.abs(y - ref))) if ref.size else 0.0
    assert r <= 2e-3 and m <= 1e-2, "%s rel_l2=%.3g max_abs=%.3g" % (what, r, m)
    return r, m
