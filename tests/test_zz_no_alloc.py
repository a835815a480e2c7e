"""The no-allocation decode entry point (moe_experts_decode_noalloc) against the
workspace one (moe_experts_decode): same kernels, so the outputs must be identical, and
both within the output bar of the oracle.  Two calls in a row, the second smaller."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_bf16_close, device_banks, t_of
from test_gpu_decode import _desc, _resident_case

pytestmark = pytest.mark.gpu


def _inputs(cfg, case):
    """Device inputs of a case; the bank tensors are returned too, since the descriptors
    hold only their addresses and the tensors must outlive every call that uses them."""
    T = case["ids"].shape[0]
    keep = {"pool": device_banks(case["banks"])}
    pool = _desc(cfg, keep["pool"])
    sh = None
    if case["shared"] is not None:
        keep["shared"] = {k: t_of(v[case["layer"]:case["layer"] + 1]).cuda() for k, v in case["shared"].items()}
        sh = _desc(cfg, keep["shared"])
    x = t_of(case["x"]).cuda()
    slots = torch.from_numpy(case["slots"]).cuda()
    w = torch.from_numpy(case["w"]).cuda()
    return T, pool, sh, x, slots, w, keep


def _both(cfg, case, nt=None):
    from expert_cache_offloaded_amd import _lib as L
    T, pool, sh, x, slots, w, keep = _inputs(cfg, case)
    ntt = None if nt is None else torch.tensor([nt], dtype=torch.int32, device="cuda")
    ws = torch.zeros(L.decode_ws_bytes(T, cfg.k, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
    y_ws = torch.full((T, cfg.H), 3.0, dtype=torch.float32, device="cuda")
    yb_ws = torch.empty((T, cfg.H), dtype=torch.int16, device="cuda")
    L.moe_experts_decode(x, slots, w, ntt, pool, sh, ws, y_ws, accumulate=0, y_bf16=yb_ws)
    y_na = torch.full((T, cfg.H), -5.0, dtype=torch.float32, device="cuda")
    yb_na = torch.empty((T, cfg.H), dtype=torch.int16, device="cuda")
    L.moe_experts_decode_noalloc(x, slots, w, ntt, pool, sh, y_na, accumulate=0, y_bf16=yb_na)
    torch.cuda.synchronize()
    return y_ws, yb_ws, y_na, yb_na


@pytest.mark.parametrize("cname,T_big,T_small,shared", [("zipf_decode", 16, 4, True),
                                                        ("qwen_decode", 1, 1, True),
                                                        ("tiny", 4, 2, False)])
def test_noalloc_equals_workspace_call(cname, T_big, T_small, shared):
    cfg = synth.CONFIGS[cname].with_(L=2)
    n_slots = {"zipf_decode": 130, "qwen_decode": 24, "tiny": 8}[cname]
    for i, T in enumerate((T_big, T_small)):                  # the second call is smaller
        case = _resident_case(cfg, T, n_slots, 0.1, seed=41 + i, shared=shared)
        y_ws, yb_ws, y_na, yb_na = _both(cfg, case)
        assert torch.equal(y_ws, y_na), (cname, T)
        assert torch.equal(yb_ws, yb_na), (cname, T)
        assert_bf16_close(yb_na, case["ref"], "%s T=%d" % (cname, T))


def test_noalloc_valid_count_after_a_larger_call():
    """A call with a device valid count after a larger one: the rows beyond the count are
    zero, and nothing left in the shared array by the earlier call leaks in."""
    cfg = synth.CONFIGS["zipf_decode"].with_(L=2)
    big = _resident_case(cfg, 16, 130, 0.0, seed=51, shared=True)
    _both(cfg, big)
    case = _resident_case(cfg, 16, 130, 0.0, seed=52, shared=True, nt=5)
    y_ws, yb_ws, y_na, yb_na = _both(cfg, case, nt=5)
    assert torch.equal(y_ws, y_na) and torch.equal(yb_ws, yb_na)
    assert torch.all(y_na[5:] == 0) and torch.all(yb_na[5:] == 0)
    assert_bf16_close(yb_na[:5], case["ref"][:5], "valid count 5")
