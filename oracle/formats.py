"""Weight and activation formats (oracle side; test infrastructure only).

MXFP4 is the experts' storage format for the DeepSeek-V4-Flash-shaped runs
([jjl357] "6.9 “精确”应该怎样理解": the native MXFP4 expert blocks are consumed
bit-exactly by every engine).  The pages name the format only; its definition is
the OCP Microscaling (MX) v1.0 one: a block of 32 FP4 E2M1 elements shares one
E8M0 power-of-two scale, value = 2^(X - 127) * e2m1(code).  X = 255 (NaN) never
occurs in the synthetic weights and is rejected here.

Layout (the library's expert layout; same bytes on host and in the slot pool):
  gate_up        [2I][H/2]  codes; rows [0, I) = gate, [I, 2I) = up
  gate_up_scale  [2I][H/32] e8m0
  down           [H][I/2]   codes
  down_scale     [H][I/32]  e8m0
  byte j of a row holds element 2j in its low nibble, element 2j+1 in the high one.
bf16 experts: gate_up [2I][H] and down [H][I] as raw bf16 bits.

Parity pins (tests/test_oracle_formats.py): the 16 E2M1 codes against the list of
representable values, every (code, scale) pair against an independent
power-of-two construction, hand-built bytes for the nibble order and block
indexing, and bf16 decoding against torch's own bf16 conversion.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: the top half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e2m1_value(code: int) -> float:
    """Value of one FP4 E2M1 code: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.

    Exponent field 0 is subnormal: 0.5 * mantissa.  Otherwise 2^(e-1) * (1 + m/2).
    """
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else (2.0 ** (e - 1)) * (1.0 + 0.5 * m)
    return -mag if s else mag


_E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def decode_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed MXFP4 rows -> float64 matrix.

    codes [..., R, C/2] uint8, scales [..., R, C/32] uint8 -> [..., R, C].
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if np.any(scales == 255):
        raise ValueError("e8m0 scale 0xFF (NaN) in weights")
    lo = codes & 0x0F
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    vals = _E2M1[nib]
    C = vals.shape[-1]
    if scales.shape[-1] * 32 != C:
        raise ValueError("scale count does not match 32-element blocks")
    exps = scales.astype(np.int64) - 127
    per_elem = np.repeat(exps, 32, axis=-1)
    return np.ldexp(vals, per_elem)


def expert_matrices(banks: dict, idx: int, fmt: str, H: int, I: int):
    """Dense float64 (W_gate [I,H], W_up [I,H], W_down [H,I]) of expert entry ``idx``."""
    if fmt == "bf16":
        gu = bf16_to_f64(banks["gate_up"][idx]).reshape(2 * I, H)
        dn = bf16_to_f64(banks["down"][idx]).reshape(H, I)
    elif fmt == "mxfp4":
        gu = decode_mxfp4(np.asarray(banks["gate_up"][idx]).reshape(2 * I, H // 2),
                          np.asarray(banks["gate_up_scale"][idx]).reshape(2 * I, H // 32))
        dn = decode_mxfp4(np.asarray(banks["down"][idx]).reshape(H, I // 2),
                          np.asarray(banks["down_scale"][idx]).reshape(H, I // 32))
    else:
        raise ValueError(fmt)
    return gu[:I], gu[I:], dn
