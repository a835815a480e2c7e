"""Pins for the oracle's weight and activation formats (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import bf16_to_f64, decode_mxfp4, e2m1_value
from synth import to_bf16_bits

# OCP MX v1.0 FP4 E2M1: the eight non-negative representable magnitudes, in code order.
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_codes_match_representable_values():
    for c in range(16):
        mag = E2M1_MAGNITUDES[c & 7]
        want = -mag if c & 8 else mag
        assert e2m1_value(c) == want
        if c == 8:
            assert np.signbit(e2m1_value(c)) or e2m1_value(c) == 0.0


def test_every_code_and_scale():
    # one row of 32 * 254 elements: block b uses scale X = b (X = 0 .. 253); every code in each block
    X = np.arange(254, dtype=np.uint8)
    codes_per_block = np.array([(c & 15) | (((c + 1) & 15) << 4) for c in range(16)], dtype=np.uint8)
    codes = np.tile(codes_per_block, X.size)[None, :]
    vals = decode_mxfp4(codes, X[None, :])[0]
    for b in range(X.size):
        scale = 1.0
        e = int(X[b]) - 127
        for _ in range(abs(e)):
            scale = scale * 2.0 if e > 0 else scale / 2.0
        for i in range(32):
            byte = int(codes_per_block[i // 2])
            code = byte & 15 if i % 2 == 0 else byte >> 4
            mag = E2M1_MAGNITUDES[code & 7] * scale
            want = -mag if code & 8 else mag
            assert vals[32 * b + i] == want, (b, i)


def test_nibble_order_and_block_index():
    # byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 16] = 0x0F   # element 32 (block 1) = code 15 (-6), element 33 = 0
    scales = np.array([[127, 129]], dtype=np.uint8)     # block 0: x1, block 1: x4
    v = decode_mxfp4(codes, scales)[0]
    assert v[0] == 0.5 and v[1] == 1.0
    assert v[32] == -24.0 and v[33] == 0.0
    assert np.count_nonzero(v) == 3


def test_nan_scale_rejected():
    with pytest.raises(ValueError):
        decode_mxfp4(np.zeros((1, 16), np.uint8), np.full((1, 1), 255, np.uint8))


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint16)
    ours = bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_generator_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    a = np.concatenate([r.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8], np.float32)])
    ours = to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
