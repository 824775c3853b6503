"""Pins of the oracle's two scalar building blocks: e4m3 decode and BF16 rounding.

Each is checked against the format definitions (golden fixtures) and against an
independent library implementation (torch's float8_e4m3fn / bfloat16 casts).
"""
import math
import os
import re

import numpy as np
import pytest
import torch

from oracle import E4M3_TABLE, bf16_bits_rne, bf16_bits_to_f64, decode_e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                yield line


def test_e4m3_anchor_values():
    n = 0
    for line in _rows("e4m3_anchors.txt"):
        code, val = line.split()[:2]
        got = E4M3_TABLE[int(code, 16)]
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val), (code, got, val)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val)), code
        n += 1
    assert n >= 15


def test_e4m3_table_matches_torch_float8_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = decode_e4m3(codes.numpy())
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(ours))
    assert nan_ref.sum() == 2  # 0x7F and 0xFF only
    assert np.array_equal(ref[~nan_ref], ours[~nan_ref])
    assert np.array_equal(np.signbit(ref[~nan_ref]), np.signbit(ours[~nan_ref]))


def test_e4m3_table_structure():
    pos = E4M3_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase strictly"
    assert np.array_equal(E4M3_TABLE[0x80:0xFF], -pos)
    # every finite value times 2^9 is an integer below 2^18 (exact-sum argument)
    scaled = pos * 512
    assert np.all(scaled == np.round(scaled)) and scaled.max() < 2 ** 18


def test_bf16_fixture_cases():
    n = 0
    for line in _rows("bf16_rne_cases.txt"):
        parts = re.split(r"\s{2,}", line)
        expr, bits = parts[0], parts[1]
        x = float(eval(expr, {"__builtins__": {}}))
        got = int(bf16_bits_rne(np.array([x]))[0])
        assert got == int(bits, 16), (expr, hex(got), bits)
        n += 1
    assert n >= 15


def test_bf16_matches_torch_on_float32_inputs():
    # For values exactly representable in float32, one rounding from float64 equals
    # torch's float32 -> bfloat16 round-to-nearest-even cast.
    g = torch.Generator().manual_seed(5)
    x = torch.randn(200000, generator=g) * torch.exp2(torch.randint(-60, 60, (200000,), generator=g).float())
    # include exact ties and near-ties in float32
    base = torch.randint(-2 ** 15, 2 ** 15, (20000,), generator=g).float() * 256 + 128
    x = torch.cat([x, base, base + 1, base - 1, torch.tensor([0.0, -0.0, 1e-40, -1e-40])])
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = bf16_bits_rne(x.double().numpy())
    assert np.array_equal(ref, ours)


def test_bf16_roundtrip_and_nan():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    finite = np.isfinite(vals)
    back = bf16_bits_rne(vals[finite])
    assert np.array_equal(back, bits[finite])
    assert bf16_bits_rne(np.array([np.nan]))[0] == 0x7FC0
