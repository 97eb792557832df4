"""Pins of the oracle's decoders and E4M3 rounding (CPU only).

Each value the oracle computes is checked against something other than
itself: torch's independent float8 views and casts (library routines, run as
black boxes), golden tables of the public OCP specifications, brute force over
the whole code table, and the FNUZ relation stated in the module notes of
vllm.models.deepseek_v41.amd.mono.weights942.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                a, b = line.split()
                rows.append((int(a, 16), float(b)))
    return rows


def _same(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


def test_e4m3_all_codes_match_torch_view():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double()
    for b in range(256):
        assert _same(oracle.e4m3_value(b), ref[b].item()), hex(b)


def test_e4m3_golden_table():
    for b, v in _golden("e4m3_values.txt"):
        assert _same(oracle.e4m3_value(b), v), hex(b)


def test_e4m3_fnuz_is_half_of_ocp():
    # weights942 module notes: the FNUZ reading of a byte is half its OCP value
    # (except the codes whose meaning differs: 0x80 is FNUZ NaN, 0x7F/0xFF are
    # OCP NaN).
    fnuz = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fnuz).double()
    for b in range(256):
        if b in (0x80, 0x7F, 0xFF):
            continue
        assert fnuz[b].item() == oracle.e4m3_value(b) / 2, hex(b)


def test_e4m3_order_and_symmetry():
    vals = [oracle.e4m3_value(b) for b in range(0x7F)]
    assert all(vals[i] < vals[i + 1] for i in range(len(vals) - 1))
    for b in range(0x7F):
        assert _same(oracle.e4m3_value(b | 0x80), -oracle.e4m3_value(b))
    finite = [b for b in range(256) if not math.isnan(oracle.e4m3_value(b))]
    assert len(finite) == 254


def test_e2m1_golden_table():
    rows = _golden("e2m1_values.txt")
    assert len(rows) == 16
    for n, v in rows:
        assert _same(oracle.e2m1_value(n), v), hex(n)


def test_e8m0_all_codes_match_torch_view():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double()
    for c in range(256):
        assert _same(oracle.e8m0_value(c), ref[c].item()), c
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(0) == 2.0 ** -127


def test_bf16_decode_matches_torch_view():
    g = np.random.default_rng(1)
    bits = np.concatenate([g.integers(0, 1 << 16, 20000), np.arange(0, 1 << 16, 257)])
    bits = bits.astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    for b, r in zip(bits.tolist(), ref.tolist()):
        assert _same(oracle.bf16_value(b), r), hex(b)


def _table():
    # the 127 non-negative finite E4M3 values, from torch's decoder
    return torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _brute_round(v, table):
    """Nearest finite e4m3 by exhaustive search, ties to even code, +-448 clamp."""
    a = abs(v)
    if a >= 448.0:
        code = 0x7E
    else:
        d = np.abs(table - a)
        best = np.flatnonzero(d == d.min())
        code = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    return code | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_e4m3_round_brute_force():
    table = _table()
    g = np.random.default_rng(2)
    vals = np.concatenate([
        g.standard_normal(3000) * 100.0,
        g.standard_normal(2000) * 2.0 ** -8,
        g.uniform(-600, 600, 1000),
        (g.integers(0, 4000, 500) - 2000) * 2.0 ** -12,   # many exact ties
    ])
    for v in vals.tolist():
        assert oracle.e4m3_round(v) == _brute_round(v, table), v


def test_e4m3_round_midpoints_go_to_even():
    table = _table()
    for c in range(0x7E):
        mid = (table[c] + table[c + 1]) / 2.0
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_round(mid) == even, c
        assert oracle.e4m3_round(-mid) == (even | 0x80), c


def test_e4m3_round_matches_torch_cast_in_range():
    # torch's float32 -> float8_e4m3fn cast rounds to nearest even (it does
    # not saturate, so only |v| < 464 is compared).
    g = np.random.default_rng(3)
    f = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * np.float32(60),
        (g.standard_normal(5000) * 2.0 ** -7).astype(np.float32),
        g.uniform(-463.9, 463.9, 5000).astype(np.float32),
    ])
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, r in zip(f.tolist(), ref.tolist()):
        assert oracle.e4m3_round(v) == r, v


def test_e4m3_round_saturates_and_keeps_zero_sign():
    for v in (448.0, 449.0, 464.0, 480.0, 1e6, float("inf")):
        assert oracle.e4m3_round(v) == 0x7E
        assert oracle.e4m3_round(-v) == 0xFE
    assert oracle.e4m3_round(0.0) == 0x00
    assert oracle.e4m3_round(-0.0) == 0x80
    assert oracle.e4m3_round(-1e-9) == 0x80
    assert oracle.e4m3_round(2.0 ** -10) == 0x00          # tie with 0 -> even
    assert oracle.e4m3_round(3 * 2.0 ** -11) == 0x01      # 0.75 * 2^-9 -> 2^-9
