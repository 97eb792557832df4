"""Pins of the oracle's ingest variants (CPU only).

orc_fold_row_codes ([rocm_native] _as_block32_scale, [weights942]
linear_copy) and orc_e4m3_from_dequant ([weights942] ocp_from_dequant) are
checked against things other than themselves: brute force over all 65,536
bf16 patterns and all finite e4m3 bytes, round trips whose bf16 weights come
from torch's CPU cast, the definition of exact recovery stated with numpy on
a mix of representable and perturbed weights, and the pinned dense linear of
the oracle on folded and expanded codes."""
import numpy as np
import pytest
import torch

import oracle
from microscaling_quantized_linear_amd import workloads as wl

E4M3, ROW32, BLK32 = 0, 0, 1


# ------------------------------------------------------------------ fold

def test_fold_inverts_row_expansion_and_refuses_disagreement():
    rng = np.random.default_rng(81)
    N, KB = 96, 7
    blk = wl.codes(rng, (N // 32, KB), 110, 140)
    rows = np.repeat(blk, 32, axis=0)
    np.testing.assert_array_equal(oracle.fold_row_codes(N, KB, rows), blk)
    for (n, b) in [(0, 0), (31, 6), (32, 3), (95, 0), (64 + 17, 4)]:
        bad = rows.copy()
        bad[n, b] ^= 1
        with pytest.raises(ValueError):
            oracle.fold_row_codes(N, KB, bad)
    with pytest.raises(ValueError):
        oracle.fold_row_codes(48, KB, rows[:48])            # N not a multiple of 32


def test_fold_keeps_the_linear():
    """The linear with folded BLK32 codes equals the linear with the
    row-expanded ROW32 codes, sum for sum (oracle linear, pinned elsewhere)."""
    rng = np.random.default_rng(82)
    N, K, M = 64, 160, 3
    w = wl.e4m3_bytes(rng, (N, K))
    blk = wl.codes(rng, (N // 32, K // 32), 118, 134)
    rows = np.repeat(blk, 32, axis=0)
    x = wl.activations(rng, (M, K))
    folded = oracle.fold_row_codes(N, K // 32, rows)
    y_blk = oracle.linear(E4M3, BLK32, N, K, w, folded.reshape(-1), M, 0, x=x)
    y_row = oracle.linear(E4M3, ROW32, N, K, w, rows.reshape(-1), M, 0, x=x)
    np.testing.assert_array_equal(y_blk, y_row)


# ------------------------------------------------------------------ e4m3 from bf16

def _torch_bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _e4m3_table():
    """The 254 finite e4m3 values, from torch's CPU float8_e4m3fn view."""
    b = np.array([i for i in range(256) if i & 0x7F != 0x7F], np.uint8)
    v = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return b, v


@pytest.mark.parametrize("code", [0, 1, 3, 4, 9, 100, 127, 150, 246, 250, 254, 255])
def test_from_dequant_brute_force_over_all_bf16(code):
    """Every bf16 pattern under one block code: recovered exactly when some
    finite e4m3 byte times 2^(code - 127) equals it (brute force over the 254
    bytes, torch's decode), with the sign of zero kept; else refused."""
    N, K = 2048, 32
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(N, K)
    codes = np.full((N // 32, 1), code, np.uint8)
    got = oracle.e4m3_from_dequant(BLK32, N, K, w, codes, strict=False).reshape(-1)
    wv = torch.from_numpy(w.reshape(-1).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()
    b, v = _e4m3_table()
    want = np.full(65536, 0xFF, np.uint8)
    if code != 255:
        scaled = np.ldexp(v, code - 127)                # exact in binary64
        for byte, val in zip(b, scaled):
            hit = (wv == val) & (np.signbit(wv) == bool(byte & 0x80))
            assert not (want[hit] != 0xFF).any()        # at most one byte per weight
            want[hit] = byte
    np.testing.assert_array_equal(got, want)
    if code != 255:
        assert (got != 0xFF).sum() >= 100               # the case is not vacuous


def test_from_dequant_round_trip_of_dequantized_bytes():
    """Bytes dequantized to bf16 (torch's cast of the exact product) come
    back unchanged, both code layouts, including -0 (0x80)."""
    rng = np.random.default_rng(83)
    N, K = 64, 96
    q = wl.e4m3_bytes(rng, (N, K))
    q[0, :4] = [0x00, 0x80, 0x01, 0x81]
    blk = wl.codes(rng, (N // 32, K // 32), 100, 150)
    rows = np.repeat(blk, 32, axis=0)
    b, v = _e4m3_table()
    val = np.zeros(256)
    val[b] = v
    scale = np.ldexp(1.0, rows.astype(np.int64) - 127).repeat(32, axis=1)
    w = _torch_bf16_bits(val[q] * scale)
    np.testing.assert_array_equal(oracle.e4m3_from_dequant(BLK32, N, K, w, blk), q)
    np.testing.assert_array_equal(oracle.e4m3_from_dequant(ROW32, N, K, w, rows), q)
    # strided bf16 rows
    wpad = np.zeros((N, K + 8), np.uint16)
    wpad[:, :K] = w
    np.testing.assert_array_equal(oracle.e4m3_from_dequant(BLK32, N, K, wpad, blk), q)
    # one weight off by a bf16 ulp (the low mantissa bit of a normal value
    # that e4m3 cannot carry) is refused
    i = np.argwhere((w & 0x7F80) != 0)[5]
    bad = w.copy()
    bad[tuple(i)] ^= 1
    with pytest.raises(ValueError):
        oracle.e4m3_from_dequant(BLK32, N, K, bad, blk)
    got = oracle.e4m3_from_dequant(BLK32, N, K, bad, blk, strict=False)
    assert got[tuple(i)] == 0xFF and (got != 0xFF).sum() == N * K - 1


def test_from_dequant_mixed_weights_by_definition():
    """A mix of representable and perturbed bf16 weights under 32x32 codes:
    a weight w is recovered exactly when w * 2^(127 - c), formed exactly in
    binary64, is one of the finite e4m3 values (a zero keeping its sign), and
    its byte is that value's; every other weight is refused (0xFF)."""
    rng = np.random.default_rng(84)
    N, K = 128, 128
    blk = wl.codes(rng, (N // 32, K // 32), 110, 140)
    c = np.repeat(np.repeat(blk, 32, axis=0), 32, axis=1).astype(np.int64)
    q = wl.e4m3_bytes(rng, (N, K))
    b, v = _e4m3_table()
    val = np.zeros(256)
    val[b] = v
    exact = val[q] * np.ldexp(1.0, c - 127)
    noisy = exact * (1 + rng.standard_normal((N, K)) * 0.02)
    w = _torch_bf16_bits(np.where(rng.random((N, K)) < 0.5, exact, noisy))
    got = oracle.e4m3_from_dequant(BLK32, N, K, w, blk, strict=False)
    wv = wl.bf16_bits_to_f32(w).astype(np.float64)
    scaled = np.ldexp(wv, 127 - c)                          # exact: a power of two
    byte_of = {float(x): int(y) for x, y in zip(v, b) if x != 0}
    want = np.full((N, K), 0xFF, np.uint8)
    for idx in np.ndindex(N, K):
        x = scaled[idx]
        if x == 0:
            want[idx] = 0x80 if np.signbit(x) else 0x00
        elif x in byte_of:
            want[idx] = byte_of[x]
    np.testing.assert_array_equal(got, want)
    assert 0.3 < (want != 0xFF).mean() < 0.9


def test_from_dequant_refuses_nonfinite_and_bad_shapes():
    N, K = 32, 32
    codes = np.full((1, 1), 127, np.uint8)
    w = np.full((N, K), 0x3F80, np.uint16)                 # 1.0: byte 0x38
    assert (oracle.e4m3_from_dequant(BLK32, N, K, w, codes) == 0x38).all()
    for bits in (0x7FC0, 0x7F80, 0xFF80):                  # NaN, +Inf, -Inf
        ww = w.copy()
        ww[3, 7] = bits
        with pytest.raises(ValueError):
            oracle.e4m3_from_dequant(BLK32, N, K, ww, codes)
    with pytest.raises(ValueError):
        oracle.e4m3_from_dequant(BLK32, N, K, w, np.full((1, 1), 255, np.uint8))
    with pytest.raises(ValueError):
        oracle.e4m3_from_dequant(BLK32, 48, K, np.full((48, K), 0x3F80, np.uint16), codes)
