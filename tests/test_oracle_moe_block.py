"""Pins of the oracle's MoE-block functions (CPU only).

orc_moe_copies, orc_silu, orc_bf16_round, orc_moe_gate_up and
orc_moe_linear_rows are each checked against something other than
themselves: torch's CPU cast, closed forms and identities of SiLU, the
inverse of the copy, and the already pinned dense / grouped linear of the
oracle on the same data (exact binary64 equality where the sums are the same
sums in the same order)."""
import math

import numpy as np
import pytest
import torch

import oracle
from microscaling_quantized_linear_amd import workloads as wl

E4M3, E2M1, ROW32 = 0, 1, 0


# ------------------------------------------------------------------ bf16 rounding

def _torch_bf16_bits(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(71)
    v = np.concatenate([
        rng.standard_normal(20000),
        rng.standard_normal(5000) * 1e30,
        rng.standard_normal(5000) * 1e-38,            # around the subnormal range
        rng.standard_normal(2000) * 1e-40,
        np.ldexp(rng.random(2000) + 1.0, rng.integers(-140, 128, 2000)),
    ])
    got = oracle.bf16_round_array(v)
    np.testing.assert_array_equal(got, _torch_bf16_bits(v))


def test_bf16_round_ties_to_even_and_edges():
    rng = np.random.default_rng(72)
    # exact midpoints between neighbouring bf16 values go to the even one
    bits = rng.integers(0x0080, 0x7F7F, 5000, dtype=np.int64).astype(np.uint16)
    lo = wl.bf16_bits_to_f32(bits).astype(np.float64)
    hi = wl.bf16_bits_to_f32(bits + 1).astype(np.float64)
    mid = (lo + hi) / 2
    even = np.where(bits % 2 == 0, bits, bits + 1).astype(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_round_array(mid), even)
    np.testing.assert_array_equal(oracle.bf16_round_array(-mid), even | 0x8000)
    # signed zeros, the largest value, overflow at half an ulp above it
    assert oracle.bf16_round(0.0) == 0 and oracle.bf16_round(-0.0) == 0x8000
    big = float.fromhex("0x1.fe0000p+127")
    ulp = float.fromhex("0x1p+120")
    assert oracle.bf16_round(big) == 0x7F7F
    assert oracle.bf16_round(big + ulp * 0.49) == 0x7F7F
    assert oracle.bf16_round(big + ulp * 0.5) == 0x7F80
    assert oracle.bf16_round(-1e39) == 0xFF80


# ------------------------------------------------------------------ SiLU

def test_silu_closed_forms_and_identity():
    assert oracle.silu(0.0) == 0.0
    l3 = math.log(3.0)                     # sigmoid(ln 3) = 3/4
    assert abs(oracle.silu(l3) - 0.75 * l3) <= 1e-15
    assert abs(oracle.silu(-l3) + 0.25 * l3) <= 1e-15
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15
    rng = np.random.default_rng(73)
    for v in rng.standard_normal(2000) * 8:
        # sigmoid(v) + sigmoid(-v) = 1
        assert abs(oracle.silu(v) - oracle.silu(-v) - v) <= 4e-16 * max(1.0, abs(v))


# ------------------------------------------------------------------ expert copies

def _experts(rng, elem, E, Np, inter, K, H):
    rowb = K // 2 if elem == E2M1 else K
    gen = (lambda shape: wl.fp4_bytes(rng, shape)) if elem == E2M1 else \
        (lambda shape: wl.e4m3_bytes(rng, shape))
    w13 = gen((E, 2 * Np, rowb))
    w13[:, inter:Np] = 0
    w13[:, Np + inter:] = 0
    s13 = wl.codes(rng, (E, 2 * Np, K // 32), 120, 134)
    r2 = Np // 2 if elem == E2M1 else Np
    w2 = gen((E, H, r2))
    w2[:, :, (inter // 2 if elem == E2M1 else inter):] = 0
    s2 = wl.codes(rng, (E, H, Np // 32), 120, 134)
    return w13, s13, w2, s2


@pytest.mark.parametrize("elem,E,Np,inter,K,H", [(E2M1, 3, 96, 64, 128, 32),
                                                 (E2M1, 2, 64, 64, 256, 16),
                                                 (E4M3, 2, 64, 32, 96, 48)])
def test_moe_copies_inverse_and_linear_invariance(elem, E, Np, inter, K, H):
    rng = np.random.default_rng([74, elem, E, Np, inter, K, H])
    w13, s13, w2, s2 = _experts(rng, elem, E, Np, inter, K, H)
    ow13, os13, ow2, os2 = oracle.moe_copies(elem, E, Np, inter, K, H, w13, s13, w2, s2)
    # inverse: even rows are the gate rows, odd rows the up rows; re-padding
    # with zero rows gives the input weights back
    back = np.zeros_like(w13)
    back[:, :inter] = ow13[:, 0::2]
    back[:, Np:Np + inter] = ow13[:, 1::2]
    np.testing.assert_array_equal(back, w13)
    np.testing.assert_array_equal(os13[:, 0::2], s13[:, :inter])
    np.testing.assert_array_equal(os13[:, 1::2], s13[:, Np:Np + inter])
    # the linear over the copies equals the linear over the original rows,
    # sum for sum (oracle linear, pinned separately)
    x = wl.activations(rng, (3, K))
    for e in range(E):
        full = oracle.linear(elem, ROW32, 2 * Np, K, w13[e], s13[e].reshape(-1), 3, 0, x=x)
        cop = oracle.linear(elem, ROW32, 2 * inter, K, ow13[e], os13[e].reshape(-1), 3, 0, x=x)
        np.testing.assert_array_equal(cop[:, 0::2], full[:, :inter])
        np.testing.assert_array_equal(cop[:, 1::2], full[:, Np:Np + inter])
        # w2 cut to inter: the same sums as over Np with zero padding
        a = wl.activations(rng, (2, Np))
        a[:, inter:] = 0
        y_full = oracle.linear(elem, ROW32, H, Np, w2[e], s2[e].reshape(-1), 2, 0, x=a)
        y_cut = oracle.linear(elem, ROW32, H, inter, ow2[e], os2[e].reshape(-1), 2, 0,
                              x=np.ascontiguousarray(a[:, :inter]))
        np.testing.assert_array_equal(y_cut, y_full)


def test_moe_copies_refuses_nonzero_padding():
    E, Np, inter, K, H = 2, 96, 64, 128, 32
    rng = np.random.default_rng(75)
    w13, s13, w2, s2 = _experts(rng, E2M1, E, Np, inter, K, H)
    oracle.moe_copies(E2M1, E, Np, inter, K, H, w13, s13, w2, s2)   # clean: fine
    s13b = s13.copy()
    s13b[:, inter:Np] = 200                       # codes of padding rows are not checked
    oracle.moe_copies(E2M1, E, Np, inter, K, H, w13, s13b, w2, s2)
    for region in range(3):
        a, b = w13.copy(), w2.copy()
        if region == 0:
            a[1, inter + 3, 5] = 0x10             # gate padding row
        elif region == 1:
            a[0, Np + inter, 0] = 0x01            # up padding row
        else:
            b[1, 7, inter // 2] = 0x80            # w2 padding column (a -0 nibble)
        with pytest.raises(ValueError):
            oracle.moe_copies(E2M1, E, Np, inter, K, H, a, s13, b, s2)
    with pytest.raises(ValueError):
        oracle.moe_copies(E2M1, E, Np, 48, K, H, w13, s13, w2, s2)  # inter % 32 != 0


# ------------------------------------------------------------------ up-gate product

@pytest.mark.parametrize("elem", [E2M1, E4M3])
def test_moe_gate_up_equals_silu_of_gate_times_up(elem):
    E, inter, K, T, topk = 4, 32, 160, 5, 2
    rng = np.random.default_rng([76, elem])
    rowb = K // 2 if elem == E2M1 else K
    w13 = wl.fp4_bytes(rng, (E, 2 * inter, rowb)) if elem == E2M1 else \
        wl.e4m3_bytes(rng, (E, 2 * inter, K))
    codes = wl.codes(rng, (E * 2 * inter, K // 32), 122, 130)
    x = wl.activations(rng, (T, K))
    ids, _ = wl.routing(rng, T, E, topk)
    ids[1, 0] = -1                                # out of range: zero row
    h = oracle.moe_gate_up(elem, E, inter, K, w13, codes, x, ids)
    c3 = codes.reshape(E, 2 * inter, K // 32)
    gate = oracle.moe_linear(elem, E, inter, K, w13[:, 0::2], c3[:, 0::2].reshape(-1), x, ids)
    up = oracle.moe_linear(elem, E, inter, K, w13[:, 1::2], c3[:, 1::2].reshape(-1), x, ids)
    silu = np.vectorize(oracle.silu)
    np.testing.assert_array_equal(h, silu(gate) * up)
    assert not h[1, 0].any()


def test_moe_gate_up_zero_gate_gives_zero():
    E, inter, K, T, topk = 2, 32, 128, 3, 2
    rng = np.random.default_rng(77)
    w13 = wl.fp4_bytes(rng, (E, 2 * inter, K // 2))
    w13[:, 0::2] = 0                              # every gate row zero: silu(0) = 0
    codes = wl.codes(rng, (E * 2 * inter, K // 32), 122, 130)
    x = wl.activations(rng, (T, K))
    ids, _ = wl.routing(rng, T, E, topk)
    assert not oracle.moe_gate_up(E2M1, E, inter, K, w13, codes, x, ids).any()


# ------------------------------------------------------------------ per-slot rows

def test_moe_linear_rows_against_pinned_linears():
    E, N, K, T, topk = 5, 48, 192, 4, 3
    rng = np.random.default_rng(78)
    w = wl.fp4_bytes(rng, (E, N, K // 2))
    codes = wl.codes(rng, (E * N, K // 32), 122, 130)
    x = wl.activations(rng, (T, K))
    ids, wts = wl.routing(rng, T, E, topk)
    ids[2, 1] = E                                 # out of range
    # every slot carrying its token's row: the grouped linear of the oracle
    rows = np.repeat(x, topk, axis=0)
    np.testing.assert_array_equal(oracle.moe_linear_rows(E2M1, E, N, K, w, codes, rows, ids),
                                  oracle.moe_linear(E2M1, E, N, K, w, codes, x, ids))
    np.testing.assert_array_equal(
        oracle.moe_linear_rows(E2M1, E, N, K, w, codes, rows, ids, wts),
        oracle.moe_linear(E2M1, E, N, K, w, codes, x, ids, wts))
    # distinct rows per slot: slot by slot, the dense linear of its expert
    a = wl.activations(rng, (T * topk, K))
    y = oracle.moe_linear_rows(E2M1, E, N, K, w, codes, a, ids)
    c3 = codes.reshape(E, N, K // 32)
    for t in range(T):
        for k in range(topk):
            e = ids[t, k]
            if not 0 <= e < E:
                assert not y[t, k].any()
                continue
            ref = oracle.linear(E2M1, ROW32, N, K, w[e], c3[e].reshape(-1), 1, 0,
                                x=a[t * topk + k:t * topk + k + 1])
            np.testing.assert_array_equal(y[t, k], ref[0])
    # combined: the weighted sum over slots, k ascending
    yc = oracle.moe_linear_rows(E2M1, E, N, K, w, codes, a, ids, wts)
    for t in range(T):
        acc = np.zeros(N)
        for k in range(topk):
            acc = acc + np.float64(wts[t, k]) * y[t, k]
        np.testing.assert_array_equal(yc[t], acc)
