"""Pins of the oracle's dense and MoE linear layers (CPU only).

Checked against: exact rational arithmetic (Python fractions) on small
inputs, with operands decoded by torch's independent float8 views; numpy's
float64 matmul of the dequantized matrices (a library routine); one-hot
activations and permutation-matrix weights, whose results are exact; and, for
the MoE, the dense oracle itself on the routed expert (E = 1, top-1 reduces to
the dense layer).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from microscaling_quantized_linear_amd import workloads as wl

E4M3, E2M1, ROW32, BLK32 = oracle.E4M3, oracle.E2M1, oracle.ROW32, oracle.BLK32
BF16, MXFP8 = oracle.ACT_BF16, oracle.ACT_MXFP8

_E4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
_E8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()


def _e2m1_table():
    vals = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                vals.append(float(line.split()[1]))
    return np.array(vals)


_E2 = _e2m1_table()


def dequant_weights(elem, layout, E, N, K, w, codes):
    """Independent dequantization: torch float8 views + the OCP e2m1 table."""
    if elem == E4M3:
        v = _E4[w.reshape(E, N, K)]
    else:
        b = w.reshape(E, N, K // 2)
        v = np.empty((E, N, K))
        v[..., 0::2] = _E2[b & 15]
        v[..., 1::2] = _E2[b >> 4]
    if layout == ROW32:
        s = _E8[codes.reshape(E, N, K // 32)]
    else:
        s = np.repeat(_E8[codes.reshape(E, N // 32, K // 32)], 32, axis=1)
    return v * np.repeat(s, 32, axis=2)


def _inputs(elem, layout, act, M, N, K, seed):
    g = np.random.default_rng(seed)
    if elem == E4M3:
        w = wl.e4m3_bytes(g, (N, K))
    else:
        w = wl.fp4_bytes(g, (N, K // 2))
    cshape = (N, K // 32) if layout == ROW32 else (N // 32, K // 32)
    codes = wl.codes(g, cshape, 110, 140)
    x = wl.activations(g, (M, K), 0.02)
    xq = xc = None
    if act == MXFP8:
        xq, xc = oracle.quant_act(x, oracle.RULE_OCP)
    return w, codes, x, xq, xc


def _act_values(act, x, xq, xc):
    if act == BF16:
        return wl.bf16_bits_to_f32(x).astype(np.float64)
    return _E4[xq] * np.repeat(_E8[xc], 32, axis=1)


CASES = [(E4M3, ROW32, BF16), (E4M3, BLK32, BF16), (E4M3, ROW32, MXFP8),
         (E4M3, BLK32, MXFP8), (E2M1, ROW32, BF16)]


@pytest.mark.parametrize("elem,layout,act", CASES)
def test_linear_vs_exact_rationals(elem, layout, act):
    M, N, K = 2, 32, 64
    w, codes, x, xq, xc = _inputs(elem, layout, act, M, N, K, 11)
    y = oracle.linear(elem, layout, N, K, w, codes, M, act, x=x, xq=xq, xcodes=xc)
    A = _act_values(act, x, xq, xc)
    W = dequant_weights(elem, layout, 1, N, K, w, codes)[0]
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(A[m, k])) * Fraction(float(W[n, k])) for k in range(K)]
            exact = sum(terms, Fraction(0))
            bound = K * 2.0 ** -53 * float(sum(abs(t) for t in terms))
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(bound), (m, n)


@pytest.mark.parametrize("elem,layout,act", CASES)
def test_linear_vs_numpy_matmul(elem, layout, act):
    M, N, K = 3, 64, 1568 if elem == E4M3 else 1536
    w, codes, x, xq, xc = _inputs(elem, layout, act, M, N, K, 12)
    bias = wl.activations(np.random.default_rng(4), (N,))
    y = oracle.linear(elem, layout, N, K, w, codes, M, act, x=x, xq=xq, xcodes=xc, bias=bias)
    A = _act_values(act, x, xq, xc)
    W = dequant_weights(elem, layout, 1, N, K, w, codes)[0]
    ref = A @ W.T + wl.bf16_bits_to_f32(bias).astype(np.float64)
    scale = np.abs(A) @ np.abs(W).T + 1.0
    assert np.all(np.abs(y - ref) <= 1e-13 * scale)


def test_one_hot_activation_gives_exact_weight_column():
    N, K = 64, 256
    w, codes, _, _, _ = _inputs(E4M3, ROW32, BF16, 1, N, K, 13)
    W = dequant_weights(E4M3, ROW32, 1, N, K, w, codes)[0]
    for k in (0, 31, 32, 255):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80                       # bf16 1.0
        y = oracle.linear(E4M3, ROW32, N, K, w, codes, 1, BF16, x=x)
        np.testing.assert_array_equal(y[0], W[:, k])


def test_permutation_weights_gather_activations():
    N = K = 64
    perm = np.random.default_rng(14).permutation(K)
    w = np.zeros((N, K), np.uint8)
    w[np.arange(N), perm] = 0x38                 # e4m3 1.0
    for layout in (ROW32, BLK32):
        cshape = (N, K // 32) if layout == ROW32 else (N // 32, K // 32)
        codes = np.full(cshape, 127, np.uint8)  # scale 1
        x = wl.activations(np.random.default_rng(15), (4, K))
        y = oracle.linear(E4M3, layout, N, K, w, codes, 4, BF16, x=x)
        np.testing.assert_array_equal(y, wl.bf16_bits_to_f32(x)[:, perm].astype(np.float64))


def test_negative_zero_weights_equal_positive_zero():
    N, K = 32, 1568
    w, codes, x, _, _ = _inputs(E4M3, ROW32, BF16, 2, N, K, 16)
    w0 = w.copy()
    w0[:, ::3] = 0x00
    w1 = w.copy()
    w1[:, ::3] = 0x80
    y0 = oracle.linear(E4M3, ROW32, N, K, w0, codes, 2, BF16, x=x)
    y1 = oracle.linear(E4M3, ROW32, N, K, w1, codes, 2, BF16, x=x)
    np.testing.assert_array_equal(y0, y1)


def test_pairs_equal_full_linear():
    M, N, K = 4, 64, 512
    w, codes, x, xq, xc = _inputs(E4M3, BLK32, MXFP8, M, N, K, 17)
    y = oracle.linear(E4M3, BLK32, N, K, w, codes, M, MXFP8, xq=xq, xcodes=xc)
    g = np.random.default_rng(5)
    ms, ns = g.integers(0, M, 50), g.integers(0, N, 50)
    yp = oracle.linear_pairs(E4M3, BLK32, N, K, w, codes, MXFP8, ms, ns, xq=xq, xcodes=xc)
    np.testing.assert_array_equal(yp, y[ms, ns])


def _moe(E=4, N=32, K=256, T=5, topk=2, seed=18):
    d = wl.moe_inputs(4, E=E, N=N, K=K, T=T, topk=topk, seed=seed)
    return d


def test_moe_single_expert_top1_equals_dense():
    d = _moe(E=1, topk=1)
    y = oracle.moe_linear(E2M1, 1, d["N"], d["K"], d["w"], d["codes"], d["x"], d["ids"])
    yd = oracle.linear(E2M1, ROW32, d["N"], d["K"], d["w"][0], d["codes"], d["T"], BF16, x=d["x"])
    np.testing.assert_array_equal(y[:, 0, :], yd)


def test_moe_slots_equal_dense_on_routed_expert_and_combine():
    d = _moe()
    E, N, K, T, topk = d["E"], d["N"], d["K"], d["T"], d["topk"]
    y = oracle.moe_linear(E2M1, E, N, K, d["w"], d["codes"], d["x"], d["ids"])
    codes = d["codes"].reshape(E, N, K // 32)
    for e in range(E):
        yd = oracle.linear(E2M1, ROW32, N, K, d["w"][e], codes[e], T, BF16, x=d["x"])
        for t in range(T):
            for k in range(topk):
                if d["ids"][t, k] == e:
                    np.testing.assert_array_equal(y[t, k], yd[t])
    yc = oracle.moe_linear(E2M1, E, N, K, d["w"], d["codes"], d["x"], d["ids"], d["weights"])
    ref = np.zeros((T, N))
    for k in range(topk):
        ref = ref + d["weights"][:, k:k + 1].astype(np.float64) * y[:, k, :]
    np.testing.assert_array_equal(yc, ref)


def test_moe_duplicate_and_out_of_range_ids():
    d = _moe()
    ids = d["ids"].copy()
    ids[0, :] = 2
    ids[1, 0] = -1
    ids[2, 1] = d["E"]
    y = oracle.moe_linear(E2M1, d["E"], d["N"], d["K"], d["w"], d["codes"], d["x"], ids)
    np.testing.assert_array_equal(y[0, 0], y[0, 1])
    assert np.all(y[1, 0] == 0) and np.all(y[2, 1] == 0)
