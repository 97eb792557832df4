"""Pins of the oracle's per-token MXFP8 activation quantization (CPU only).

Scale rules (oracle readings R1/R2):
  ocp      code = clamp(floor(log2 amax) - 8 + 127, 0, 254), saturating elements
  ceil448  code = clamp(ceil(log2(max(amax, 2^-126) / 448)) + 127, 0, 254), the
           rule of vllm.model_executor.kernels.linear.mxfp8.rocm_native,
           _quant_mxfp8_tile.
The code rules are checked exhaustively over every positive finite bf16 amax
against numpy's log2; the element bytes against torch's independent
float32 -> float8_e4m3fn cast and a brute-force nearest-value search; and the
round trip of exact e4m3 x 2^(code-127) blocks (the exactness statement of
vllm.models.deepseek_v41.amd.mono.weights942, ocp_from_dequant).
"""
import math

import numpy as np
import torch

import oracle
from microscaling_quantized_linear_amd import workloads as wl

OCP, CEIL = oracle.RULE_OCP, oracle.RULE_CEIL448


def _all_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)  # +min subnormal .. +max finite
    return bits, wl.bf16_bits_to_f32(bits).astype(np.float64)


def test_code_rules_exhaustive_over_bf16():
    bits, vals = _all_positive_bf16()
    assert len(vals) == 32639
    ocp_ref = np.clip(np.floor(np.log2(vals)) - 8 + 127, 0, 254)
    tiny = 2.0 ** -126
    ceil_ref = np.clip(np.ceil(np.log2(np.maximum(vals, tiny) / 448.0)) + 127, 0, 254)
    # the page evaluates its rule in float32; on bf16 inputs that agrees too
    v32 = np.maximum(vals.astype(np.float32), np.float32(tiny))
    ceil32 = np.clip(np.ceil(np.log2(v32 / np.float32(448.0))) + 127, 0, 254)
    for v, a, b, c in zip(vals.tolist(), ocp_ref.tolist(), ceil_ref.tolist(), ceil32.tolist()):
        assert oracle.act_code(v, OCP) == a, v
        assert oracle.act_code(v, CEIL) == b == c, v
    assert oracle.act_code(0.0, OCP) == 0
    assert oracle.act_code(0.0, CEIL) == 0


def test_rules_differ_exactly_when_mantissa_above_1_75():
    # floor(log2 a) - 8 vs ceil(log2(a/448)): they differ by one iff a/2^E > 1.75
    _, vals = _all_positive_bf16()
    for v in vals[::7].tolist():
        e = math.floor(math.log2(v))
        mu = v / 2.0 ** e
        o, c = oracle.act_code(v, OCP), oracle.act_code(v, CEIL)
        if 0 < o < 254 and 0 < c < 254:
            assert c - o == (1 if mu > 1.75 else 0), v


def _torch_quant(x_bits, rule):
    """Independent float32 implementation of the per-block steps with torch's
    e4m3 cast: codes from numpy log2, elements cast by torch (saturated first
    under the ocp rule)."""
    x = torch.from_numpy(wl.bf16_bits_to_f32(x_bits).copy())
    M, K = x.shape
    xb = x.view(M, K // 32, 32)
    amax = xb.abs().amax(dim=2).double().numpy()
    if rule == OCP:
        with np.errstate(divide="ignore"):
            code = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1))) - 8 + 127, 0)
    else:
        code = np.ceil(np.log2(np.maximum(amax, 2.0 ** -126) / 448.0)) + 127
    code = np.clip(code, 0, 254)
    mul = torch.from_numpy(np.exp2(127.0 - code)).float()
    v = xb * mul[:, :, None]
    if rule == OCP:
        v = v.clamp(-448.0, 448.0)
    q = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(M, K).numpy()
    return q, code.astype(np.uint8)


def test_quant_matches_torch_cast_both_rules():
    g = wl.rng(99, 0)
    x = wl.activations(g, (24, 1024), outliers=0.01)
    # add blocks that exercise zero, -0, tiny and huge magnitudes
    x[0, :32] = 0
    x[0, 32:64] = 0x8000
    x[1, :32] = wl.f32_to_bf16_bits(np.full(32, 1e-39, np.float32))
    x[2, :32] = wl.f32_to_bf16_bits(np.linspace(-3e38, 3e38, 32).astype(np.float32))
    for rule in (OCP, CEIL):
        xq, codes = oracle.quant_act(x, rule)
        rq, rc = _torch_quant(x, rule)
        np.testing.assert_array_equal(codes, rc)
        np.testing.assert_array_equal(xq, rq)


def test_quant_elements_brute_force():
    table = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    g = wl.rng(99, 1)
    x = wl.activations(g, (4, 256), outliers=0.05)
    for rule in (OCP, CEIL):
        xq, codes = oracle.quant_act(x, rule)
        xv = wl.bf16_bits_to_f32(x).astype(np.float64)
        for m in range(4):
            for k in range(256):
                v = xv[m, k] * 2.0 ** (127 - int(codes[m, k // 32]))
                a = abs(v)
                if a >= 448:
                    want = 0x7E
                else:
                    d = np.abs(table - a)
                    best = np.flatnonzero(d == d.min())
                    want = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
                want |= 0x80 if math.copysign(1.0, v) < 0 else 0
                assert xq[m, k] == want, (rule, m, k)


def test_round_trip_of_exact_blocks():
    # a block dec(b) * 2^(c-127) whose largest byte is 0x7E (448) makes both
    # rules pick exactly c, and quantizes back to the bytes b.
    g = np.random.default_rng(5)
    M, nb = 16, 8
    b = wl.e4m3_bytes(g, (M, nb * 32))
    b[:, ::32] = np.where(g.random((M, nb)) < 0.5, 0x7E, 0xFE)
    c = g.integers(100, 150, size=(M, nb))
    val = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    xv = val[b] * np.exp2(np.repeat(c, 32, axis=1) - 127.0)
    x = wl.f32_to_bf16_bits(xv.astype(np.float32))
    assert np.array_equal(wl.bf16_bits_to_f32(x).astype(np.float64), xv)  # exact in bf16
    for rule in (OCP, CEIL):
        xq, codes = oracle.quant_act(x, rule)
        np.testing.assert_array_equal(codes, c)
        np.testing.assert_array_equal(xq, b)


def test_scale_shift_invariance():
    g = wl.rng(99, 2)
    x = wl.activations(g, (8, 512))
    xv = wl.bf16_bits_to_f32(x)
    for t in (-20, -3, 1, 7, 30):
        xs = wl.f32_to_bf16_bits(xv * np.float32(2.0 ** t))
        for rule in (OCP, CEIL):
            q0, c0 = oracle.quant_act(x, rule)
            q1, c1 = oracle.quant_act(xs, rule)
            np.testing.assert_array_equal(q1, q0)
            np.testing.assert_array_equal(c1.astype(int), c0.astype(int) + t)


def test_ocp_rule_puts_block_max_in_256_512_then_saturates():
    g = wl.rng(99, 3)
    x = wl.activations(g, (8, 1024), outliers=0.02)
    xq, codes = oracle.quant_act(x, OCP)
    xv = wl.bf16_bits_to_f32(x).astype(np.float64).reshape(8, 32, 32)
    amax = np.abs(xv).max(axis=2)
    scaled = amax * np.exp2(127.0 - codes)
    assert np.all((scaled >= 256) & (scaled < 512))
    qv = torch.from_numpy(xq).view(torch.float8_e4m3fn).double().numpy().reshape(8, 32, 32)
    assert np.all(np.abs(qv).max(axis=2) <= 448)
    # the ceil448 rule never needs saturation: scaled max in (224, 448]
    xq2, codes2 = oracle.quant_act(x, CEIL)
    scaled2 = amax * np.exp2(127.0 - codes2)
    assert np.all((scaled2 > 224) & (scaled2 <= 448))


def test_zero_and_negative_zero_blocks():
    x = np.zeros((2, 64), np.uint16)
    x[1, :] = 0x8000
    for rule in (OCP, CEIL):
        xq, codes = oracle.quant_act(x, rule)
        assert np.all(codes == 0)
        assert np.all(xq[0] == 0x00) and np.all(xq[1] == 0x80)
