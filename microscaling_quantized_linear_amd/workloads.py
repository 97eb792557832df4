"""Seeded synthetic workloads for the MX linear layer.

This module only draws random inputs; it holds none of the layer's arithmetic
and imports neither the HIP library nor the oracle.  Tests, the benchmark and
the smoke check all take their inputs from here, so the oracle and the GPU see
identical bytes.

Every tensor comes from numpy's PCG64 seeded with ``[seed, wid,
tensor_id]`` (wid: the workload's id below).  Distributions:

* e4m3 weight bytes: uniform over the 254 non-NaN codes (0x7F and 0xFF left out).
* e2m1 weight bytes: uniform bytes, i.e. uniform nibbles, -0 (0x8) included.
* E8M0 codes: uniform integers in an inclusive range.
* activations: N(0, 1) in float32, then rounded to bfloat16 (nearest-even);
  optionally a Bernoulli(p) mask of entries multiplied by 50 before rounding.
* MoE routing: N(0, 1) logits [T, E]; each token takes its top-k experts
  (so k distinct experts, uniformly at random) and softmax weights over the
  k selected logits.
"""
from __future__ import annotations

import numpy as np

# tensor ids inside one workload's seed stream
T_WEIGHT, T_CODES, T_X, T_OUTLIER, T_ROUTE, T_BIAS = range(6)

E4M3, E2M1 = 0, 1
ROW32, BLK32 = 0, 1
RULE_OCP, RULE_CEIL448 = 0, 1
ACT_BF16, ACT_MXFP8 = 0, 1

# The five workloads, by id.  "name" is what the benchmark prints as config.workload.
WORKLOADS = {
    1: dict(name="mxfp8_a16w8_gemv_M1_N256_K512_row32", kind="linear", elem=E4M3,
            layout=ROW32, act=ACT_BF16, Ms=(1,), N=256, K=512, codes=(120, 134),
            outliers=0.0),
    2: dict(name="mxfp8_w8a8_gemv_M16_N7168_K7168_blk32", kind="linear", elem=E4M3,
            layout=BLK32, act=ACT_MXFP8, rule=RULE_OCP, Ms=(1, 4, 16), N=7168,
            K=7168, codes=(118, 132), outliers=0.01),
    3: dict(name="mxfp8_a16w8_gemv_M8_N4096_K1568_row32", kind="linear", elem=E4M3,
            layout=ROW32, act=ACT_BF16, Ms=(8,), N=4096, K=1568, codes=(120, 134),
            outliers=0.0),
    4: dict(name="mxfp4_a16w4_moe_E32_N3072_K3072_T16_top8", kind="moe", elem=E2M1,
            layout=ROW32, act=ACT_BF16, E=32, N=3072, K=3072, T=16, topk=8,
            codes=(122, 130), outliers=0.0),
    5: dict(name="mxfp8_w8a8_gemm_M4096_N7168_K7168_blk32", kind="linear", elem=E4M3,
            layout=BLK32, act=ACT_MXFP8, rule=RULE_OCP, Ms=(4096,), N=7168, K=7168,
            codes=(118, 132), outliers=0.0),
}


def rng(wid: int, tensor_id: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, wid, tensor_id])


def e4m3_bytes(g: np.random.Generator, shape) -> np.ndarray:
    """Uniform over the 254 finite e4m3 codes."""
    v = g.integers(0, 254, size=shape, dtype=np.int32)
    return (v + (v >= 0x7F)).astype(np.uint8)


def fp4_bytes(g: np.random.Generator, shape) -> np.ndarray:
    """Uniform packed e2m1 bytes (two nibbles each, -0 included)."""
    return g.integers(0, 256, size=shape, dtype=np.int32).astype(np.uint8)


def codes(g: np.random.Generator, shape, lo: int, hi: int) -> np.ndarray:
    """Uniform E8M0 codes in [lo, hi]."""
    return g.integers(lo, hi + 1, size=shape, dtype=np.int32).astype(np.uint8)


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(g: np.random.Generator, shape, outliers: float = 0.0,
                g_mask: np.random.Generator | None = None) -> np.ndarray:
    """bf16 bits of N(0,1) samples; a Bernoulli(outliers) subset scaled by 50."""
    f = g.standard_normal(size=shape, dtype=np.float32)
    if outliers > 0.0:
        mask = (g_mask if g_mask is not None else g).random(size=shape) < outliers
        f = np.where(mask, f * np.float32(50.0), f).astype(np.float32)
    return f32_to_bf16_bits(f)


def routing(g: np.random.Generator, T: int, E: int, topk: int):
    """(ids int32 [T, topk], weights float32 [T, topk]) from N(0,1) logits."""
    logits = g.standard_normal(size=(T, E), dtype=np.float32)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :topk].astype(np.int32)
    sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    w = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def linear_inputs(wid: int, M=None, N=None, K=None, seed: int = 0):
    """Inputs of a dense config (optionally at another shape, same recipe).

    Returns dict(w [N, K] uint8, codes ROW32 [N, K/32] or BLK32 [N/32, K/32],
    x bf16 bits [M, K]); M defaults to the largest M of the config.
    """
    c = WORKLOADS[wid]
    N = c["N"] if N is None else N
    K = c["K"] if K is None else K
    M = max(c["Ms"]) if M is None else M
    w = e4m3_bytes(rng(wid, T_WEIGHT, seed), (N, K))
    cshape = (N, K // 32) if c["layout"] == ROW32 else (N // 32, K // 32)
    cd = codes(rng(wid, T_CODES, seed), cshape, *c["codes"])
    x = activations(rng(wid, T_X, seed), (M, K), c["outliers"],
                    rng(wid, T_OUTLIER, seed))
    return dict(w=w, codes=cd, x=x, M=M, N=N, K=K, elem=c["elem"],
                layout=c["layout"], act=c["act"], rule=c.get("rule", RULE_OCP))


def moe_inputs(wid: int = 4, E=None, N=None, K=None, T=None, topk=None,
               seed: int = 0):
    """Inputs of the MoE config: w [E, N, K/2] e2m1, codes [E*N, K/32], x, ids, weights."""
    c = WORKLOADS[wid]
    E = c["E"] if E is None else E
    N = c["N"] if N is None else N
    K = c["K"] if K is None else K
    T = c["T"] if T is None else T
    topk = c["topk"] if topk is None else topk
    w = fp4_bytes(rng(wid, T_WEIGHT, seed), (E, N, K // 2))
    cd = codes(rng(wid, T_CODES, seed), (E * N, K // 32), *c["codes"])
    x = activations(rng(wid, T_X, seed), (T, K))
    ids, wts = routing(rng(wid, T_ROUTE, seed), T, E, topk)
    return dict(w=w, codes=cd, x=x, ids=ids, weights=wts, E=E, N=N, K=K, T=T,
                topk=topk, elem=E2M1, layout=ROW32)


def bias(wid: int, N: int, seed: int = 0) -> np.ndarray:
    return activations(rng(wid, T_BIAS, seed), (N,))
