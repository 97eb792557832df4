"""Properties of the HIP path that hold at any size (through the C ABI).

- Token permutation: permuting the rows of x permutes the rows of y, bit
  for bit (each token's output depends only on that token), on the decode
  GEMVs, the prefill GEMM and the grouped MoE.
- Output-row permutation: permuting the weight rows (with their codes; whole
  32-row groups for 32x32 block codes) permutes the columns of y, bit for
  bit.
- K-block permutation: permuting the 32-value K blocks of x, W and the codes
  together leaves the exact result unchanged, so y meets the bar against the
  oracle of the unpermuted problem.
- Exact products: a one-hot x reads out one scaled weight per output, and a
  permutation-matrix W (one 1.0 per row, code 127) reads out one activation
  per output (the bf16 value, or its MXFP8 quantization); both are single
  nonzero products that bf16 holds exactly, so y equals them bit for bit.
- Scale shift: x * 2^k quantizes to the same e4m3 bytes with every code
  raised by k (the OCP MX rule and the pages' ceil rule both take the code
  from the block maximum's exponent), and the W8A8 product then equals
  y * 2^k bit for bit (powers of two commute with the fp32 sums and the
  bf16 rounding).
"""
import numpy as np
import pytest

import oracle
from microscaling_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu

E4M3, E2M1, ROW32, BLK32 = 0, 1, 0, 1
BF16, MXFP8, OCP, CEIL = 0, 1, 0, 1
COMBOS = [(E4M3, ROW32, BF16), (E4M3, BLK32, BF16), (E4M3, ROW32, MXFP8),
          (E4M3, BLK32, MXFP8), (E2M1, ROW32, BF16)]


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxgpu
    return mxgpu


def _inputs(seed, elem, layout, M, N, K):
    rng = np.random.default_rng(seed)
    w = wl.e4m3_bytes(rng, (N, K)) if elem == E4M3 else wl.fp4_bytes(rng, (N, K // 2))
    codes = wl.codes(rng, (N, K // 32) if layout == ROW32 else (N // 32, K // 32), 112, 140)
    x = wl.activations(rng, (M, K), 0.01)
    return rng, w, codes, x


def _rules(act):
    return (OCP, CEIL) if act == MXFP8 else (OCP,)


# (M, N, K): one token tile, a ragged K tail, three token tiles (the decode
# GEMV), and M = 200 (the prefill GEMM for MXFP8 activations)
PERM_SHAPES = [(16, 256, 1024), (13, 128, 1568), (40, 64, 512), (200, 256, 512)]


@pytest.mark.parametrize("elem,layout,act", COMBOS)
@pytest.mark.parametrize("M,N,K", PERM_SHAPES)
def test_token_permutation(g, elem, layout, act, M, N, K):
    rng, w, codes, x = _inputs([90, elem, layout, act, M, N, K], elem, layout, M, N, K)
    wp, cp = g.pack(elem, layout, 1, N, K, w, codes)
    perm = rng.permutation(M)
    for rule in _rules(act):
        y = g.linear(elem, layout, N, K, wp, cp, act, x=x, rule=rule)
        yp = g.linear(elem, layout, N, K, wp, cp, act, x=np.ascontiguousarray(x[perm]), rule=rule)
        assert np.array_equal(yp, y[perm]), f"token permutation, rule {rule}"


@pytest.mark.parametrize("elem,layout,act", COMBOS)
@pytest.mark.parametrize("M,N,K", PERM_SHAPES)
def test_output_row_permutation(g, elem, layout, act, M, N, K):
    rng, w, codes, x = _inputs([91, elem, layout, act, M, N, K], elem, layout, M, N, K)
    if layout == BLK32:
        # whole 32-row groups move with their block codes
        gp = rng.permutation(N // 32)
        perm = (gp[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
        codes_p = codes[gp]
    else:
        perm = rng.permutation(N)
        codes_p = codes[perm]
    wp, cp = g.pack(elem, layout, 1, N, K, w, codes)
    wq, cq = g.pack(elem, layout, 1, N, K, np.ascontiguousarray(w[perm]),
                    np.ascontiguousarray(codes_p))
    for rule in _rules(act):
        y = g.linear(elem, layout, N, K, wp, cp, act, x=x, rule=rule)
        yp = g.linear(elem, layout, N, K, wq, cq, act, x=x, rule=rule)
        assert np.array_equal(yp, y[:, perm]), f"output-row permutation, rule {rule}"


@pytest.mark.parametrize("elem,layout,act", COMBOS)
@pytest.mark.parametrize("M,N,K", [(16, 128, 1024), (5, 64, 1568), (100, 128, 512)])
def test_k_block_permutation(g, elem, layout, act, M, N, K):
    rng, w, codes, x = _inputs([92, elem, layout, act, M, N, K], elem, layout, M, N, K)
    kb = K // 32
    bp = rng.permutation(kb)
    cols = (bp[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    xp = np.ascontiguousarray(x[:, cols])
    if elem == E4M3:
        wperm = np.ascontiguousarray(w[:, cols])
    else:
        # two e2m1 values a byte: a 32-value block is 16 whole bytes
        bcols = (bp[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
        wperm = np.ascontiguousarray(w[:, bcols])
    cperm = np.ascontiguousarray(codes[:, bp])
    wq, cq = g.pack(elem, layout, 1, N, K, wperm, cperm)
    for rule in _rules(act):
        if act == MXFP8:
            oq, oc = oracle.quant_act(x, rule)
            ref = oracle.linear(elem, layout, N, K, w, codes, M, act, xq=oq, xcodes=oc)
        else:
            ref = oracle.linear(elem, layout, N, K, w, codes, M, act, x=x)
        yp = g.linear(elem, layout, N, K, wq, cq, act, x=xp, rule=rule)
        g.assert_close(yp, ref, f"K-block permutation, rule {rule}")


@pytest.mark.parametrize("elem,layout,act", COMBOS)
@pytest.mark.parametrize("M,N,K", [(16, 256, 1024), (9, 64, 1568), (80, 128, 512)])
def test_one_hot_activations_exact(g, elem, layout, act, M, N, K):
    rng, w, codes, _ = _inputs([93, elem, layout, act, M, N, K], elem, layout, M, N, K)
    ks = rng.integers(0, K, size=M)
    signs = np.where(rng.random(M) < 0.5, -1.0, 1.0)
    xf = np.zeros((M, K))
    xf[np.arange(M), ks] = signs
    x = wl.f32_to_bf16_bits(xf.astype(np.float32))
    wp, cp = g.pack(elem, layout, 1, N, K, w, codes)
    # y[m, n] = sign_m * Wf[n, k_m]: one scaled weight, exact in bf16; a zero
    # product leaves the sum at +0 (the sums start from +0)
    want = np.array([[signs[m] * oracle.weight(elem, layout, 1, N, K, w, codes, 0, n, ks[m])
                      for n in range(N)] for m in range(M)]) + 0.0
    for rule in _rules(act):
        y = g.linear(elem, layout, N, K, wp, cp, act, x=x, rule=rule)
        assert np.array_equal(y, oracle.bf16_round_array(want)), f"one-hot, rule {rule}"
        assert np.array_equal(g.bf16_to_f64(y), want), "one-hot value not exact in bf16"


@pytest.mark.parametrize("elem,layout,act", COMBOS)
@pytest.mark.parametrize("M,N,K", [(16, 256, 1024), (7, 64, 1568), (90, 128, 512)])
def test_permutation_matrix_weights_exact(g, elem, layout, act, M, N, K):
    rng = np.random.default_rng([94, elem, layout, act, M, N, K])
    pi = rng.choice(K, size=N, replace=False)            # y[:, n] reads x[:, pi[n]]
    if elem == E4M3:
        w = np.zeros((N, K), np.uint8)
        w[np.arange(N), pi] = 0x38                       # e4m3 1.0
    else:
        nib = np.zeros((N, K), np.uint8)
        nib[np.arange(N), pi] = 0x2                      # e2m1 1.0
        w = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    codes = np.full((N, K // 32) if layout == ROW32 else (N // 32, K // 32), 127, np.uint8)
    x = wl.activations(rng, (M, K), 0.01)
    wp, cp = g.pack(elem, layout, 1, N, K, w, codes)
    for rule in _rules(act):
        y = g.linear(elem, layout, N, K, wp, cp, act, x=x, rule=rule)
        if act == BF16:
            assert np.array_equal(y, x[:, pi]), "bf16 activations read out"
        else:
            oq, oc = oracle.quant_act(x, rule)
            deq = np.array([[oracle.e4m3_value(int(oq[m, k])) *
                             oracle.e8m0_value(int(oc[m, k // 32])) for k in pi]
                            for m in range(M)]) + 0.0
            assert np.array_equal(y, oracle.bf16_round_array(deq)), f"MXFP8 read out, rule {rule}"
            assert np.array_equal(g.bf16_to_f64(y), deq), "MXFP8 value not exact in bf16"


def _shift_bf16(x_bits: np.ndarray, k: int) -> np.ndarray:
    """x * 2^k for bf16 bits whose values stay normal (exact)."""
    v = wl.bf16_bits_to_f32(x_bits).astype(np.float64) * 2.0 ** k
    out = wl.f32_to_bf16_bits(v.astype(np.float32))
    assert np.array_equal(wl.bf16_bits_to_f32(out).astype(np.float64), v)
    return out


@pytest.mark.parametrize("k", [-40, -3, 5, 30])
@pytest.mark.parametrize("rule", [OCP, CEIL])
def test_quant_scale_shift(g, k, rule):
    rng = np.random.default_rng([95, k + 64, rule])
    M, K = 24, 1568
    x = wl.activations(rng, (M, K), 0.01)
    xs = _shift_bf16(x, k)
    q, c = g.quant(x, rule)
    qs, cs = g.quant(xs, rule)
    assert np.array_equal(qs, q), "bytes change under a power-of-two shift"
    assert np.array_equal(cs.astype(int), c.astype(int) + k), "codes do not shift by k"
    tq, tc = g.quant_t16(x, rule)
    tqs, tcs = g.quant_t16(xs, rule)
    d, cc = g.t16_unpack(tq.cpu().numpy(), tc.cpu().numpy(), M, K)
    ds, ccs = g.t16_unpack(tqs.cpu().numpy(), tcs.cpu().numpy(), M, K)
    assert np.array_equal(ds, d)
    live = (np.arange(cc.shape[0])[:, None] < M) & (np.arange(cc.shape[1])[None, :] < K // 32)
    assert np.array_equal(ccs.astype(int)[live], cc.astype(int)[live] + k)


@pytest.mark.parametrize("layout", [ROW32, BLK32])
@pytest.mark.parametrize("M,N,K", [(16, 7168, 7168), (3, 256, 1568), (130, 256, 1024)])
@pytest.mark.parametrize("k", [-9, 6])
def test_w8a8_product_scale_shift(g, layout, M, N, K, k):
    rng, w, codes, x = _inputs([96, layout, M, N, K, k + 64], E4M3, layout, M, N, K)
    wp, cp = g.pack(E4M3, layout, 1, N, K, w, codes)
    xs = _shift_bf16(x, k)
    for rule in (OCP, CEIL):
        y = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=x, rule=rule)
        ys = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=xs, rule=rule)
        want = wl.f32_to_bf16_bits((g.bf16_to_f64(y) * 2.0 ** k).astype(np.float32))
        assert np.array_equal(ys, want), f"W8A8 product under a 2^{k} shift, rule {rule}"


@pytest.mark.parametrize("elem,E,N,K,T,topk", [(E2M1, 32, 3072, 3072, 16, 8),
                                               (E2M1, 8, 128, 1024, 11, 3),
                                               (E4M3, 6, 64, 1568, 16, 4)])
def test_moe_token_permutation(g, elem, E, N, K, T, topk):
    rng = np.random.default_rng([97, elem, E, N, K, T, topk])
    w = wl.fp4_bytes(rng, (E, N, K // 2)) if elem == E2M1 else wl.e4m3_bytes(rng, (E, N, K))
    codes = wl.codes(rng, (E * N, K // 32), 120, 132)
    x = wl.activations(rng, (T, K))
    ids, wts = wl.routing(rng, T, E, topk)
    wp, cp = g.pack(elem, ROW32, E, N, K, w, codes)
    perm = rng.permutation(T)
    xp, idp, wtp = (np.ascontiguousarray(a[perm]) for a in (x, ids, wts))
    y = g.moe(elem, E, N, K, wp, cp, x, ids)
    yp = g.moe(elem, E, N, K, wp, cp, xp, idp)
    assert np.array_equal(yp.reshape(T, topk, N), y.reshape(T, topk, N)[perm]), "per slot"
    yc = g.moe(elem, E, N, K, wp, cp, x, ids, wts)
    ycp = g.moe(elem, E, N, K, wp, cp, xp, idp, wtp)
    assert np.array_equal(ycp.reshape(T, N), yc.reshape(T, N)[perm]), "combined"
