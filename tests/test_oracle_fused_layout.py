"""Pins of the oracle's attention-layout permutations (CPU only).

orc_q_fused_perm, orc_o_fused_perm ([fused_layout] q_fused_permutation,
o_fused_permutation) are checked against a numpy reshape/transpose statement
of the same layouts and against the page's construction (arange scattered at
the fused index); orc_fused_layout_permute ([fused_layout] permute_wq_b_,
permute_wo_a_) against the pinned oracle linear: permuted rows give the
output columns in the fused Q order, sum for sum, and permuted columns with
the activation in the fused O order give the standard product."""
import numpy as np
import pytest

import oracle
from microscaling_quantized_linear_amd import workloads as wl

E4M3, ROW32, BLK32, BF16 = 0, 0, 1, 0


@pytest.mark.parametrize("H,D", [(1, 16), (4, 32), (3, 64), (8, 128), (16, 192)])
def test_q_perm_layout(H, D):
    perm = oracle.q_fused_perm(H, D)
    std = np.arange(H * D)
    # [head, chunk, 16] -> [chunk, head, 16]
    want = std.reshape(H, D // 16, 16).transpose(1, 0, 2).reshape(-1)
    np.testing.assert_array_equal(perm, want)
    # the page's construction: arange scattered at each standard index's fused index
    h, d = np.meshgrid(np.arange(H), np.arange(D), indexing="ij")
    fused_index = (d // 16) * (H * 16) + h * 16 + d % 16
    built = np.empty(H * D, np.int64)
    built[fused_index.reshape(-1)] = np.arange(H * D)
    np.testing.assert_array_equal(perm, built)


@pytest.mark.parametrize("G,D", [(1, 32), (8, 64), (4, 128), (8, 512)])
def test_o_perm_layout(G, D):
    perm = oracle.o_fused_perm(G, D)
    want = np.arange(G * D).reshape(G, D // 32, 32).transpose(1, 0, 2).reshape(-1)
    np.testing.assert_array_equal(perm, want)
    h, c, j = np.meshgrid(np.arange(G), np.arange(D // 32), np.arange(32), indexing="ij")
    built = np.empty(G * D, np.int64)
    built[((c * G + h) * 32 + j).reshape(-1)] = np.arange(G * D)
    np.testing.assert_array_equal(perm, built)


def test_perm_shape_refusals():
    with pytest.raises(ValueError):
        oracle.q_fused_perm(4, 40)
    with pytest.raises(ValueError):
        oracle.o_fused_perm(8, 48)


@pytest.mark.parametrize("heads,D,K", [(4, 32, 96), (2, 64, 160), (8, 16, 64)])
def test_q_rows_give_the_fused_output_order(heads, D, K):
    rng = np.random.default_rng([111, heads, D, K])
    N = heads * D
    w = wl.e4m3_bytes(rng, (N, K))
    codes = wl.codes(rng, (N, K // 32), 118, 134)
    wq, cq = oracle.fused_layout_permute(0, ROW32, N, K, heads, w, codes)
    perm = oracle.q_fused_perm(heads, D)
    np.testing.assert_array_equal(wq, w[perm])
    np.testing.assert_array_equal(cq, codes[perm])
    x = wl.activations(rng, (3, K))
    y = oracle.linear(E4M3, ROW32, N, K, w, codes.reshape(-1), 3, BF16, x=x)
    yq = oracle.linear(E4M3, ROW32, N, K, wq, cq.reshape(-1), 3, BF16, x=x)
    np.testing.assert_array_equal(yq, y[:, perm])
    with pytest.raises(ValueError):
        oracle.fused_layout_permute(0, BLK32, N, K, heads, w, codes[: N // 32])


@pytest.mark.parametrize("layout,G,D,N", [(ROW32, 8, 64, 48), (BLK32, 4, 128, 64),
                                          (BLK32, 2, 32, 32)])
def test_o_cols_take_the_fused_activation(layout, G, D, N):
    rng = np.random.default_rng([112, layout, G, D, N])
    K = G * D
    w = wl.e4m3_bytes(rng, (N, K))
    codes = wl.codes(rng, (N // 32 if layout == BLK32 else N, K // 32), 118, 134)
    wo, co = oracle.fused_layout_permute(1, layout, N, K, G, w, codes)
    perm = oracle.o_fused_perm(G, D)
    np.testing.assert_array_equal(wo, w[:, perm])
    x = wl.activations(rng, (4, K))
    y = oracle.linear(E4M3, layout, N, K, w, codes.reshape(-1), 4, BF16, x=x)
    yo = oracle.linear(E4M3, layout, N, K, wo, co.reshape(-1), 4, BF16,
                       x=np.ascontiguousarray(x[:, perm]))
    # the same products summed in another order (binary64)
    np.testing.assert_allclose(yo, y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
    # dequantized weights move with their columns: every weight keeps its code
    for n in range(0, N, 7):
        for f in range(0, K, 13):
            assert oracle.weight(E4M3, layout, 1, N, K, wo, co.reshape(-1), 0, n, f) == \
                oracle.weight(E4M3, layout, 1, N, K, w, codes.reshape(-1), 0, n, perm[f])
