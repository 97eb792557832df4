"""Batch invariance of mx_linear through the C ABI.

The decode GEMVs sum each output in an order fixed by K alone, so a token
row's result must be bit-identical whatever the number of rows in the call:
for every A16 call and W8A8 up to 64 rows by default, and for W8A8 at any
number of rows in the batch-invariant mode ([rocm_native]
process_weights_after_loading: the page's GEMM, whose split of K varies with
M, is left under VLLM_BATCH_INVARIANT).  Outputs are also held to the oracle."""
import numpy as np
import pytest

import oracle
from microscaling_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu

E4M3, ROW32, BLK32 = 0, 0, 1
BF16, MXFP8 = 0, 1
MS = (1, 5, 16, 17, 64, 65, 130)


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxgpu
    return mxgpu


@pytest.fixture
def invariant():
    import microscaling_quantized_linear_amd as mx
    prev = mx.mx_set_batch_invariant(True)
    yield
    mx.mx_set_batch_invariant(prev)


def _setup(g, layout, N, K, seed):
    rng = np.random.default_rng([101, layout, N, K, seed])
    w = wl.e4m3_bytes(rng, (N, K))
    codes = wl.codes(rng, (N // 32 if layout == BLK32 else N, K // 32), 118, 132)
    x = wl.activations(rng, (200, K))
    wp, cp = g.pack(E4M3, layout, 1, N, K, w, codes)
    return w, codes, x, wp, cp


def _check_oracle(g, layout, N, K, w, codes, x, y, act):
    rng = np.random.default_rng(7)
    ms = rng.integers(0, x.shape[0], 256)
    ns = rng.integers(0, N, 256)
    if act == MXFP8:
        xq, xc = oracle.quant_act(x, oracle.RULE_OCP)
        ref = oracle.linear_pairs(E4M3, layout, N, K, w, codes.reshape(-1), MXFP8, ms, ns,
                                  xq=xq, xcodes=xc)
    else:
        ref = oracle.linear_pairs(E4M3, layout, N, K, w, codes.reshape(-1), BF16, ms, ns, x=x)
    g.assert_close(y[ms, ns], ref, "rows")


@pytest.mark.parametrize("layout,N,K", [(BLK32, 512, 1024), (ROW32, 256, 1568),
                                        (BLK32, 384, 896)])
def test_w8a8_rows_independent_of_m_in_invariant_mode(g, invariant, layout, N, K):
    w, codes, x, wp, cp = _setup(g, layout, N, K, 0)
    full = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=x)
    _check_oracle(g, layout, N, K, w, codes, x, full, MXFP8)
    for M in MS:
        np.testing.assert_array_equal(g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=x[:M]),
                                      full[:M], err_msg=f"M={M}")
    # pre-quantized row-major input takes the same GEMV
    xq, xc = oracle.quant_act(x, oracle.RULE_OCP)
    for M in (200, 65):
        np.testing.assert_array_equal(
            g.linear(E4M3, layout, N, K, wp, cp, MXFP8, xq=xq[:M], xcodes=xc[:M]), full[:M])


@pytest.mark.parametrize("layout,N,K", [(BLK32, 512, 1024), (ROW32, 256, 1568)])
def test_decode_rows_independent_of_m_by_default(g, layout, N, K):
    import microscaling_quantized_linear_amd as mx
    prev = mx.mx_set_batch_invariant(False)
    try:
        w, codes, x, wp, cp = _setup(g, layout, N, K, 1)
        y64 = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=x[:64])
        for M in (1, 5, 16, 17, 40):
            np.testing.assert_array_equal(g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=x[:M]),
                                          y64[:M], err_msg=f"W8A8 M={M}")
        a200 = g.linear(E4M3, layout, N, K, wp, cp, BF16, x=x)
        _check_oracle(g, layout, N, K, w, codes, x, a200, BF16)
        for M in MS:
            np.testing.assert_array_equal(g.linear(E4M3, layout, N, K, wp, cp, BF16, x=x[:M]),
                                          a200[:M], err_msg=f"A16 M={M}")
        # above 64 rows W8A8 runs the GEMM: held to the oracle, not to the GEMV's bits
        y200 = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=x)
        _check_oracle(g, layout, N, K, w, codes, x, y200, MXFP8)
    finally:
        mx.mx_set_batch_invariant(prev)
