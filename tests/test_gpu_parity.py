"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Packs and quantized activations must match bit for bit; bf16 outputs must
meet the bar in tests/mxgpu.py (relative L2 <= 2e-3, every element within
1e-2 of its oracle row's largest magnitude).  Small cases span several tiles
and ragged K tails; the five workloads run at full size, checked on every
output and held to the plain relative-L2 bar."""
import numpy as np
import pytest

import oracle
from microscaling_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu

E4M3, E2M1, ROW32, BLK32 = 0, 1, 0, 1
BF16, MXFP8, MXFP8_T16, OCP, CEIL = 0, 1, 2, 0, 1


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxgpu
    return mxgpu


# ------------------------------------------------------------------ packs

PACK_SHAPES = [
    (E4M3, ROW32, 1, 32, 512), (E4M3, ROW32, 1, 48, 1568), (E4M3, BLK32, 1, 64, 1568),
    (E4M3, BLK32, 1, 96, 896), (E2M1, ROW32, 3, 32, 384), (E2M1, ROW32, 2, 16, 160),
    (E2M1, BLK32, 2, 32, 256), (E4M3, ROW32, 1, 16, 32),
]


@pytest.mark.parametrize("elem,layout,E,N,K", PACK_SHAPES)
def test_pack_bit_exact_small(g, elem, layout, E, N, K):
    rng = np.random.default_rng([21, elem, layout, E, N, K])
    kb = K if elem == E4M3 else K // 2
    w = rng.integers(0, 256, (E, N, kb), dtype=np.int32).astype(np.uint8)
    cshape = (E * N, K // 32) if layout == ROW32 else (E * N // 32, K // 32)
    codes = rng.integers(0, 255, cshape, dtype=np.int32).astype(np.uint8)
    wp, cp = g.pack(elem, layout, E, N, K, w, codes)
    owp, ocp = oracle.pack_weights(elem, layout, E, N, K, w, codes)
    np.testing.assert_array_equal(wp.cpu().numpy(), owp)
    np.testing.assert_array_equal(cp.cpu().numpy(), ocp)


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_pack_bit_exact_workloads(g, cid):
    d = wl.linear_inputs(cid, M=1)
    wp, cp = g.pack(d["elem"], d["layout"], 1, d["N"], d["K"], d["w"], d["codes"])
    owp, ocp = oracle.pack_weights(d["elem"], d["layout"], 1, d["N"], d["K"], d["w"], d["codes"])
    assert np.array_equal(wp.cpu().numpy(), owp)
    assert np.array_equal(cp.cpu().numpy(), ocp)


def test_pack_bit_exact_moe_workload(g):
    d = wl.moe_inputs(4)
    wp, cp = g.pack(E2M1, ROW32, d["E"], d["N"], d["K"], d["w"], d["codes"])
    owp, ocp = oracle.pack_weights(E2M1, ROW32, d["E"], d["N"], d["K"], d["w"], d["codes"])
    assert np.array_equal(wp.cpu().numpy(), owp)
    assert np.array_equal(cp.cpu().numpy(), ocp)


def test_pack_rejects_code_255(g):
    import microscaling_quantized_linear_amd as mx
    w = np.zeros((32, 128), np.uint8)
    codes = np.full((32, 4), 127, np.uint8)
    codes[5, 2] = 255
    with pytest.raises(mx.MXError) as ei:
        g.pack(E4M3, ROW32, 1, 32, 128, w, codes)
    assert ei.value.status == 4


# ------------------------------------------------------------------ quant

@pytest.mark.parametrize("rule", [OCP, CEIL])
@pytest.mark.parametrize("M,K,outl", [(16, 7168, 0.01), (5, 96, 0.05), (3, 1568, 0.0), (64, 512, 0.2)])
def test_quant_bit_exact(g, rule, M, K, outl):
    x = wl.activations(wl.rng(31, M * K), (M, K), outl)
    xq, xc = g.quant(x, rule)
    oq, oc = oracle.quant_act(x, rule)
    np.testing.assert_array_equal(xc, oc)
    np.testing.assert_array_equal(xq, oq)


@pytest.mark.parametrize("rule", [OCP, CEIL])
@pytest.mark.parametrize("order", ["sorted", "shuffled"])
def test_quant_every_finite_bf16(g, rule, order):
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    x = bits[finite].astype(np.uint16)            # 65280 finite patterns incl. +-0, subnormals
    if order == "shuffled":
        x = np.random.default_rng(5).permutation(x)
    x = x.reshape(-1, 32 * 40)[:, :]              # 51 rows x 1280
    xq, xc = g.quant(x, rule)
    oq, oc = oracle.quant_act(x, rule)
    np.testing.assert_array_equal(xc, oc)
    np.testing.assert_array_equal(xq, oq)


def test_quant_strided_output(g):
    x = wl.activations(wl.rng(32, 0), (7, 256), 0.01)
    xq, xc = g.quant(x, OCP, ldq=272)
    oq, oc = oracle.quant_act(x, OCP)
    np.testing.assert_array_equal(xq, oq)
    np.testing.assert_array_equal(xc, oc)


# ------------------------------------------------------------------ dense linear

def _dense_inputs(seed, elem, layout, M, N, K, lo=110, hi=140):
    rng = np.random.default_rng(seed)
    w = wl.e4m3_bytes(rng, (N, K)) if elem == E4M3 else wl.fp4_bytes(rng, (N, K // 2))
    cshape = (N, K // 32) if layout == ROW32 else (N // 32, K // 32)
    codes = wl.codes(rng, cshape, lo, hi)
    x = wl.activations(rng, (M, K), 0.01)
    bias = wl.activations(rng, (N,))
    return w, codes, x, bias


SMALL = [(1, 32, 128), (3, 64, 160), (16, 64, 1568), (5, 96, 96), (8, 128, 512),
         (17, 64, 256), (33, 32, 384)]
COMBOS = [(E4M3, ROW32, BF16), (E4M3, BLK32, BF16), (E4M3, ROW32, MXFP8),
          (E4M3, BLK32, MXFP8), (E2M1, ROW32, BF16)]


@pytest.mark.parametrize("elem,layout,act", COMBOS)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_linear_small(g, elem, layout, act, M, N, K):
    w, codes, x, bias = _dense_inputs([41, M, N, K, elem, layout], elem, layout, M, N, K)
    wp, cp = g.pack(elem, layout, 1, N, K, w, codes)
    use_bias = (M + N) % 2 == 1
    b = bias if use_bias else None
    for rule in ((OCP, CEIL) if act == MXFP8 else (OCP,)):
        if act == MXFP8:
            oq, oc = oracle.quant_act(x, rule)
            ref = oracle.linear(elem, layout, N, K, w, codes, M, MXFP8, xq=oq, xcodes=oc, bias=b)
            y = g.linear(elem, layout, N, K, wp, cp, MXFP8, x=x, rule=rule, bias=b)
            g.assert_close(y, ref, "quantized in call")
            y2 = g.linear(elem, layout, N, K, wp, cp, MXFP8, xq=oq, xcodes=oc, bias=b)
            g.assert_close(y2, ref, "pre-quantized")
            assert np.array_equal(y, y2)
        else:
            ref = oracle.linear(elem, layout, N, K, w, codes, M, BF16, x=x, bias=b)
            y = g.linear(elem, layout, N, K, wp, cp, BF16, x=x, bias=b)
            g.assert_close(y, ref)


@pytest.mark.parametrize("layout", [ROW32, BLK32])
@pytest.mark.parametrize("M,N,K", [(65, 64, 256), (300, 256, 384), (257, 1792, 1568),
                                   (512, 512, 1024)])
def test_gemm_small(g, layout, M, N, K):
    w, codes, x, bias = _dense_inputs([42, M, N, K, layout], E4M3, layout, M, N, K)
    wp, cp = g.pack(E4M3, layout, 1, N, K, w, codes)
    oq, oc = oracle.quant_act(x, OCP)
    b = bias if M % 2 else None
    ref = oracle.linear(E4M3, layout, N, K, w, codes, M, MXFP8, xq=oq, xcodes=oc, bias=b)
    y = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=x, rule=OCP, bias=b)
    g.assert_close(y, ref, "gemm")
    # row-major pre-quantized input (restaged into the tile-major layout in
    # the workspace) gives the same bits
    y2 = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, xq=oq, xcodes=oc, bias=b)
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("K", [96, 640, 928, 1152, 1184, 1280, 1408, 1536, 1664, 1792, 1920, 2048])
def test_gemm_step_remainders(g, K):
    """The GEMM's K loop runs eight 128-K steps an iteration and then the
    S % 8 steps left (S = ceil(K / 128)): every remainder 0 .. 7, with and
    without a partial last step, with fewer than eight steps and with more."""
    M, N = 80, 64
    for layout in (ROW32, BLK32):
        w, codes, x, bias = _dense_inputs([46, M, N, K, layout], E4M3, layout, M, N, K)
        wp, cp = g.pack(E4M3, layout, 1, N, K, w, codes)
        oq, oc = oracle.quant_act(x, OCP)
        ref = oracle.linear(E4M3, layout, N, K, w, codes, M, MXFP8, xq=oq, xcodes=oc, bias=bias)
        y = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=x, rule=OCP, bias=bias)
        g.assert_close(y, ref, f"gemm K={K} layout={layout}")


def test_extreme_codes_w8a8(g):
    # weight codes 0, 1 and 254 with activations scaled by 2^-100, so that the
    # results stay inside bf16's range; activation codes near 19
    M, N, K = 4, 64, 256
    rng = np.random.default_rng(43)
    w = wl.e4m3_bytes(rng, (N, K))
    codes = rng.choice(np.array([0, 1, 127, 200, 254], np.uint8), (N, K // 32))
    x = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(wl.activations(rng, (M, K))) * np.float32(2.0 ** -100))
    wp, cp = g.pack(E4M3, ROW32, 1, N, K, w, codes)
    oq, oc = oracle.quant_act(x, OCP)
    assert oc.min() < 30
    ref = oracle.linear(E4M3, ROW32, N, K, w, codes, M, MXFP8, xq=oq, xcodes=oc)
    y = g.linear(E4M3, ROW32, N, K, wp, cp, MXFP8, xq=oq, xcodes=oc)
    g.assert_close(y, ref, "extreme codes w8a8")


def test_extreme_codes_a16(g):
    # codes 0, 1 and 150 mixed with 127 on the decode path (the code extremes
    # have their own tests)
    M, N, K = 4, 64, 256
    rng = np.random.default_rng(44)
    w = wl.e4m3_bytes(rng, (N, K))
    codes = rng.choice(np.array([0, 1, 127, 150], np.uint8), (N, K // 32))
    x = wl.activations(rng, (M, K))
    wp, cp = g.pack(E4M3, ROW32, 1, N, K, w, codes)
    ref = oracle.linear(E4M3, ROW32, N, K, w, codes, M, BF16, x=x)
    y = g.linear(E4M3, ROW32, N, K, wp, cp, BF16, x=x)
    g.assert_close(y, ref, "extreme codes a16")


# ------------------------------------------------------------------ the five workloads

def test_a16w8_gemv_m1_n256_k512_full(g):
    d = wl.linear_inputs(1)
    wp, cp = g.pack(E4M3, ROW32, 1, d["N"], d["K"], d["w"], d["codes"])
    ref = oracle.linear(E4M3, ROW32, d["N"], d["K"], d["w"], d["codes"], d["M"], BF16, x=d["x"])
    y = g.linear(E4M3, ROW32, d["N"], d["K"], wp, cp, BF16, x=d["x"])
    g.assert_close(y, ref, "a16w8 M=1 N=256 K=512", strict=True)


@pytest.mark.parametrize("rule", [OCP, CEIL])
def test_w8a8_gemv_n7168_k7168_full(g, rule):
    d = wl.linear_inputs(2)
    N, K = d["N"], d["K"]
    wp, cp = g.pack(E4M3, BLK32, 1, N, K, d["w"], d["codes"])
    for M in (1, 4, 16):
        x = d["x"][:M]
        xq, xc = g.quant(x, rule)
        oq, oc = oracle.quant_act(x, rule)
        assert np.array_equal(xq, oq) and np.array_equal(xc, oc)
        ref = oracle.linear(E4M3, BLK32, N, K, d["w"], d["codes"], M, MXFP8, xq=oq, xcodes=oc)
        y = g.linear(E4M3, BLK32, N, K, wp, cp, MXFP8, x=x, rule=rule)
        g.assert_close(y, ref, f"w8a8 N=K=7168 M={M}", strict=True)
        y2 = g.linear(E4M3, BLK32, N, K, wp, cp, MXFP8, x=x, rule=rule)
        assert np.array_equal(y, y2), "not deterministic"


def test_a16w8_gemv_m8_n4096_k1568_full_and_negative_zero(g):
    d = wl.linear_inputs(3)
    N, K, M = d["N"], d["K"], d["M"]
    wp, cp = g.pack(E4M3, ROW32, 1, N, K, d["w"], d["codes"])
    ref = oracle.linear(E4M3, ROW32, N, K, d["w"], d["codes"], M, BF16, x=d["x"])
    y = g.linear(E4M3, ROW32, N, K, wp, cp, BF16, x=d["x"])
    g.assert_close(y, ref, "a16w8 M=8 N=4096 K=1568", strict=True)
    # -0 (0x80) decodes equal to +0: swapping them leaves the output unchanged
    w0 = d["w"].copy()
    w0[w0 == 0x80] = 0x00
    w0[:, ::7] = 0x00
    w1 = w0.copy()
    w1[w0 == 0x00] = 0x80
    assert (w1 == 0x80).sum() > 1000
    y0 = g.linear(E4M3, ROW32, N, K, *g.pack(E4M3, ROW32, 1, N, K, w0, d["codes"]), BF16, x=d["x"])
    y1 = g.linear(E4M3, ROW32, N, K, *g.pack(E4M3, ROW32, 1, N, K, w1, d["codes"]), BF16, x=d["x"])
    assert np.array_equal(y0, y1)
    # the W8A8 variant of the same shape
    oq, oc = oracle.quant_act(d["x"], OCP)
    ref8 = oracle.linear(E4M3, ROW32, N, K, d["w"], d["codes"], M, MXFP8, xq=oq, xcodes=oc)
    y8 = g.linear(E4M3, ROW32, N, K, wp, cp, MXFP8, x=d["x"], rule=OCP)
    g.assert_close(y8, ref8, "w8a8 M=8 N=4096 K=1568")


def test_moe_e32_n3072_k3072_t16_top8_full(g):
    d = wl.moe_inputs(4)
    E, N, K = d["E"], d["N"], d["K"]
    wp, cp = g.pack(E2M1, ROW32, E, N, K, d["w"], d["codes"])
    ref = oracle.moe_linear(E2M1, E, N, K, d["w"], d["codes"], d["x"], d["ids"])
    y = g.moe(E2M1, E, N, K, wp, cp, d["x"], d["ids"])
    g.assert_close(y, ref, "moe E=32 per slot", strict=True)
    refc = oracle.moe_linear(E2M1, E, N, K, d["w"], d["codes"], d["x"], d["ids"], d["weights"])
    yc = g.moe(E2M1, E, N, K, wp, cp, d["x"], d["ids"], d["weights"])
    g.assert_close(yc, refc, "moe E=32 combined", strict=True)


def test_gemm_m4096_n7168_k7168_every_row(g):
    """The prefill GEMM at its full size, in the launch configuration the
    benchmark times, against the oracle on every output (4096 x 7168), with
    the per-token quantization of every row checked bit for bit."""
    d = wl.linear_inputs(5)
    N, K, M = d["N"], d["K"], d["M"]
    wp, cp = g.pack(E4M3, BLK32, 1, N, K, d["w"], d["codes"])
    y = g.linear(E4M3, BLK32, N, K, wp, cp, MXFP8, x=d["x"], rule=OCP)
    oq, oc = oracle.quant_act(d["x"], OCP)
    gq, gc = g.quant(d["x"], OCP)
    assert np.array_equal(gq, oq) and np.array_equal(gc, oc)
    ref = oracle.linear(E4M3, BLK32, N, K, d["w"], d["codes"], M, MXFP8, xq=oq, xcodes=oc)
    g.assert_close(y, ref, "gemm M=4096 N=K=7168", strict=True)
    # and per 256-token workgroup tile: no tile may hide behind the others
    yv = g.bf16_to_f64(y).reshape(M, N)
    for t in range(0, M, 256):
        e = np.linalg.norm(yv[t:t + 256] - ref[t:t + 256]) / np.linalg.norm(ref[t:t + 256])
        assert e <= g.REL_L2, f"tokens {t}..{t + 255}: relative L2 {e:.3e}"


# ------------------------------------------------------------------ MoE edges

def test_moe_edges(g):
    E, N, K, T, topk = 6, 32, 256, 40, 2
    d = wl.moe_inputs(4, E=E, N=N, K=K, T=T, topk=topk, seed=3)
    ids = d["ids"].copy()
    ids[:, 0] = 0                  # expert 0 gets all 40 tokens: 3 slot batches
    ids[1, 1] = -3                 # out of range: zero rows
    ids[2, 1] = E
    ids[3, 1] = 0                  # duplicate of slot 0
    ids[ids == 5] = 4              # expert 5 receives nothing
    wp, cp = g.pack(E2M1, ROW32, E, N, K, d["w"], d["codes"])
    ref = oracle.moe_linear(E2M1, E, N, K, d["w"], d["codes"], d["x"], ids)
    y = g.moe(E2M1, E, N, K, wp, cp, d["x"], ids)
    g.assert_close(y, ref, "moe edges")
    yv = y.reshape(T, topk, N)
    assert np.all(yv[1, 1] == 0) and np.all(yv[2, 1] == 0)
    assert np.array_equal(yv[3, 0], yv[3, 1])
    refc = oracle.moe_linear(E2M1, E, N, K, d["w"], d["codes"], d["x"], ids, d["weights"])
    yc = g.moe(E2M1, E, N, K, wp, cp, d["x"], ids, d["weights"])
    g.assert_close(yc, refc, "moe edges combined")


def test_moe_e4m3_weights(g):
    E, N, K, T, topk = 4, 48, 1568, 6, 2
    rng = np.random.default_rng(61)
    w = wl.e4m3_bytes(rng, (E, N, K))
    codes = wl.codes(rng, (E * N, K // 32), 118, 132)
    x = wl.activations(rng, (T, K))
    ids, wts = wl.routing(rng, T, E, topk)
    wp, cp = g.pack(E4M3, ROW32, E, N, K, w, codes)
    ref = oracle.moe_linear(E4M3, E, N, K, w, codes, x, ids)
    y = g.moe(E4M3, E, N, K, wp, cp, x, ids)
    g.assert_close(y, ref, "moe e4m3")


# ------------------------------------------------- T16 activation layout

T16_SHAPES = [(1, 128), (3, 160), (16, 7168), (17, 1568), (64, 512), (300, 384)]


@pytest.mark.parametrize("rule", [OCP, CEIL])
@pytest.mark.parametrize("M,K", T16_SHAPES)
def test_quant_t16_bit_exact(g, rule, M, K):
    """mx_quant_act_t16 holds exactly the oracle's bytes and codes, in the
    documented layout; padding tokens and K hold byte 0 and code 127."""
    x = wl.activations(np.random.default_rng([43, M, K]), (M, K), 0.02)
    xq, xc = g.quant_t16(x, rule)
    d, c = g.t16_unpack(xq.cpu().numpy(), xc.cpu().numpy(), M, K)
    oq, oc = oracle.quant_act(x, rule)
    np.testing.assert_array_equal(d[:M, :K], oq)
    np.testing.assert_array_equal(c[:M, :K // 32], oc)
    assert not d[M:].any() and not d[:, K:].any()
    assert (c[M:] == 127).all() and (c[:, K // 32:] == 127).all()


@pytest.mark.parametrize("layout", [ROW32, BLK32])
@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (5, 96, 1568), (16, 256, 7168), (40, 64, 384),
                                   (300, 256, 384)])
def test_linear_t16_equals_in_call(g, layout, M, N, K):
    """A linear on a T16 activation gives the in-call result bit for bit
    (decode GEMV for M <= 64, prefill GEMM above), within the bar of the
    oracle."""
    w, codes, x, bias = _dense_inputs([44, M, N, K, layout], E4M3, layout, M, N, K)
    wp, cp = g.pack(E4M3, layout, 1, N, K, w, codes)
    b = bias if M % 2 else None
    xq, xc = g.quant_t16(x, OCP)
    y = g.linear(E4M3, layout, N, K, wp, cp, MXFP8_T16, xq=xq, xcodes=xc, bias=b, M=M)
    y_in = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=x, rule=OCP, bias=b)
    assert np.array_equal(y, y_in)
    oq, oc = oracle.quant_act(x, OCP)
    ref = oracle.linear(E4M3, layout, N, K, w, codes, M, MXFP8, xq=oq, xcodes=oc, bias=b)
    g.assert_close(y, ref, "T16 activation")


# ------------------------------------------------------------------ fused quantization

FUSED_SHAPES = [(1, 64, 1024), (2, 96, 2048), (15, 256, 4096), (16, 1792, 7168), (17, 64, 8192),
                (33, 32, 1024), (64, 128, 2048), (4, 7168, 7168),
                # whole token tiles at four and eight steps a wavefront (the
                # activation copies go into a ring of LDS slots)
                (16, 256, 4096), (32, 64, 8192)]


@pytest.mark.parametrize("layout", [ROW32, BLK32])
@pytest.mark.parametrize("M,N,K", FUSED_SHAPES)
def test_fused_quant_gemv(g, layout, M, N, K):
    """Quantization inside the decode GEMV (no workspace) gives the result of
    mx_quant_act_t16 followed by the GEMV on it, and of the row-major
    pre-quantized path, bit for bit, under both rules; within the bar of the
    oracle."""
    import microscaling_quantized_linear_amd as mx
    if layout == BLK32 and N % 32:
        pytest.skip("BLK32 needs N % 32 == 0")
    assert mx.mx_linear_workspace(E4M3, layout, N, K, M, MXFP8, 0) == 0
    w, codes, x, bias = _dense_inputs([45, M, N, K, layout], E4M3, layout, M, N, K)
    wp, cp = g.pack(E4M3, layout, 1, N, K, w, codes)
    for rule in (OCP, CEIL):
        b = bias if (M + rule) % 2 else None
        y = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, x=x, rule=rule, bias=b)
        xq, xc = g.quant_t16(x, rule)
        y16 = g.linear(E4M3, layout, N, K, wp, cp, MXFP8_T16, xq=xq, xcodes=xc, bias=b, M=M)
        assert np.array_equal(y, y16), "fused != T16 path"
        oq, oc = oracle.quant_act(x, rule)
        yr = g.linear(E4M3, layout, N, K, wp, cp, MXFP8, xq=oq, xcodes=oc, bias=b)
        assert np.array_equal(y, yr), "fused != row-major pre-quantized path"
        ref = oracle.linear(E4M3, layout, N, K, w, codes, M, MXFP8, xq=oq, xcodes=oc, bias=b)
        g.assert_close(y, ref, f"fused quant rule {rule}")


# ------------------------------------------------------------------ more MoE shapes

MOE_SHAPES = [
    # elem, E, N, K, T, topk
    (E2M1, 8, 64, 1024, 5, 2),
    (E2M1, 16, 128, 3072, 16, 8),
    (E2M1, 12, 96, 992, 7, 3),        # K % 128 != 0: padded tail
    (E4M3, 4, 48, 2048, 6, 2),
    (E4M3, 5, 32, 3072, 16, 4),
    (E2M1, 64, 16, 1024, 16, 8),      # one tile per expert, many experts per workgroup
    (E2M1, 300, 16, 1024, 4, 4),
    (E2M1, 16, 64, 512, 5, 12),       # combine over more than 8 slots (two groups)
    (E2M1, 24, 32, 256, 3, 24),       # topk = E, three groups of 8
]


@pytest.mark.parametrize("elem,E,N,K,T,topk", MOE_SHAPES)
def test_moe_shapes(g, elem, E, N, K, T, topk):
    """The grouped GEMV at further shapes: long K, a ragged K tail, e4m3
    weights, one tile per expert with many experts; per-slot and combined,
    deterministic, against the oracle."""
    rng = np.random.default_rng([62, elem, E, N, K, T, topk])
    if elem == E2M1:
        w = wl.fp4_bytes(rng, (E, N, K // 2))
    else:
        w = wl.e4m3_bytes(rng, (E, N, K))
    codes = wl.codes(rng, (E * N, K // 32), 120, 132)
    x = wl.activations(rng, (T, K))
    ids, wts = wl.routing(rng, T, E, topk)
    wp, cp = g.pack(elem, ROW32, E, N, K, w, codes)
    ref = oracle.moe_linear(elem, E, N, K, w, codes, x, ids)
    y = g.moe(elem, E, N, K, wp, cp, x, ids)
    g.assert_close(y, ref, "moe")
    assert np.array_equal(y, g.moe(elem, E, N, K, wp, cp, x, ids)), "not deterministic"
    refc = oracle.moe_linear(elem, E, N, K, w, codes, x, ids, wts)
    yc = g.moe(elem, E, N, K, wp, cp, x, ids, wts)
    g.assert_close(yc, refc, "moe combined")


def test_moe_edges_long_k(g):
    """Routing edges at K = 1024: an expert with 40 slots (three batches of
    16), ids out of range (zero rows), a duplicate id, an expert nobody routes
    to, and no valid id at all."""
    E, N, K, T, topk = 6, 32, 1024, 40, 2
    d = wl.moe_inputs(4, E=E, N=N, K=K, T=T, topk=topk, seed=3)
    ids = d["ids"].copy()
    ids[:, 0] = 0
    ids[1, 1] = -3
    ids[2, 1] = E
    ids[3, 1] = 0
    ids[ids == 5] = 4
    wp, cp = g.pack(E2M1, ROW32, E, N, K, d["w"], d["codes"])
    ref = oracle.moe_linear(E2M1, E, N, K, d["w"], d["codes"], d["x"], ids)
    y = g.moe(E2M1, E, N, K, wp, cp, d["x"], ids)
    g.assert_close(y, ref, "moe edges")
    yv = y.reshape(T, topk, N)
    assert np.all(yv[1, 1] == 0) and np.all(yv[2, 1] == 0)
    assert np.array_equal(yv[3, 0], yv[3, 1])
    refc = oracle.moe_linear(E2M1, E, N, K, d["w"], d["codes"], d["x"], ids, d["weights"])
    yc = g.moe(E2M1, E, N, K, wp, cp, d["x"], ids, d["weights"])
    g.assert_close(yc, refc, "moe edges combined")
    # no valid id at all: every row zero
    bad = np.full_like(ids, -1)
    assert not g.moe(E2M1, E, N, K, wp, cp, d["x"], bad).any()


# ------------------------------------------------------------------ MoE block

def _moe_block_inputs(seed, elem, E, Np, inter, K, H, T, topk):
    rng = np.random.default_rng(seed)
    rowb = K // 2 if elem == E2M1 else K
    gen = (lambda shape: wl.fp4_bytes(rng, shape)) if elem == E2M1 else \
        (lambda shape: wl.e4m3_bytes(rng, shape))
    w13 = gen((E, 2 * Np, rowb))
    w13[:, inter:Np] = 0
    w13[:, Np + inter:] = 0
    s13 = wl.codes(rng, (E, 2 * Np, K // 32), 120, 128)
    w2 = gen((E, H, Np // 2 if elem == E2M1 else Np))
    w2[:, :, (inter // 2 if elem == E2M1 else inter):] = 0
    s2 = wl.codes(rng, (E, H, Np // 32), 120, 128)
    x = wl.activations(rng, (T, K))
    ids, wts = wl.routing(rng, T, E, topk)
    return w13, s13, w2, s2, x, ids, wts


MOE_BLOCK = [(E2M1, 8, 96, 64, 256, 96, 5, 2), (E2M1, 6, 128, 128, 1024, 64, 16, 4),
             (E4M3, 4, 64, 32, 160, 48, 3, 2), (E2M1, 4, 576, 576, 512, 64, 4, 2)]


@pytest.mark.parametrize("elem,E,Np,inter,K,H,T,topk", MOE_BLOCK)
def test_moe_block(g, elem, E, Np, inter, K, H, T, topk):
    """mx_moe_copies bit for bit; mx_moe_gate_up (silu(gate) * up) and
    mx_moe_down (per-slot hidden rows, per slot and combined) against the
    oracle; the whole block chained against the oracle's chain with the hidden
    rows rounded to bf16 in between."""
    w13, s13, w2, s2, x, ids, wts = _moe_block_inputs([46, elem, E, Np, K], elem, E, Np, inter,
                                                      K, H, T, topk)
    ids[0, -1] = -1                               # an id out of range: zero rows
    o = oracle.moe_copies(elem, E, Np, inter, K, H, w13, s13, w2, s2)
    gpu = g.moe_copies(elem, E, Np, inter, K, H, w13, s13, w2, s2)
    for a, b in zip(gpu, o):
        np.testing.assert_array_equal(a, b)
    ow13, os13, ow2, os2 = o
    wp13, cp13 = g.pack(elem, ROW32, E, 2 * inter, K, ow13, os13.reshape(-1))
    wp2, cp2 = g.pack(elem, ROW32, E, H, inter, ow2, os2.reshape(-1))
    # up-gate with the fused silu
    href = oracle.moe_gate_up(elem, E, inter, K, ow13, os13.reshape(-1), x, ids)
    h = g.moe_gate_up(elem, E, inter, K, wp13, cp13, x, ids, ldh=inter + 8 * (inter % 16 == 0))
    g.assert_close(h.reshape(T, topk, inter), href, "gate_up")
    assert not h.reshape(T, topk, inter)[0, -1].any()
    # down on seeded hidden rows (the same input for both sides)
    a = wl.activations(np.random.default_rng([47, E, H]), (T * topk, inter))
    yref = oracle.moe_linear_rows(elem, E, H, inter, ow2, os2.reshape(-1), a, ids)
    y = g.moe_down(elem, E, H, inter, wp2, cp2, a, ids)
    g.assert_close(y.reshape(T, topk, H), yref, "down")
    ycref = oracle.moe_linear_rows(elem, E, H, inter, ow2, os2.reshape(-1), a, ids, wts)
    yc = g.moe_down(elem, E, H, inter, wp2, cp2, a, ids, wts)
    g.assert_close(yc.reshape(T, H), ycref, "down combined")
    # the block: gate_up -> down -> combine, against the oracle's chain (hidden
    # rows rounded to bf16 between the two products, as the block hands them on)
    hb = oracle.bf16_round_array(href).reshape(T * topk, inter)
    chain = oracle.moe_linear_rows(elem, E, H, inter, ow2, os2.reshape(-1), hb, ids, wts)
    yb = g.moe_down(elem, E, H, inter, wp2, cp2, h, ids, wts)
    g.assert_close(yb.reshape(T, H), chain, "block")


def test_moe_copies_refuses_padding(g):
    import microscaling_quantized_linear_amd as mx
    E, Np, inter, K, H = 2, 96, 64, 128, 32
    w13, s13, w2, s2, _, _, _ = _moe_block_inputs(48, E2M1, E, Np, inter, K, H, 2, 1)
    w13[1, Np + inter + 1, 3] = 0x22
    with pytest.raises(mx.MXError) as ei:
        g.moe_copies(E2M1, E, Np, inter, K, H, w13, s13, w2, s2)
    assert ei.value.status == 4                   # MX_ERR_VALUE


@pytest.mark.parametrize("K", [128, 1024])
def test_moe_max_pairs(g, K):
    """T * topk at the routing scan's maximum (4096 pairs): the ballot walks 64
    rounds, the slot list is full, and the expert everyone routes to gets 16
    batches of slots; one pair more is refused before any launch.  K = 128
    runs the one-wavefront launch; K = 1024 the two-wavefront one, whose
    first 128 ids and first weight chunk are requested ahead of the scan."""
    import microscaling_quantized_linear_amd as mx
    E, N, T, topk = 16, 32, 512, 8
    rng = np.random.default_rng([63, K])
    w = wl.fp4_bytes(rng, (E, N, K // 2))
    codes = wl.codes(rng, (E * N, K // 32), 120, 132)
    x = wl.activations(rng, (T, K))
    ids, wts = wl.routing(rng, T, E, topk)
    ids[:, 0] = 3                                # expert 3: every token, 512+ slots
    sub = ids[:, 1:]
    sub[sub == 3] = 14                           # a repeated id gives identical rows
    wp, cp = g.pack(E2M1, ROW32, E, N, K, w, codes)
    g.assert_close(g.moe(E2M1, E, N, K, wp, cp, x, ids),
                   oracle.moe_linear(E2M1, E, N, K, w, codes, x, ids), "moe 4096 pairs")
    g.assert_close(g.moe(E2M1, E, N, K, wp, cp, x, ids, wts),
                   oracle.moe_linear(E2M1, E, N, K, w, codes, x, ids, wts), "moe 4096 combined")
    with pytest.raises(mx.MXError) as ei:
        mx.mx_moe_workspace(E2M1, E, N, K, 4097, 1, 0)
    assert ei.value.status == 2                  # MX_ERR_SHAPE


@pytest.mark.parametrize("path", ["a16", "w8a8_fused", "w8a8_gemm", "w8a8_t16"])
def test_strided_activation_and_output(g, path):
    """Leading dimensions above K (activations) and N (output): every path
    gives the contiguous call's bits and leaves the padding columns of y
    untouched."""
    import torch
    import microscaling_quantized_linear_amd as mx
    layout = BLK32 if path != "a16" else ROW32
    M = {"a16": 5, "w8a8_fused": 16, "w8a8_gemm": 200, "w8a8_t16": 7}[path]
    N, K = 512, 1024
    w, codes, x, bias = _dense_inputs([48, M, N, K, layout], E4M3, layout, M, N, K)
    wp, cp = g.pack(E4M3, layout, 1, N, K, w, codes)
    act = BF16 if path == "a16" else MXFP8
    want = g.linear(E4M3, layout, N, K, wp, cp, act, x=x, rule=OCP, bias=bias)
    ldx, ldy = K + 24, N + 40
    xs = np.zeros((M, ldx), np.uint16)
    xs[:, :K] = x
    xd = g.dev(xs)
    bd = g.dev(bias)
    y = torch.full((M, ldy), 0x7A7A, dtype=torch.int16, device=g.DEV)
    if path == "w8a8_t16":
        qb, cb = mx.mx_act_t16_sizes(M, K)
        xq = torch.empty(qb, dtype=torch.uint8, device=g.DEV)
        xc = torch.empty(cb, dtype=torch.uint8, device=g.DEV)
        mx.mx_quant_act_t16(M, K, xd, ldx, xq, xc, OCP)
        mx.mx_linear(E4M3, layout, N, K, wp, cp, M, MXFP8_T16, 0, None, 0, xq, 0, xc, 0, bd, y,
                     ldy, None, 0)
    else:
        need = mx.mx_linear_workspace(E4M3, layout, N, K, M, act, 0)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=g.DEV)
        mx.mx_linear(E4M3, layout, N, K, wp, cp, M, act, OCP, xd, ldx, None, 0, None, 0, bd, y,
                     ldy, ws, need)
    torch.cuda.synchronize()
    got = g.host_u16(y)
    np.testing.assert_array_equal(got[:, :N], want)
    assert (got[:, N:] == 0x7A7A).all()
