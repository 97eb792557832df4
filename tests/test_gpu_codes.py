"""Parity over the whole E8M0 code range, through the C ABI.

Two kinds of test:

* Code extremes on random data.  Every row's codes lie at the top of the
  range (247 .. 254, where an e4m3 value times 2^(code - 127) exceeds bf16's
  largest number) with the activations scaled by 2^-100, or at the bottom
  (0 .. 9, where the scaled weights fall below bf16's smallest normal) with
  the activations scaled by 2^+100, so every output stays inside bf16's
  range and the oracle's result is finite.  Each A16 path (A16W8 with 1x32
  and 32x32 codes, A16W4, the grouped MoE with e2m1 and e4m3 weights, the
  MoE block's up-gate and down projection) and the W8A8 paths are held to
  the usual bar against the oracle.

* Exhaustive decode.  Row n of the weight matrix holds the byte n (e4m3,
  the two NaN codes 0x7F / 0xFF replaced by 0) or the nibble n (e2m1) at
  every K; block b of every row has code b (b = 0 .. 254).  Token b is
  one-hot at one K of block b with the value 2^t, t = 127 - b kept inside
  bf16's normal exponents, so y[b][n] = dec(n) * 2^(b - 127 + t): every
  byte (nibble) at every code, each product alone in its sum.  The GPU's
  outputs must equal the oracle's value for value (a sum of one exact term
  and zeros is exact; -0 equals +0).
"""
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


def _scaled(x_bits, e):
    """bf16 activations times 2^e (exact: every value stays normal)."""
    return wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(x_bits) * np.float32(2.0 ** e))


HIGH = np.arange(247, 255, dtype=np.uint8)        # top of the code range
LOW = np.arange(0, 10, dtype=np.uint8)            # bottom: below kLo of e4m3 (10)
LOW4 = np.arange(0, 3, dtype=np.uint8)            # bottom for e2m1 (kLo 2)


def _extreme(seed, elem, layout, M, N, K, codes_from, xscale):
    rng = np.random.default_rng(seed)
    w = wl.e4m3_bytes(rng, (N, K)) if elem == E4M3 else wl.fp4_bytes(rng, (N, K // 2))
    cshape = (N, K // 32) if layout == ROW32 else (N // 32, K // 32)
    codes = rng.choice(codes_from, cshape).astype(np.uint8)
    x = _scaled(wl.activations(rng, (M, K)), xscale)
    return w, codes, x


CASES_A16 = [
    (E4M3, ROW32, HIGH, -100), (E4M3, ROW32, LOW, 100),
    (E4M3, BLK32, HIGH, -100), (E4M3, BLK32, LOW, 100),
    (E2M1, ROW32, HIGH, -100), (E2M1, ROW32, LOW4, 100),
]


@pytest.mark.parametrize("elem,layout,codes_from,xscale", CASES_A16)
@pytest.mark.parametrize("M,N,K", [(4, 64, 256), (16, 96, 1568), (3, 64, 7168)])
def test_a16_code_extremes(g, elem, layout, codes_from, xscale, M, N, K):
    w, codes, x = _extreme([71, elem, layout, int(codes_from[0]), M, N, K], elem, layout, M, N, K,
                           codes_from, xscale)
    wp, cp = g.pack(elem, layout, 1, N, K, w, codes)
    ref = oracle.linear(elem, layout, N, K, w, codes, M, BF16, x=x)
    assert np.all(np.isfinite(ref))
    y = g.linear(elem, layout, N, K, wp, cp, BF16, x=x)
    g.assert_close(y, ref, f"a16 codes {codes_from[0]}..{codes_from[-1]}")


def test_a16_code_extremes_mixed_rows(g):
    """A row whose blocks mix extreme and ordinary codes, with the ordinary
    blocks' weights zero: only the extreme blocks contribute, and a wavefront
    switches to the exact form mid-tensor."""
    M, N, K = 8, 64, 2048
    rng = np.random.default_rng(72)
    w = wl.e4m3_bytes(rng, (N, K))
    codes = np.full((N, K // 32), 127, np.uint8)
    hot = rng.random((N, K // 32)) < 0.2
    codes[hot] = rng.choice(HIGH, hot.sum())
    w.reshape(N, K // 32, 32)[~hot] = 0
    x = _scaled(wl.activations(rng, (M, K)), -100)
    wp, cp = g.pack(E4M3, ROW32, 1, N, K, w, codes)
    ref = oracle.linear(E4M3, ROW32, N, K, w, codes, M, BF16, x=x)
    y = g.linear(E4M3, ROW32, N, K, wp, cp, BF16, x=x)
    g.assert_close(y, ref, "a16 mixed extreme rows")


@pytest.mark.parametrize("codes_from,xscale", [(HIGH, -100), (LOW, 100)])
def test_w8a8_code_extremes(g, codes_from, xscale):
    M, N, K = 16, 128, 1024
    w, codes, x = _extreme([73, int(codes_from[0])], E4M3, BLK32, M, N, K, codes_from, xscale)
    wp, cp = g.pack(E4M3, BLK32, 1, N, K, w, codes)
    oq, oc = oracle.quant_act(x, OCP)
    ref = oracle.linear(E4M3, BLK32, N, K, w, codes, M, MXFP8, xq=oq, xcodes=oc)
    y = g.linear(E4M3, BLK32, N, K, wp, cp, MXFP8, x=x, rule=OCP)
    g.assert_close(y, ref, "w8a8 extreme codes")


@pytest.mark.parametrize("elem,codes_from,xscale", [(E2M1, HIGH, -100), (E2M1, LOW4, 100),
                                                   (E4M3, HIGH, -100), (E4M3, LOW, 100)])
def test_moe_code_extremes(g, elem, codes_from, xscale):
    E, N, K, T, topk = 4, 64, 1536, 6, 2
    rng = np.random.default_rng([74, elem, int(codes_from[0])])
    w = wl.e4m3_bytes(rng, (E, N, K)) if elem == E4M3 else wl.fp4_bytes(rng, (E, N, K // 2))
    codes = rng.choice(codes_from, (E * N, K // 32)).astype(np.uint8)
    x = _scaled(wl.activations(rng, (T, K)), xscale)
    ids, wts = wl.routing(rng, T, E, topk)
    wp, cp = g.pack(elem, ROW32, E, N, K, w, codes)
    ref = oracle.moe_linear(elem, E, N, K, w, codes, x, ids)
    y = g.moe(elem, E, N, K, wp, cp, x, ids)
    g.assert_close(y, ref, "moe extreme codes")
    refc = oracle.moe_linear(elem, E, N, K, w, codes, x, ids, wts)
    yc = g.moe(elem, E, N, K, wp, cp, x, ids, wts)
    g.assert_close(yc, refc, "moe extreme codes, combined")


def test_moe_block_code_extremes(g):
    """Up-gate (SiLU product) and down projection with top-of-range codes."""
    E, inter, H, T, topk = 4, 64, 512, 4, 2
    rng = np.random.default_rng(75)
    w13 = wl.fp4_bytes(rng, (E, 2 * inter, H // 2))
    c13 = rng.choice(HIGH, (E * 2 * inter, H // 32)).astype(np.uint8)
    w2 = wl.fp4_bytes(rng, (E, H, inter // 2))
    c2 = rng.choice(HIGH, (E * H, inter // 32)).astype(np.uint8)
    # weights near 2^(250 - 127) against x * 2^-100: gate and up sums near
    # 2^30, h = silu(gate) * up near 2^60
    x = _scaled(wl.activations(rng, (T, H)), -100)
    ids, wts = wl.routing(rng, T, E, topk)
    w13p, c13p = g.pack(E2M1, ROW32, E, 2 * inter, H, w13, c13)
    h = g.moe_gate_up(E2M1, E, inter, H, w13p, c13p, x, ids)
    href = oracle.moe_gate_up(E2M1, E, inter, H, w13, c13, x, ids)
    g.assert_close(h, href.reshape(T * topk, inter), "moe gate_up extreme codes")
    # the down projection's rows scaled by 2^-175 (two exact steps), so its
    # sums land near 2^10
    hs = _scaled(_scaled(h, -100), -75)
    w2p, c2p = g.pack(E2M1, ROW32, E, H, inter, w2, c2)
    yref = oracle.moe_linear_rows(E2M1, E, H, inter, w2, c2, hs, ids, wts)
    yb = g.moe_down(E2M1, E, H, inter, w2p, c2p, hs, ids, wts)
    g.assert_close(yb, yref, "moe down extreme codes")


# ------------------------------------------------------------ exhaustive decode

NCODES = 255                     # codes 0 .. 254 (255 is NaN and refused by the pack)
KX = 32 * 256                    # 256 blocks: block b has code b, block 255 code 127


def _onehot_x():
    """Token b: one-hot at K 32 b + b % 32 with the value 2^(127 - b), the
    exponent kept in [-126, 127] (bf16 normal)."""
    x = np.zeros((NCODES, KX), np.uint16)
    for b in range(NCODES):
        t = min(max(127 - b, -126), 127)
        x[b, 32 * b + b % 32] = (t + 127) << 7           # bf16 bits of 2^t
    return x


def _decode_weights(elem):
    if elem == E4M3:
        n = np.arange(256, dtype=np.uint8)
        n[[0x7F, 0xFF]] = 0                              # the NaN codes: no finite value
        return np.repeat(n[:, None], KX, axis=1)
    nib = np.arange(16, dtype=np.uint8)
    return np.repeat((nib | (nib << 4))[:, None], KX // 2, axis=1)


def _decode_codes(N, layout):
    blk = np.minimum(np.arange(KX // 32), 254).astype(np.uint8)
    blk[255] = 127
    rows = N if layout == ROW32 else N // 32
    return np.repeat(blk[None, :], rows, axis=0)


def _values_equal(y_bits, ref, what):
    y = g_bf16(y_bits).reshape(ref.shape)
    r = g_bf16(wl.f32_to_bf16_bits(ref.astype(np.float32))).reshape(ref.shape)
    bad = y != r
    assert not bad.any(), (f"{what}: {bad.sum()} outputs differ, first at "
                           f"{np.argwhere(bad)[0].tolist()}")


def g_bf16(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("elem,layout", [(E4M3, ROW32), (E4M3, BLK32), (E2M1, ROW32)])
def test_decode_every_code_a16(g, elem, layout):
    N = 256 if elem == E4M3 else 16
    w, codes, x = _decode_weights(elem), _decode_codes(N, layout), _onehot_x()
    ref = oracle.linear(elem, layout, N, KX, w, codes, NCODES, BF16, x=x)
    wp, cp = g.pack(elem, layout, 1, N, KX, w, codes)
    _values_equal(g.linear(elem, layout, N, KX, wp, cp, BF16, x=x), ref, "a16 decode")


@pytest.mark.parametrize("elem", [E4M3, E2M1])
def test_decode_every_code_moe(g, elem):
    """The grouped MoE GEMV: two experts with the same weights, tokens routed
    alternately to each."""
    N = 256 if elem == E4M3 else 16
    w1, x = _decode_weights(elem), _onehot_x()
    w = np.stack([w1, w1])
    codes = np.concatenate([_decode_codes(N, ROW32)] * 2)
    ids = (np.arange(NCODES, dtype=np.int32) % 2)[:, None]
    ref = oracle.moe_linear(elem, 2, N, KX, w, codes, x, ids)
    wp, cp = g.pack(elem, ROW32, 2, N, KX, w, codes)
    _values_equal(g.moe(elem, 2, N, KX, wp, cp, x, ids), ref, "moe decode")


@pytest.mark.parametrize("layout", [ROW32, BLK32])
def test_decode_every_code_w8a8(g, layout):
    """W8A8: the weight decode inside the scaled matrix-core product, on the
    GEMM (255 tokens) and on the decode GEMV (64 tokens a call: quantized in
    the call, pre-quantized row-major and T16)."""
    N = 256
    w, codes, x = _decode_weights(E4M3), _decode_codes(N, layout), _onehot_x()
    oq, oc = oracle.quant_act(x, OCP)
    ref = oracle.linear(E4M3, layout, N, KX, w, codes, NCODES, MXFP8, xq=oq, xcodes=oc)
    wp, cp = g.pack(E4M3, layout, 1, N, KX, w, codes)
    _values_equal(g.linear(E4M3, layout, N, KX, wp, cp, MXFP8, x=x, rule=OCP), ref, "gemm decode")
    for m0 in range(0, NCODES, 64):
        xs = x[m0:m0 + 64]
        rs = ref[m0:m0 + 64]
        _values_equal(g.linear(E4M3, layout, N, KX, wp, cp, MXFP8, x=xs, rule=OCP), rs,
                      f"gemv decode (in call) tokens {m0}..")
        _values_equal(g.linear(E4M3, layout, N, KX, wp, cp, MXFP8, xq=oq[m0:m0 + 64],
                               xcodes=oc[m0:m0 + 64]), rs, f"gemv decode (row-major) {m0}..")
        qd, qc = g.quant_t16(xs, OCP)
        _values_equal(g.linear(E4M3, layout, N, KX, wp, cp, MXFP8_T16, xq=qd, xcodes=qc,
                               M=len(xs)), rs, f"gemv decode (T16) {m0}..")
