"""Pins of the oracle's load-time packs (CPU only).

The oracle writes each pack as a loop over destination offsets.  Here the same
layouts are stated a second, independent way -- as numpy reshape/transpose of
the padded standard tensors, the style in which the pages state their own
repacks (vllm.models.deepseek_v41.amd.mono.weights942: dense_copy,
fp4_tile_major, codes_tile_rounds), with each tile's bytes then cut to 16 row
lengths (the padding of a K % 128 tail sits past the valid prefix of the
tile's last chunk and is not stored) -- and the weight pack is checked to be
a permutation of the unpadded input (packed = standard[perm], the identity
that vllm.models.deepseek_v41.common.ops.fused_layout builds its
permutations on), the codes to carry padding code 128, and the 16 bytes
after the codes to hold the smallest and largest given code.
"""
import numpy as np
import pytest

import oracle
from microscaling_quantized_linear_amd import workloads as wl

E4M3, E2M1, ROW32, BLK32 = oracle.E4M3, oracle.E2M1, oracle.ROW32, oracle.BLK32


def _pad_cols(a, n, value):
    out = np.full(a.shape[:-1] + (n,), value, a.dtype)
    out[..., : a.shape[-1]] = a
    return out


def _ref_weights(elem, E, N, K, w):
    Kp = -(-K // 128) * 128
    S, T = Kp // 128, N // 16
    if elem == E4M3:
        v = _pad_cols(w.reshape(E, N, K), Kp, 0).reshape(E, T, 16, S, 2, 4, 16)
        v = v.transpose(0, 1, 3, 4, 5, 2, 6)                  # [e,t,s,h,j,r,c]
        tileb = 16 * K
    else:
        v = _pad_cols(w.reshape(E, N, K // 2), Kp // 2, 0).reshape(E, T, 16, S, 4, 16)
        v = v.transpose(0, 1, 3, 4, 2, 5)                     # [e,t,s,j,r,c]
        tileb = 8 * K
    # per tile, the padded bytes all lie past the first 16 row lengths
    v = v.reshape(E * T, -1)
    assert not v[:, tileb:].any() or K % 128 == 0
    return np.ascontiguousarray(v[:, :tileb]).reshape(-1)


def _trailer(codes):
    """16 bytes after the packed codes: the smallest and the largest given
    code, then zeros."""
    t = np.zeros(16, np.uint8)
    t[0], t[1] = codes.min(), codes.max()
    return t


def _ref_codes(layout, E, N, K, codes):
    Kp = -(-K // 128) * 128
    S, T = Kp // 128, N // 16
    Q = -(-S // 4)
    if layout == ROW32:
        v = _pad_cols(codes.reshape(E * N, K // 32), 16 * Q, 128).reshape(E, T, 16, Q, 4, 4)
        body = v.transpose(0, 1, 3, 5, 2, 4).reshape(-1)      # [e,t,q,j,r,u]
    else:
        v = _pad_cols(codes.reshape(E * N // 32, K // 32), 16 * Q, 128).reshape(-1, Q, 4, 4)
        body = v.transpose(0, 1, 3, 2).reshape(-1)            # [R,q,j,u]
    return np.concatenate([body, _trailer(codes)])


SHAPES = [
    (E4M3, ROW32, 1, 32, 512),
    (E4M3, ROW32, 1, 48, 1568),     # K tail: Kp = 1664, S = 13
    (E4M3, BLK32, 1, 64, 1568),
    (E4M3, BLK32, 1, 96, 896),
    (E2M1, ROW32, 3, 32, 384),
    (E2M1, ROW32, 2, 16, 160),      # K tail for e2m1
    (E2M1, BLK32, 2, 32, 256),
]


@pytest.mark.parametrize("elem,layout,E,N,K", SHAPES)
def test_pack_matches_reshape_statement(elem, layout, E, N, K):
    g = np.random.default_rng([7, elem, layout, E, N, K])
    kb = K if elem == E4M3 else K // 2
    w = g.integers(0, 256, size=(E, N, kb), dtype=np.int32).astype(np.uint8)
    cshape = (E * N, K // 32) if layout == ROW32 else (E * N // 32, K // 32)
    codes = g.integers(0, 255, size=cshape, dtype=np.int32).astype(np.uint8)
    wp, cp = oracle.pack_weights(elem, layout, E, N, K, w, codes)
    np.testing.assert_array_equal(wp, _ref_weights(elem, E, N, K, w))
    np.testing.assert_array_equal(cp, _ref_codes(layout, E, N, K, codes))


def _labels(n):
    idx = np.arange(n, dtype=np.int64)
    return [((idx >> (8 * p)) & 0xFF).astype(np.uint8) for p in range(3)]


@pytest.mark.parametrize("elem,K", [(E4M3, 256), (E2M1, 256), (E4M3, 160), (E4M3, 224),
                                    (E4M3, 192), (E2M1, 160), (E2M1, 224)])
def test_weight_pack_is_a_permutation(elem, K):
    # no stored padding, also with a K % 128 tail: the pack is a bijection of
    # the standard bytes
    E, N = 2, 32
    kb = K if elem == E4M3 else K // 2
    n = E * N * kb
    codes = np.zeros((E * N, K // 32), np.uint8)
    src = np.zeros(n, np.int64)
    for p, plane in enumerate(_labels(n)):
        wp, _ = oracle.pack_weights(elem, ROW32, E, N, K, plane.reshape(E, N, kb), codes)
        assert wp.size == n
        src |= wp.astype(np.int64) << (8 * p)
    perm = src                                   # packed[i] = standard[perm[i]]
    assert np.array_equal(np.sort(perm), np.arange(n))
    # the inverse, built by scattering arange (the fused_layout construction)
    inv = np.empty(n, np.int64)
    inv[perm] = np.arange(n)
    std = np.random.default_rng(3).integers(0, 256, n).astype(np.uint8)
    wp, _ = oracle.pack_weights(elem, ROW32, E, N, K, std.reshape(E, N, kb), codes)
    np.testing.assert_array_equal(wp, std[perm])
    np.testing.assert_array_equal(wp[inv], std)
    # lane ownership: lane l = 16 j + r of chunk (t, s) reads row 16 t + r as
    # 16-byte pieces at 16 l (+ 1024): e4m3 K 16 j.. and 64 + 16 j.. of the
    # step, e2m1 the 32-value block j of the step; a tile is 16 row lengths
    S, T = -(-K // 128), N // 16
    chunk, tileb = (2048, 16 * K) if elem == E4M3 else (1024, 8 * K)
    for (e, t, s, l) in [(0, 0, 0, 0), (1, 1, 1, 63), (0, 1, 0, 17), (1, 0, 1, 40),
                         (1, 1, S - 1, 5), (0, 0, S - 1, 20)]:
        r, j = l % 16, l // 16
        base = (e * T + t) * tileb + s * chunk
        if elem == E4M3:
            row = std.reshape(E, N, K)[e, 16 * t + r]
            for h in range(2):
                k0 = 128 * s + 64 * h + 16 * j
                if k0 < K:
                    np.testing.assert_array_equal(
                        wp[base + 1024 * h + 16 * l: base + 1024 * h + 16 * l + 16],
                        row[k0: k0 + 16])
        else:
            b0 = 64 * s + 16 * j
            if b0 < K // 2:
                want = std.reshape(E, N, K // 2)[e, 16 * t + r, b0: b0 + 16]
                np.testing.assert_array_equal(wp[base + 16 * l: base + 16 * l + 16], want)


def test_row32_code_pack_is_a_permutation_and_lane_dwords():
    E, N, K = 1, 32, 1024          # S = 8, Q = 2: no padding
    n = E * N * (K // 32)
    w = np.zeros((E, N, K), np.uint8)
    src = np.zeros(n, np.int64)
    for p, plane in enumerate(_labels(n)):
        _, cp = oracle.pack_weights(E4M3, ROW32, E, N, K, w, plane.reshape(E * N, K // 32))
        np.testing.assert_array_equal(cp[-16:], _trailer(plane))
        src |= cp[:-16].astype(np.int64) << (8 * p)
    assert np.array_equal(np.sort(src), np.arange(n))
    # lane l's dword of quad q holds its row's codes of blocks 4 (4 q + u) + j
    rows, kc = np.divmod(src, K // 32)
    T, Q = N // 16, 2
    for t in range(T):
        for q in range(Q):
            for l in range(64):
                for u in range(4):
                    i = (t * Q + q) * 256 + 4 * l + u
                    assert rows[i] == 16 * t + l % 16
                    assert kc[i] == 4 * (4 * q + u) + l // 16


def test_no_weight_padding_and_codes_128():
    E, N, K = 1, 32, 1568
    Kp = 1664
    w = np.full((E, N, K), 0x11, np.uint8)
    codes = np.full((E * N, K // 32), 7, np.uint8)
    wp, cp = oracle.pack_weights(E4M3, ROW32, E, N, K, w, codes)
    assert Kp > K and wp.size == N * K            # the K tail stores no padding
    assert np.count_nonzero(wp == 0x11) == N * K
    S, Q = 13, 4
    assert cp.size == (N // 16) * Q * 256 + 16
    body, trailer = cp[:-16], cp[-16:]
    assert np.count_nonzero(body == 7) == N * (K // 32)
    assert np.count_nonzero(body == 128) == body.size - N * (K // 32)
    # the padding code 128 is not counted in the trailer's range
    np.testing.assert_array_equal(trailer, [7, 7] + [0] * 14)
    wb, cb = oracle.packed_sizes(E4M3, BLK32, 1, 64, K)
    w2 = np.full((1, 64, K), 0x22, np.uint8)
    c2 = np.full((2, K // 32), 9, np.uint8)
    c2[1, 5] = 0
    c2[0, 48] = 254
    wp2, cp2 = oracle.pack_weights(E4M3, BLK32, 1, 64, K, w2, c2)
    assert cp2.shape == (2 * Q * 16 + 16,) and cb == cp2.size
    # 49 real blocks per 32-row group, the other 15 of the 4 quads are padding
    assert np.count_nonzero(cp2[:-16] == 9) == 2 * (K // 32) - 2
    assert np.count_nonzero(cp2[:-16] == 128) == 2 * (16 * Q - K // 32)
    np.testing.assert_array_equal(cp2[-16:], [0, 254] + [0] * 14)


def test_pack_rejects_bad_shapes():
    for args in [(E4M3, ROW32, 1, 24, 512), (E4M3, BLK32, 1, 48, 512), (E4M3, ROW32, 1, 32, 100)]:
        with pytest.raises(ValueError):
            oracle.packed_sizes(*args)
