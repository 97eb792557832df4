"""Python view of the CPU oracle (oracle/mx_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product library.  It loads
``oracle/libmx_oracle.so`` (built with gcc by :func:`build`) and marshals numpy
arrays to it; every piece of arithmetic lives in the C file.

Arrays: e4m3/e2m1/code bytes are ``uint8``; bf16 values travel as their
``uint16`` bit patterns; results of the linear layers are ``float64``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mx_oracle.c")
# MX_ORACLE_LIB: another build of the same source (the sanitizer test runs the
# oracle's pins on an AddressSanitizer / UBSan build this way)
LIB = os.environ.get("MX_ORACLE_LIB") or os.path.join(HERE, "libmx_oracle.so")

E4M3, E2M1 = 0, 1
ROW32, BLK32 = 0, 1
RULE_OCP, RULE_CEIL448 = 0, 1
ACT_BF16, ACT_MXFP8 = 0, 1

_lib = None


def build(out: str | None = None, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP over rows);
    sanitize: an AddressSanitizer + UndefinedBehaviorSanitizer build (any
    finding aborts) written to `out`."""
    out = out or LIB
    flags = ["-O2"]
    if sanitize:
        flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=all"]
    cmd = ["gcc", *flags, "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall",
           "-o", out + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = C.CDLL(LIB)
        _declare(_lib)
    return _lib


def _declare(L):
    i64, i32, dbl = C.c_int64, C.c_int, C.c_double
    p = C.c_void_p
    L.orc_e4m3_value.argtypes = [i32]; L.orc_e4m3_value.restype = dbl
    L.orc_e2m1_value.argtypes = [i32]; L.orc_e2m1_value.restype = dbl
    L.orc_e8m0_value.argtypes = [i32]; L.orc_e8m0_value.restype = dbl
    L.orc_bf16_value.argtypes = [C.c_uint16]; L.orc_bf16_value.restype = dbl
    L.orc_e4m3_round.argtypes = [dbl]; L.orc_e4m3_round.restype = i32
    L.orc_act_code.argtypes = [dbl, i32]; L.orc_act_code.restype = i32
    L.orc_quant_act.argtypes = [i64, i64, p, i64, p, i64, p, i64, i32]
    L.orc_quant_act.restype = None
    L.orc_padded_k.argtypes = [i64]; L.orc_padded_k.restype = i64
    L.orc_packed_sizes.argtypes = [i32, i32, i64, i64, i64, p, p]
    L.orc_packed_sizes.restype = i32
    L.orc_pack_weights.argtypes = [i32, i32, i64, i64, i64, p, p, p, p]
    L.orc_pack_weights.restype = i32
    L.orc_weight.argtypes = [i32, i32, i64, i64, i64, p, p, i64, i64, i64]
    L.orc_weight.restype = dbl
    L.orc_linear.argtypes = [i32, i32, i64, i64, p, p, i64, i32, p, i64, p, i64,
                             p, i64, p, p]
    L.orc_linear.restype = None
    L.orc_linear_pairs.argtypes = [i32, i32, i64, i64, p, p, i32, p, i64, p, i64,
                                   p, i64, p, i64, p, p, p]
    L.orc_linear_pairs.restype = None
    L.orc_moe_linear.argtypes = [i32, i64, i64, i64, p, p, i64, i64, p, i64, p,
                                 p, p]
    L.orc_moe_linear.restype = None
    L.orc_moe_copies.argtypes = [i32, i64, i64, i64, i64, i64, p, p, p, p, p, p, p, p]
    L.orc_moe_copies.restype = i32
    L.orc_silu.argtypes = [dbl]; L.orc_silu.restype = dbl
    L.orc_bf16_round.argtypes = [dbl]; L.orc_bf16_round.restype = C.c_uint16
    L.orc_moe_gate_up.argtypes = [i32, i64, i64, i64, p, p, i64, i64, p, i64, p, p]
    L.orc_moe_gate_up.restype = None
    L.orc_moe_linear_rows.argtypes = [i32, i64, i64, i64, p, p, i64, i64, p, i64, p, p, p]
    L.orc_moe_linear_rows.restype = None
    L.orc_fold_row_codes.argtypes = [i64, i64, p, p]; L.orc_fold_row_codes.restype = i32
    L.orc_e4m3_from_dequant.argtypes = [i32, i64, i64, p, i64, p, p]
    L.orc_e4m3_from_dequant.restype = i64
    L.orc_q_fused_perm.argtypes = [i64, i64, p]; L.orc_q_fused_perm.restype = i32
    L.orc_o_fused_perm.argtypes = [i64, i64, p]; L.orc_o_fused_perm.restype = i32
    L.orc_fused_layout_permute.argtypes = [i32, i32, i64, i64, i64, p, p, p, p]
    L.orc_fused_layout_permute.restype = i32
    L.orc_threads.argtypes = []
    L.orc_threads.restype = i32
    L.orc_set_threads.argtypes = [i32]
    L.orc_set_threads.restype = i32


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


# --- scalar decoders ----------------------------------------------------

def e4m3_value(b: int) -> float:
    return lib().orc_e4m3_value(int(b))


def e2m1_value(n: int) -> float:
    return lib().orc_e2m1_value(int(n))


def e8m0_value(c: int) -> float:
    return lib().orc_e8m0_value(int(c))


def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(int(bits))


def e4m3_round(v: float) -> int:
    return lib().orc_e4m3_round(float(v))


def act_code(amax: float, rule: int) -> int:
    return lib().orc_act_code(float(amax), int(rule))


# --- array entry points ---------------------------------------------------

def quant_act(x_bits: np.ndarray, rule: int):
    """x_bits uint16 [M, K] (bf16 patterns) -> (xq uint8 [M, K], codes uint8 [M, K/32])."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    xq = np.zeros((M, K), np.uint8)
    codes = np.zeros((M, K // 32), np.uint8)
    lib().orc_quant_act(M, K, _ptr(x), K, _ptr(xq), K, _ptr(codes), K // 32, rule)
    return xq, codes


def padded_k(K: int) -> int:
    return lib().orc_padded_k(K)


def packed_sizes(elem, layout, E, N, K):
    wb, cb = C.c_int64(), C.c_int64()
    rc = lib().orc_packed_sizes(elem, layout, E, N, K, C.byref(wb), C.byref(cb))
    if rc:
        raise ValueError(f"shape not packable: elem={elem} layout={layout} E={E} N={N} K={K}")
    return wb.value, cb.value


def pack_weights(elem, layout, E, N, K, w, codes):
    """Standard bytes + codes -> (packed weight bytes, packed codes), 1-D uint8."""
    wb, cb = packed_sizes(elem, layout, E, N, K)
    w = _c(w, np.uint8)
    codes = _c(codes, np.uint8)
    wp = np.empty(wb, np.uint8)
    cp = np.empty(cb, np.uint8)
    rc = lib().orc_pack_weights(elem, layout, E, N, K, _ptr(w), _ptr(codes), _ptr(wp), _ptr(cp))
    if rc:
        raise ValueError("pack failed")
    return wp, cp


def weight(elem, layout, E, N, K, w, codes, e, n, k) -> float:
    w = _c(w, np.uint8)
    codes = _c(codes, np.uint8)
    return lib().orc_weight(elem, layout, E, N, K, _ptr(w), _ptr(codes), e, n, k)


def linear(elem, layout, N, K, w, codes, M, act, x=None, xq=None, xcodes=None, bias=None):
    """fp64 y [M, N] = a . Wf^T (+ bias); x bf16 bits [M, K] or (xq, xcodes)."""
    w = _c(w, np.uint8)
    codes = _c(codes, np.uint8)
    x = _c(x, np.uint16)
    xq = _c(xq, np.uint8)
    xcodes = _c(xcodes, np.uint8)
    bias = _c(bias, np.uint16)
    y = np.empty((M, N), np.float64)
    lib().orc_linear(elem, layout, N, K, _ptr(w), _ptr(codes), M, act,
                     _ptr(x), K, _ptr(xq), K, _ptr(xcodes), K // 32, _ptr(bias), _ptr(y))
    return y


def linear_pairs(elem, layout, N, K, w, codes, act, ms, ns, x=None, xq=None,
                 xcodes=None, bias=None):
    """fp64 y[ms[p], ns[p]] for each pair p."""
    w = _c(w, np.uint8)
    codes = _c(codes, np.uint8)
    x = _c(x, np.uint16)
    xq = _c(xq, np.uint8)
    xcodes = _c(xcodes, np.uint8)
    bias = _c(bias, np.uint16)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    out = np.empty(len(ms), np.float64)
    lib().orc_linear_pairs(elem, layout, N, K, _ptr(w), _ptr(codes), act,
                           _ptr(x), K, _ptr(xq), K, _ptr(xcodes), K // 32,
                           _ptr(bias), len(ms), _ptr(ms), _ptr(ns), _ptr(out))
    return out


def moe_linear(elem, E, N, K, w, codes, x, ids, weights=None):
    """fp64 per-slot y [T, topk, N], or combined [T, N] when weights is given."""
    w = _c(w, np.uint8)
    codes = _c(codes, np.uint8)
    x = _c(x, np.uint16)
    ids = _c(ids, np.int32)
    T, topk = ids.shape
    weights = _c(weights, np.float32)
    shape = (T, N) if weights is not None else (T, topk, N)
    y = np.empty(shape, np.float64)
    lib().orc_moe_linear(elem, E, N, K, _ptr(w), _ptr(codes), T, topk, _ptr(x),
                         x.shape[1], _ptr(ids), _ptr(weights), _ptr(y))
    return y


def moe_copies(elem, E, Np, inter, K, H, w13, s13, w2, s2):
    """The load-time expert copies: interleaved w13 [E, 2 inter, rowb] with
    codes [E, 2 inter, K/32], and w2 cut to [E, H, inter values] with codes
    [E, H, inter/32].  Raises ValueError when the weights' padding is not zero."""
    w13, s13, w2, s2 = (_c(a, np.uint8) for a in (w13, s13, w2, s2))
    rowb = K // 2 if elem == E2M1 else K
    r2 = inter // 2 if elem == E2M1 else inter
    ow13 = np.empty((E, 2 * inter, rowb), np.uint8)
    os13 = np.empty((E, 2 * inter, K // 32), np.uint8)
    ow2 = np.empty((E, H, r2), np.uint8)
    os2 = np.empty((E, H, inter // 32), np.uint8)
    rc = lib().orc_moe_copies(elem, E, Np, inter, K, H, _ptr(w13), _ptr(s13), _ptr(w2),
                              _ptr(s2), _ptr(ow13), _ptr(os13), _ptr(ow2), _ptr(os2))
    if rc == 1:
        raise ValueError("the expert padding is not zero")
    if rc:
        raise ValueError("bad shape")
    return ow13, os13, ow2, os2


def silu(v: float) -> float:
    return lib().orc_silu(float(v))


def bf16_round(v: float) -> int:
    return int(lib().orc_bf16_round(float(v)))


def bf16_round_array(a: np.ndarray) -> np.ndarray:
    """Elementwise orc_bf16_round, as uint16 bit patterns."""
    f = np.vectorize(lambda v: lib().orc_bf16_round(float(v)), otypes=[np.uint16])
    return f(np.asarray(a, np.float64))


def moe_gate_up(elem, E, inter, K, w13, codes, x, ids):
    """fp64 h [T, topk, inter] = silu(x . gate^T) * (x . up^T) over the
    interleaved expert rows (even row 2 i: gate row i; the odd row after it:
    up row i)."""
    w13 = _c(w13, np.uint8)
    codes = _c(codes, np.uint8)
    x = _c(x, np.uint16)
    ids = _c(ids, np.int32)
    T, topk = ids.shape
    h = np.empty((T, topk, inter), np.float64)
    lib().orc_moe_gate_up(elem, E, inter, K, _ptr(w13), _ptr(codes), T, topk, _ptr(x),
                          x.shape[1], _ptr(ids), _ptr(h))
    return h


def moe_linear_rows(elem, E, N, K, w, codes, a, ids, weights=None):
    """The grouped linear with one bf16 activation row per slot: a [T*topk, K]
    (or [T, topk, K]); fp64 per-slot [T, topk, N] or combined [T, N]."""
    w = _c(w, np.uint8)
    codes = _c(codes, np.uint8)
    ids = _c(ids, np.int32)
    T, topk = ids.shape
    a = _c(np.asarray(a).reshape(T * topk, -1), np.uint16)
    weights = _c(weights, np.float32)
    shape = (T, N) if weights is not None else (T, topk, N)
    y = np.empty(shape, np.float64)
    lib().orc_moe_linear_rows(elem, E, N, K, _ptr(w), _ptr(codes), T, topk, _ptr(a),
                              a.shape[1], _ptr(ids), _ptr(weights), _ptr(y))
    return y


def fold_row_codes(N, KB, codes_row):
    """[N/32, KB] block codes from row-expanded [N, KB] codes; ValueError when
    a block's 32 rows disagree (or N is not a multiple of 32)."""
    c = _c(codes_row, np.uint8)
    out = np.empty((N // 32, KB), np.uint8)
    rc = lib().orc_fold_row_codes(N, KB, _ptr(c), _ptr(out))
    if rc == 1:
        raise ValueError("row codes are not 32 x 32 blocks")
    if rc:
        raise ValueError("bad shape")
    return out


def e4m3_from_dequant(layout, N, K, w_bits, codes, strict=True):
    """e4m3 bytes [N, K] behind bf16 weights w_bits [N, >= K] (bit patterns)
    dequantized with `codes` (ROW32 [N, K/32] or BLK32 [N/32, K/32]).  With
    strict, ValueError when any weight does not come back exactly; else the
    bytes with 0xFF marking those weights."""
    w = _c(w_bits, np.uint16)
    c = _c(codes, np.uint8)
    out = np.empty((N, K), np.uint8)
    bad = lib().orc_e4m3_from_dequant(layout, N, K, _ptr(w), w.shape[1], _ptr(c), _ptr(out))
    if bad < 0:
        raise ValueError("bad shape")
    if strict and bad:
        raise ValueError(f"{bad} of {N * K} values are not e4m3 x scale")
    return out


def q_fused_perm(H, D):
    """perm with fused = standard[perm] for the attention kernel's Q layout."""
    perm = np.empty(H * D, np.int64)
    if lib().orc_q_fused_perm(H, D, _ptr(perm)):
        raise ValueError("D must be a multiple of 16")
    return perm


def o_fused_perm(G, D):
    """perm with fused = standard[perm] for the attention kernel's O layout."""
    perm = np.empty(G * D, np.int64)
    if lib().orc_o_fused_perm(G, D, _ptr(perm)):
        raise ValueError("D must be a multiple of 32")
    return perm


def fused_layout_permute(kind, layout, N, K, heads, w, codes):
    """Q rows (kind 0) or O columns (kind 1) of an MXFP8 weight [N, K] and
    its codes, in the attention kernel's layout."""
    w = _c(w, np.uint8)
    codes = _c(codes, np.uint8)
    wo = np.empty((N, K), np.uint8)
    co = np.empty_like(codes)
    rc = lib().orc_fused_layout_permute(kind, layout, N, K, heads, _ptr(w), _ptr(codes),
                                        _ptr(wo), _ptr(co))
    if rc:
        raise ValueError("shape or layout outside the permutation")
    return wo, co


def threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return lib().orc_threads()


def set_threads(n: int) -> int:
    """Run the oracle's loops on n OpenMP threads from now on; returns the
    previous count."""
    return lib().orc_set_threads(int(n))
