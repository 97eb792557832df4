"""GPU-side helpers for the parity tests: move numpy inputs to the device,
call libmx through its binding, bring results back, and apply the accuracy
bar for bf16 outputs.  No arithmetic of the layer lives here."""
from __future__ import annotations

import numpy as np
import torch

import microscaling_quantized_linear_amd as mx
from microscaling_quantized_linear_amd import workloads as wl

DEV = "cuda:0"

# accuracy bar for bf16 outputs against the fp64 oracle
REL_L2 = 2e-3          # ||y - ref||_2 / ||ref||_2
ROW_FRAC = 1e-2        # |y - ref| <= ROW_FRAC * max |ref row|


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def pack(elem, layout, E, N, K, w: np.ndarray, codes: np.ndarray):
    wb, cb = mx.mx_packed_sizes(elem, layout, E, N, K)
    wp = torch.empty(wb, dtype=torch.uint8, device=DEV)
    cp = torch.empty(cb, dtype=torch.uint8, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    mx.mx_pack_weights(elem, layout, E, N, K, dev(w), dev(codes), wp, cp, ws, 256)
    return wp, cp


def quant(x: np.ndarray, rule: int, ldq: int | None = None):
    M, K = x.shape
    ldq = ldq or (K + 15) // 16 * 16
    xd = dev(x)
    xq = torch.zeros((M, ldq), dtype=torch.uint8, device=DEV)
    xc = torch.zeros((M, K // 32), dtype=torch.uint8, device=DEV)
    mx.mx_quant_act(M, K, xd, K, xq, ldq, xc, K // 32, rule)
    torch.cuda.synchronize()
    return xq.cpu().numpy()[:, :K], xc.cpu().numpy()


def quant_t16(x: np.ndarray, rule: int):
    """mx_quant_act_t16 of bf16 bits x [M, K]: the two device buffers."""
    M, K = x.shape
    qb, cb = mx.mx_act_t16_sizes(M, K)
    xq = torch.full((qb,), 0xAB, dtype=torch.uint8, device=DEV)   # every byte must be written
    xc = torch.full((cb,), 0xCD, dtype=torch.uint8, device=DEV)
    mx.mx_quant_act_t16(M, K, dev(x), K, xq, xc, rule)
    torch.cuda.synchronize()
    return xq, xc


def t16_unpack(xq: np.ndarray, xc: np.ndarray, M: int, K: int):
    """The T16 layout as a reshape: data [MB][S][h][j][r][c] -> token 16 mb + r,
    K 128 s + 64 h + 16 j + c; codes [MB][Q][j][r][u] -> token 16 mb + r, block
    4 (4 q + u) + j.  Returns the padded row-major arrays [16 MB, 128 S] and
    [16 MB, 16 Q]."""
    S = -(-K // 128)
    Q = -(-S // 4)
    MB = -(-M // 16)
    d = xq.reshape(MB, S, 2, 4, 16, 16).transpose(0, 4, 1, 2, 3, 5).reshape(MB * 16, S * 128)
    c = xc.reshape(MB, Q, 4, 16, 4).transpose(0, 3, 1, 4, 2).reshape(MB * 16, Q * 16)
    return d, c


def linear(elem, layout, N, K, wp, cp, act, x=None, xq=None, xcodes=None, rule=0, bias=None,
           M=None):
    """Run mx_linear; x is bf16 bits [M, K] (quantized inside the call when
    act is MXFP8 and xq is None) or (xq, xcodes) pre-quantized: host arrays
    row-major, or the device buffers of quant_t16 when act is MXFP8_T16 (then
    M is given)."""
    if M is None:
        M = x.shape[0] if x is not None else xq.shape[0]
    y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    xd = dev(x) if x is not None else None
    xqd = xcd = None
    ldq = ldc = 0
    if act == mx.MX_ACT_MXFP8_T16:
        xqd, xcd = xq, xcodes                       # device buffers of quant_t16
    elif xq is not None:
        ldq = (K + 15) // 16 * 16
        buf = np.zeros((M, ldq), np.uint8)
        buf[:, :K] = xq
        xqd, xcd, ldc = dev(buf), dev(xcodes), xcodes.shape[1]
    need = mx.mx_linear_workspace(elem, layout, N, K, M, act, xq is not None)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    bd = dev(bias) if bias is not None else None
    mx.mx_linear(elem, layout, N, K, wp, cp, M, act, rule, xd, K if x is not None else 0,
                 xqd, ldq, xcd, ldc, bd, y, N, ws, need)
    torch.cuda.synchronize()
    return host_u16(y)


def moe(elem, E, N, K, wp, cp, x, ids, weights=None):
    T, topk = ids.shape
    combine = weights is not None
    y = torch.empty((T, N) if combine else (T, topk, N), dtype=torch.int16, device=DEV)
    need = mx.mx_moe_workspace(elem, E, N, K, T, topk, combine)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    mx.mx_moe_linear(elem, E, N, K, wp, cp, T, topk, dev(x), K, dev(ids),
                     dev(weights) if combine else None, y, ws, need)
    torch.cuda.synchronize()
    return host_u16(y)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def rounding_floor(ref: np.ndarray) -> float:
    """Relative L2 error of the exact result rounded once to bf16: no bf16
    output can do better (torch's float64 -> bfloat16 cast, nearest-even)."""
    r = torch.from_numpy(np.ascontiguousarray(ref)).to(torch.bfloat16).double().numpy()
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(r - ref) / n) if n > 0 else 0.0


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def assert_close(y_bits: np.ndarray, ref: np.ndarray, what: str = "", strict: bool = False):
    """The bar: relative L2 <= 2e-3 and every |err| <= 1e-2 * max|oracle row|.

    strict: the relative-L2 bar holds as stated, with no fallback (the
    full-size workloads have enough outputs that the rounding floor sits
    well below 2e-3).

    Where the exact result rounded once to bf16 does not itself reach the
    2e-3 bar (cases with few outputs: the rounding floor of the relative L2
    is then >= 1.9e-3), the relative-L2 test is replaced by a per-element one:
    every output within one bf16 ulp of the exact result (the correctly
    rounded value or its neighbour), or within 2^-12 of its row's largest
    magnitude -- for outputs whose accuracy is set by the fp32 accumulation of
    their inputs rather than by the output rounding (tiny values, e.g. SiLU of
    a very negative gate, where e^g amplifies the gate's absolute error); the
    contract's own per-element bound is 1e-2 of the row's largest magnitude."""
    y = bf16_to_f64(y_bits).reshape(ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = y - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    if rel > REL_L2:
        assert not strict, f"{what}: relative L2 {rel:.3e} > {REL_L2}"
        floor = rounding_floor(ref)
        assert floor >= 0.95 * REL_L2, f"{what}: relative L2 {rel:.3e} > {REL_L2} (floor {floor:.3e})"
        rowmax1 = np.abs(ref.reshape(-1, ref.shape[-1])).max(axis=1, keepdims=True)
        noise = np.broadcast_to(rowmax1, ref.reshape(-1, ref.shape[-1]).shape).reshape(ref.shape)
        far = np.abs(err) > np.maximum(bf16_ulp(ref), 2.0 ** -12 * noise)
        assert not far.any(), f"{what}: {far.sum()} outputs more than one bf16 ulp off"
    r2 = ref.reshape(-1, ref.shape[-1])
    e2 = np.abs(err.reshape(-1, ref.shape[-1]))
    rowmax = np.abs(r2).max(axis=1, keepdims=True)
    bad = e2 > ROW_FRAC * rowmax
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond 1e-2 * row max"
    return rel


def moe_copies(elem, E, Np, inter, K, H, w13, s13, w2, s2):
    """mx_moe_copies of host arrays: the four outputs as host arrays."""
    rowb = K // 2 if elem == 1 else K
    r2 = inter // 2 if elem == 1 else inter
    outs = [torch.full(shape, 0xAB, dtype=torch.uint8, device=DEV)
            for shape in ((E, 2 * inter, rowb), (E, 2 * inter, K // 32), (E, H, r2),
                          (E, H, inter // 32))]
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    mx.mx_moe_copies(elem, E, Np, inter, K, H, dev(w13), dev(s13), dev(w2), dev(s2), *outs, ws,
                     256)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def moe_gate_up(elem, E, inter, K, wp, cp, x, ids, ldh=None):
    T, topk = ids.shape
    ldh = ldh or inter
    h = torch.full((T * topk, ldh), 0x7FC0, dtype=torch.int16, device=DEV)
    mx.mx_moe_gate_up(elem, E, inter, K, wp, cp, T, topk, dev(x), x.shape[1], dev(ids), h, ldh)
    torch.cuda.synchronize()
    return host_u16(h)[:, :inter]


def moe_down(elem, E, H, inter, wp, cp, h, ids, weights=None):
    T, topk = ids.shape
    combine = weights is not None
    y = torch.empty((T, H) if combine else (T, topk, H), dtype=torch.int16, device=DEV)
    need = mx.mx_moe_workspace(elem, E, H, inter, T, topk, combine)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    hd = dev(np.ascontiguousarray(h.reshape(T * topk, -1)))
    mx.mx_moe_down(elem, E, H, inter, wp, cp, T, topk, hd, hd.shape[1], dev(ids),
                   dev(weights) if combine else None, y, ws, need)
    torch.cuda.synchronize()
    return host_u16(y)
