"""MX (OCP microscaling) quantized linear layer for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``include/mx.h`` (``libmx.so``, built
in-tree by :mod:`microscaling_quantized_linear_amd.build`).  The functions
here only marshal arguments: tensors are passed as device pointers, streams
as HIP stream handles, and every step of the computation runs in the HIP
kernels.  There is no fallback: if ``libmx.so`` is missing or a call fails,
an exception is raised.

Each function takes the same arguments as the C entry point of the same
name; a tensor argument may be a ``torch.Tensor`` (its ``data_ptr()`` is
used) or a raw integer pointer.  ``stream=None`` means torch's current
stream on the current device.
"""
from __future__ import annotations

import ctypes as C
import os

__all__ = [
    "MX_E4M3", "MX_E2M1", "MX_SCALE_ROW32", "MX_SCALE_BLK32", "MX_RULE_OCP",
    "MX_RULE_CEIL448", "MX_ACT_BF16", "MX_ACT_MXFP8", "MX_ACT_MXFP8_T16", "MXError", "lib",
    "mx_packed_sizes", "mx_pack_weights", "mx_quant_act", "mx_act_t16_sizes",
    "mx_quant_act_t16", "mx_linear_workspace",
    "mx_linear", "mx_moe_workspace", "mx_moe_linear", "mx_moe_copies", "mx_moe_gate_up",
    "mx_moe_down", "mx_fold_row_codes", "mx_e4m3_from_dequant", "mx_set_batch_invariant",
    "mx_fused_layout_permute", "MX_PERM_Q_ROWS", "MX_PERM_O_COLS", "mx_status_str",
    "mx_arch_supported",
]

MX_E4M3, MX_E2M1 = 0, 1
MX_SCALE_ROW32, MX_SCALE_BLK32 = 0, 1
MX_RULE_OCP, MX_RULE_CEIL448 = 0, 1
MX_ACT_BF16, MX_ACT_MXFP8, MX_ACT_MXFP8_T16 = 0, 1, 2
MX_PERM_Q_ROWS, MX_PERM_O_COLS = 0, 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmx.so")
_lib = None


class MXError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({mx_status_str(status)})")


def lib() -> C.CDLL:
    """Load libmx.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m microscaling_quantized_linear_amd.build`")
        L = C.CDLL(LIB_PATH)
        i64, i32, p, sz = C.c_int64, C.c_int, C.c_void_p, C.c_size_t
        L.mx_status_str.argtypes = [i32]
        L.mx_status_str.restype = C.c_char_p
        L.mx_arch_supported.argtypes = [C.c_char_p]
        L.mx_arch_supported.restype = i32
        L.mx_packed_sizes.argtypes = [i32, i32, i64, i64, i64, C.POINTER(sz), C.POINTER(sz)]
        L.mx_pack_weights.argtypes = [i32, i32, i64, i64, i64, p, p, p, p, p, sz, p]
        L.mx_quant_act.argtypes = [i64, i64, p, i64, p, i64, p, i64, i32, p]
        L.mx_act_t16_sizes.argtypes = [i64, i64, C.POINTER(sz), C.POINTER(sz)]
        L.mx_quant_act_t16.argtypes = [i64, i64, p, i64, p, p, i32, p]
        L.mx_linear_workspace.argtypes = [i32, i32, i64, i64, i64, i32, i32, C.POINTER(sz)]
        L.mx_linear.argtypes = [i32, i32, i64, i64, p, p, i64, i32, i32, p, i64, p, i64,
                                p, i64, p, p, i64, p, sz, p]
        L.mx_moe_workspace.argtypes = [i32, i64, i64, i64, i64, i64, i32, C.POINTER(sz)]
        L.mx_moe_linear.argtypes = [i32, i64, i64, i64, p, p, i64, i64, p, i64, p, p, p,
                                    p, sz, p]
        L.mx_moe_linear_noalloc.argtypes = [i32, i64, i64, i64, p, p, i64, i64, p, i64, p,
                                            p, p, p]
        L.mx_moe_copies.argtypes = [i32, i64, i64, i64, i64, i64, p, p, p, p, p, p, p, p, p,
                                    sz, p]
        L.mx_moe_gate_up.argtypes = [i32, i64, i64, i64, p, p, i64, i64, p, i64, p, p, i64, p]
        L.mx_moe_down.argtypes = [i32, i64, i64, i64, p, p, i64, i64, p, i64, p, p, p, p, sz,
                                  p]
        L.mx_set_batch_invariant.argtypes = [i32]
        L.mx_set_batch_invariant.restype = i32
        L.mx_fold_row_codes.argtypes = [i64, i64, p, i64, p, p, sz, p]
        L.mx_fused_layout_permute.argtypes = [i32, i32, i64, i64, i64, p, p, p, p, p]
        L.mx_e4m3_from_dequant.argtypes = [i32, i64, i64, p, i64, p, p, p, sz, p]
        for name in ("mx_packed_sizes", "mx_pack_weights", "mx_quant_act", "mx_act_t16_sizes",
                     "mx_quant_act_t16", "mx_linear_workspace", "mx_linear", "mx_moe_workspace",
                     "mx_moe_linear", "mx_moe_linear_noalloc", "mx_moe_copies",
                     "mx_moe_gate_up", "mx_moe_down",
                     "mx_fold_row_codes", "mx_e4m3_from_dequant", "mx_fused_layout_permute"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise MXError(status, where)


def mx_status_str(status: int) -> str:
    return lib().mx_status_str(int(status)).decode()


def mx_arch_supported(name: str) -> bool:
    return bool(lib().mx_arch_supported(name.encode()))


def mx_packed_sizes(elem, layout, E, N, K):
    wb, cb = C.c_size_t(), C.c_size_t()
    _check(lib().mx_packed_sizes(elem, layout, E, N, K, C.byref(wb), C.byref(cb)),
           "mx_packed_sizes")
    return wb.value, cb.value


def mx_pack_weights(elem, layout, E, N, K, w, codes, w_packed, codes_packed, ws, ws_bytes,
                    stream=None):
    _check(lib().mx_pack_weights(elem, layout, E, N, K, _ptr(w), _ptr(codes), _ptr(w_packed),
                                 _ptr(codes_packed), _ptr(ws), ws_bytes, _stream(stream)),
           "mx_pack_weights")


def mx_quant_act(M, K, x, ldx, xq, ldq, xcodes, ldc, rule, stream=None):
    _check(lib().mx_quant_act(M, K, _ptr(x), ldx, _ptr(xq), ldq, _ptr(xcodes), ldc, rule,
                              _stream(stream)), "mx_quant_act")


def mx_act_t16_sizes(M, K):
    qb, cb = C.c_size_t(), C.c_size_t()
    _check(lib().mx_act_t16_sizes(M, K, C.byref(qb), C.byref(cb)), "mx_act_t16_sizes")
    return qb.value, cb.value


def mx_quant_act_t16(M, K, x, ldx, xq, xcodes, rule, stream=None):
    _check(lib().mx_quant_act_t16(M, K, _ptr(x), ldx, _ptr(xq), _ptr(xcodes), rule,
                                  _stream(stream)), "mx_quant_act_t16")


def mx_linear_workspace(elem, layout, N, K, M, act, prequantized):
    b = C.c_size_t()
    _check(lib().mx_linear_workspace(elem, layout, N, K, M, act, int(prequantized), C.byref(b)),
           "mx_linear_workspace")
    return b.value


def mx_linear(elem, layout, N, K, w_packed, codes_packed, M, act, rule, x, ldx, xq, ldq,
              xcodes, ldc, bias, y, ldy, ws, ws_bytes, stream=None):
    _check(lib().mx_linear(elem, layout, N, K, _ptr(w_packed), _ptr(codes_packed), M, act, rule,
                           _ptr(x), ldx, _ptr(xq), ldq, _ptr(xcodes), ldc, _ptr(bias), _ptr(y),
                           ldy, _ptr(ws), ws_bytes, _stream(stream)), "mx_linear")


def mx_moe_workspace(elem, E, N, K, T, topk, combine):
    b = C.c_size_t()
    _check(lib().mx_moe_workspace(elem, E, N, K, T, topk, int(combine), C.byref(b)),
           "mx_moe_workspace")
    return b.value


def mx_moe_linear(elem, E, N, K, w_packed, codes_packed, T, topk, x, ldx, topk_ids,
                  topk_weights, y, ws, ws_bytes, stream=None):
    _check(lib().mx_moe_linear(elem, E, N, K, _ptr(w_packed), _ptr(codes_packed), T, topk,
                               _ptr(x), ldx, _ptr(topk_ids), _ptr(topk_weights), _ptr(y),
                               _ptr(ws), ws_bytes, _stream(stream)), "mx_moe_linear")


def mx_moe_linear_noalloc(elem, E, N, K, w_packed, codes_packed, T, topk, x, ldx, topk_ids,
                          topk_weights, y, stream=None):
    _check(lib().mx_moe_linear_noalloc(elem, E, N, K, _ptr(w_packed), _ptr(codes_packed), T,
                                       topk, _ptr(x), ldx, _ptr(topk_ids), _ptr(topk_weights),
                                       _ptr(y), _stream(stream)), "mx_moe_linear_noalloc")


def mx_moe_copies(elem, E, Np, inter, K, H, w13, s13, w2, s2, w13_out, s13_out, w2_out, s2_out,
                  ws, ws_bytes, stream=None):
    _check(lib().mx_moe_copies(elem, E, Np, inter, K, H, _ptr(w13), _ptr(s13), _ptr(w2),
                               _ptr(s2), _ptr(w13_out), _ptr(s13_out), _ptr(w2_out),
                               _ptr(s2_out), _ptr(ws), ws_bytes, _stream(stream)),
           "mx_moe_copies")


def mx_moe_gate_up(elem, E, inter, K, w13_packed, codes_packed, T, topk, x, ldx, topk_ids, h,
                   ldh, stream=None):
    _check(lib().mx_moe_gate_up(elem, E, inter, K, _ptr(w13_packed), _ptr(codes_packed), T,
                                topk, _ptr(x), ldx, _ptr(topk_ids), _ptr(h), ldh,
                                _stream(stream)), "mx_moe_gate_up")


def mx_moe_down(elem, E, H, inter, w2_packed, codes_packed, T, topk, h, ldh, topk_ids,
                topk_weights, y, ws, ws_bytes, stream=None):
    _check(lib().mx_moe_down(elem, E, H, inter, _ptr(w2_packed), _ptr(codes_packed), T, topk,
                             _ptr(h), ldh, _ptr(topk_ids), _ptr(topk_weights), _ptr(y),
                             _ptr(ws), ws_bytes, _stream(stream)), "mx_moe_down")


def mx_fold_row_codes(N, K, codes_row, ldc, codes_blk, ws, ws_bytes, stream=None):
    _check(lib().mx_fold_row_codes(N, K, _ptr(codes_row), ldc, _ptr(codes_blk), _ptr(ws),
                                   ws_bytes, _stream(stream)), "mx_fold_row_codes")


def mx_e4m3_from_dequant(layout, N, K, w_bf16, ldw, codes, w_out, ws, ws_bytes, stream=None):
    _check(lib().mx_e4m3_from_dequant(layout, N, K, _ptr(w_bf16), ldw, _ptr(codes), _ptr(w_out),
                                      _ptr(ws), ws_bytes, _stream(stream)),
           "mx_e4m3_from_dequant")


def mx_set_batch_invariant(on: bool) -> bool:
    """Turn the process-wide batch-invariant mode on or off; the previous setting."""
    return bool(lib().mx_set_batch_invariant(1 if on else 0))


def mx_fused_layout_permute(kind, layout, N, K, heads, w, codes, w_out, codes_out, stream=None):
    _check(lib().mx_fused_layout_permute(kind, layout, N, K, heads, _ptr(w), _ptr(codes),
                                         _ptr(w_out), _ptr(codes_out), _stream(stream)),
           "mx_fused_layout_permute")
