"""CPU-side tests of libmx: the library loads, exports every entry point that
include/mx.h declares, sizes packed buffers like the oracle's layout
definition, and rejects bad arguments with the documented status before any
device work (no GPU is needed for any of these)."""
import ctypes as C
import os
import re

import pytest

import microscaling_quantized_linear_amd as mx
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, ALIGN, VALUE, UNSUP, DEVICE, WS, LAUNCH = range(9)


def _declared():
    src = open(os.path.join(ROOT, "include", "mx.h")).read()
    return sorted(set(re.findall(r"^\s*(?:mx_status|const char \*|int)\s*\**\s*(mx_\w+)\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"mx_pack_weights", "mx_quant_act", "mx_linear", "mx_moe_linear"} <= set(names)
    L = mx.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(9):
        assert mx.mx_status_str(s)
    assert mx.mx_status_str(77) == "unknown status"


def test_arch_gate_strings():
    assert mx.mx_arch_supported("gfx950")
    assert mx.mx_arch_supported("gfx950:sramecc+:xnack-")
    for bad in ("gfx942", "gfx942:sramecc+:xnack-", "gfx9500", "gfx90a", "", "sm_90"):
        assert not mx.mx_arch_supported(bad)


@pytest.mark.parametrize("elem,layout,E,N,K", [
    (0, 0, 1, 256, 512), (0, 1, 1, 7168, 7168), (0, 0, 1, 4096, 1568),
    (1, 0, 32, 3072, 3072), (1, 0, 2, 16, 160), (0, 1, 3, 64, 96)])
def test_packed_sizes_match_oracle_layout(elem, layout, E, N, K):
    assert mx.mx_packed_sizes(elem, layout, E, N, K) == oracle.packed_sizes(elem, layout, E, N, K)


def _status(fn, *args):
    return getattr(mx.lib(), fn)(*args)


def test_shape_and_enum_errors():
    wb, cb = C.c_size_t(), C.c_size_t()
    L = mx.lib()
    assert L.mx_packed_sizes(0, 0, 1, 24, 512, C.byref(wb), C.byref(cb)) == SHAPE
    assert L.mx_packed_sizes(0, 1, 1, 48, 512, C.byref(wb), C.byref(cb)) == SHAPE
    assert L.mx_packed_sizes(0, 0, 1, 32, 100, C.byref(wb), C.byref(cb)) == SHAPE
    assert L.mx_packed_sizes(0, 0, 0, 32, 128, C.byref(wb), C.byref(cb)) == SHAPE
    assert L.mx_packed_sizes(2, 0, 1, 32, 128, C.byref(wb), C.byref(cb)) == UNSUP
    assert L.mx_packed_sizes(0, 5, 1, 32, 128, C.byref(wb), C.byref(cb)) == UNSUP
    assert L.mx_packed_sizes(0, 0, 1, 32, 128, None, C.byref(cb)) == NULL


A = 1 << 20          # fake, 16-byte aligned "device" addresses: never dereferenced


def _linear(**kw):
    a = dict(elem=0, layout=0, N=64, K=256, w=A, c=A, M=4, act=0, rule=0, x=A, ldx=256,
             xq=None, ldq=0, xc=None, ldc=0, bias=None, y=A, ldy=64, ws=None, wsb=0)
    a.update(kw)
    return mx.lib().mx_linear(a["elem"], a["layout"], a["N"], a["K"], a["w"], a["c"], a["M"],
                              a["act"], a["rule"], a["x"], a["ldx"], a["xq"], a["ldq"], a["xc"],
                              a["ldc"], a["bias"], a["y"], a["ldy"], a["ws"], a["wsb"], None)


def test_linear_validation_paths():
    assert _linear(N=40) == SHAPE
    assert _linear(K=100) == SHAPE
    assert _linear(M=0) == SHAPE
    assert _linear(ldx=128) == SHAPE
    assert _linear(ldy=32) == SHAPE
    assert _linear(layout=1, N=48) == SHAPE
    assert _linear(elem=1, act=1) == UNSUP
    assert _linear(elem=1, layout=1) == UNSUP
    assert _linear(act=3) == UNSUP
    # T16 activations: both buffers required, 16-byte aligned
    assert _linear(act=2) == NULL
    assert _linear(act=2, x=None, xq=A, xc=A + 4) == ALIGN
    assert _linear(rule=3) == UNSUP
    assert _linear(x=None) == NULL
    assert _linear(y=None) == NULL
    assert _linear(w=A + 8) == ALIGN
    assert _linear(x=A + 4) == ALIGN
    assert _linear(ldx=260) == ALIGN
    assert _linear(ldy=68) == ALIGN
    assert _linear(bias=A + 1) == ALIGN
    # W8A8 quantized in the call needs a workspace
    assert _linear(act=1) == WS
    need = mx.mx_linear_workspace(0, 0, 64, 256, 4, 1, 0)
    assert need >= 4 * 256 + 4 * 8
    assert _linear(act=1, ws=A, wsb=need - 1) == WS
    # pre-quantized activations: strides checked; the decode GEMV needs no
    # workspace for them, nor for bf16 activations
    assert _linear(act=1, x=None, xq=A, ldq=256, xc=A, ldc=4) == SHAPE
    assert _linear(act=1, x=None, xq=A, ldq=264, xc=A, ldc=8) == ALIGN
    assert mx.mx_linear_workspace(0, 0, 64, 256, 4, 1, 1) == 0
    assert mx.mx_linear_workspace(0, 0, 64, 256, 4, 0, 0) == 0
    # the prefill GEMM restages the activation codes even when pre-quantized
    assert mx.mx_linear_workspace(0, 0, 64, 256, 65, 1, 1) > 0
    # quantization inside the decode GEMV (K % 128 == 0, S = K / 128 in
    # {8, 16, 32, 56, 64}, even tiles): no workspace
    for layout, N, K, M in [(1, 7168, 7168, 16), (0, 256, 1024, 4), (1, 64, 8192, 64),
                            (0, 96, 2048, 1)]:
        assert mx.mx_linear_workspace(0, layout, N, K, M, 1, 0) == 0, (layout, N, K, M)
    # K = 1536 (S = 12) and K = 1568 (ragged) stay with a quantization launch
    assert mx.mx_linear_workspace(0, 1, 256, 1536, 4, 1, 0) > 0
    assert mx.mx_linear_workspace(0, 0, 256, 1568, 4, 1, 0) > 0
    # a valid call on a machine without a gfx950 device stops at the gate
    import torch
    if not torch.cuda.is_available():
        assert _linear() == DEVICE
        assert _linear(act=1, x=None, xq=A, ldq=256, xc=A, ldc=8) == DEVICE


def test_t16_sizes_and_quant_validation():
    # S = ceil(K / 128) steps, Q = ceil(S / 4), MB = ceil(M / 16)
    for M, K in [(1, 128), (16, 7168), (17, 160), (64, 1568)]:
        S = -(-K // 128)
        Q = -(-S // 4)
        MB = -(-M // 16)
        assert mx.mx_act_t16_sizes(M, K) == (MB * S * 2048, MB * Q * 256)
    L = mx.lib()
    qb, cb = C.c_size_t(), C.c_size_t()
    assert L.mx_act_t16_sizes(0, 128, C.byref(qb), C.byref(cb)) == SHAPE
    assert L.mx_act_t16_sizes(4, 100, C.byref(qb), C.byref(cb)) == SHAPE
    assert L.mx_act_t16_sizes(4, 128, None, C.byref(cb)) == NULL
    assert L.mx_quant_act_t16(4, 128, A, 120, A, A, 0, None) == SHAPE
    assert L.mx_quant_act_t16(4, 128, None, 128, A, A, 0, None) == NULL
    assert L.mx_quant_act_t16(4, 128, A, 128, A, A + 8, 0, None) == ALIGN
    assert L.mx_quant_act_t16(4, 128, A, 128, A, A, 5, None) == UNSUP


def test_quant_and_pack_and_moe_validation_paths():
    L = mx.lib()
    assert L.mx_quant_act(4, 100, A, 128, A, 128, A, 4, 0, None) == SHAPE
    assert L.mx_quant_act(4, 128, A, 120, A, 128, A, 4, 0, None) == SHAPE
    assert L.mx_quant_act(4, 128, A, 136, A, 136, A, 4, 0, None) == ALIGN
    assert L.mx_quant_act(4, 128, None, 128, A, 128, A, 4, 0, None) == NULL
    assert L.mx_quant_act(4, 128, A, 128, A, 128, A, 4, 9, None) == UNSUP
    assert L.mx_pack_weights(0, 0, 1, 32, 128, A, A, A, A, A, 255, None) == WS
    assert L.mx_pack_weights(0, 0, 1, 32, 128, A, A, A + 4, A, A, 256, None) == ALIGN
    assert L.mx_pack_weights(0, 0, 1, 32, 128, A, None, A, A, A, 256, None) == NULL

    def moe(**kw):
        a = dict(elem=1, E=8, N=64, K=256, w=A, c=A, T=4, topk=2, x=A, ldx=256, ids=A,
                 wts=None, y=A, ws=None, wsb=0)
        a.update(kw)
        return L.mx_moe_linear(a["elem"], a["E"], a["N"], a["K"], a["w"], a["c"], a["T"],
                               a["topk"], a["x"], a["ldx"], a["ids"], a["wts"], a["y"], a["ws"],
                               a["wsb"], None)
    assert moe(topk=9) == SHAPE
    assert moe(T=4097, topk=1) == SHAPE
    assert moe(N=40) == SHAPE
    assert moe(ids=None) == NULL
    assert moe(ids=A + 2) == ALIGN
    assert moe(wts=A) == WS
    assert mx.mx_moe_workspace(1, 8, 64, 256, 4, 2, 1) == 4 * 2 * 64 * 4
    import torch
    if not torch.cuda.is_available():
        assert moe() == DEVICE


def test_moe_block_validation_paths():
    L = mx.lib()

    def cop(**kw):
        a = dict(elem=1, E=2, Np=96, inter=64, K=128, H=32, ws=A, wsb=256)
        a.update(kw)
        return L.mx_moe_copies(a["elem"], a["E"], a["Np"], a["inter"], a["K"], a["H"], A, A, A, A,
                               A, A, A, A, a["ws"], a["wsb"], None)
    assert cop(inter=48) == SHAPE            # inter % 32
    assert cop(inter=128) == SHAPE           # inter > Np
    assert cop(K=100) == SHAPE
    assert cop(elem=3) == UNSUP
    assert cop(ws=None) == NULL
    assert cop(wsb=100) == WS

    def gu(**kw):
        a = dict(elem=1, E=8, inter=64, K=256, T=4, topk=2, ldx=256, h=A, ldh=64)
        a.update(kw)
        return L.mx_moe_gate_up(a["elem"], a["E"], a["inter"], a["K"], A, A, a["T"], a["topk"],
                                A, a["ldx"], A, a["h"], a["ldh"], None)
    assert gu(ldh=32) == SHAPE               # ldh < inter
    assert gu(ldh=68) == ALIGN
    assert gu(inter=12) == SHAPE
    assert gu(h=None) == NULL
    assert gu(topk=9) == SHAPE

    def dn(**kw):
        a = dict(elem=1, E=8, H=64, inter=256, T=4, topk=2, ldh=256, wts=None, ws=None, wsb=0)
        a.update(kw)
        return L.mx_moe_down(a["elem"], a["E"], a["H"], a["inter"], A, A, a["T"], a["topk"], A,
                             a["ldh"], A, a["wts"], A, a["ws"], a["wsb"], None)
    assert dn(ldh=128) == SHAPE              # ldh < inter (K of the down projection)
    assert dn(wts=A) == WS                   # combined needs the workspace
    assert dn(H=40) == SHAPE
    import torch
    if not torch.cuda.is_available():
        assert cop() == DEVICE and gu() == DEVICE and dn() == DEVICE


def test_ingest_validation_paths():
    L = mx.lib()

    def fold(**kw):
        a = dict(N=64, K=128, ldc=4, out=A, ws=A, wsb=256)
        a.update(kw)
        return L.mx_fold_row_codes(a["N"], a["K"], A, a["ldc"], a["out"], a["ws"], a["wsb"], None)
    assert fold(N=48) == SHAPE               # N % 32
    assert fold(K=100) == SHAPE
    assert fold(ldc=3) == SHAPE              # ldc < K / 32
    assert fold(out=None) == NULL
    assert fold(wsb=16) == WS

    def rec(**kw):
        a = dict(layout=1, N=64, K=128, ldw=128, out=A, ws=A, wsb=256)
        a.update(kw)
        return L.mx_e4m3_from_dequant(a["layout"], a["N"], a["K"], A, a["ldw"], A, a["out"],
                                      a["ws"], a["wsb"], None)
    assert rec(layout=2) == UNSUP
    assert rec(N=48) == SHAPE                # BLK32 needs N % 32
    assert rec(K=96 + 8) == SHAPE
    assert rec(ldw=120) == SHAPE             # ldw < K
    assert rec(ldw=132) == ALIGN             # ldw % 8
    assert rec(out=None) == NULL
    assert rec(wsb=0) == WS
    import torch
    if not torch.cuda.is_available():
        assert fold() == DEVICE and rec() == DEVICE and rec(layout=0, N=48) == DEVICE


def test_batch_invariant_switch_and_workspace():
    """The mode switch returns the previous setting; with it on, a
    row-major pre-quantized W8A8 call above 64 rows needs no restaging
    workspace (it runs the GEMV, not the GEMM)."""
    prev = mx.mx_set_batch_invariant(False)
    try:
        assert mx.mx_linear_workspace(0, 1, 512, 1024, 200, 1, True) > 0
        assert mx.mx_linear_workspace(0, 1, 512, 1024, 64, 1, True) == 0
        assert mx.mx_set_batch_invariant(True) is False
        assert mx.mx_linear_workspace(0, 1, 512, 1024, 200, 1, True) == 0
        # in-call quantization: the T16 staging either way
        assert mx.mx_linear_workspace(0, 1, 512, 1024, 200, 1, False) > 0
        assert mx.mx_set_batch_invariant(True) is True
    finally:
        mx.mx_set_batch_invariant(prev)


def test_fused_layout_validation_paths():
    L = mx.lib()

    def perm(**kw):
        a = dict(kind=0, layout=0, N=128, K=256, heads=4, out=A)
        a.update(kw)
        return L.mx_fused_layout_permute(a["kind"], a["layout"], a["N"], a["K"], a["heads"], A,
                                         A, a["out"], A, None)
    assert perm(kind=2) == UNSUP
    assert perm(layout=1) == UNSUP           # Q rows need per-row codes
    assert perm(heads=3) == SHAPE            # N % heads
    assert perm(N=96, heads=4) == SHAPE      # D = 24: not a multiple of 16
    assert perm(kind=1, heads=16) == SHAPE   # D = 16: not a multiple of 32
    assert perm(kind=1, layout=1, N=48, heads=4) == SHAPE
    assert perm(K=100) == SHAPE
    assert perm(out=None) == NULL
    import torch
    if not torch.cuda.is_available():
        assert perm() == DEVICE and perm(kind=1, layout=1) == DEVICE


def test_binding_raises_without_touching_the_device():
    with pytest.raises(mx.MXError) as ei:
        mx.mx_packed_sizes(0, 0, 1, 24, 512)
    assert ei.value.status == SHAPE


def test_fused_quant_kill_switch():
    """MX_FUSED_QUANT=0 (read once per process) turns off the quantization
    inside the decode GEMV: the same call then stages the T16 activation in
    the workspace (a quantization launch before the GEMV, whose output the
    GPU tests hold equal to the fused one bit for bit)."""
    import subprocess
    import sys
    args = (0, 1, 7168, 7168, 16, 1, False)         # W8A8 BLK32, M=16, bf16 input
    assert mx.mx_linear_workspace(*args) == 0
    code = ("import microscaling_quantized_linear_amd as mx; "
            f"print(mx.mx_linear_workspace(*{args!r}))")
    env = dict(os.environ, MX_FUSED_QUANT="0")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=120, check=True).stdout
    t16 = 16 * 7168 + 16 * (7168 // 32)                # one 16-token tile of bytes and codes
    assert int(out.strip().splitlines()[-1]) >= t16


def test_noalloc_moe_refuses_combine_beyond_its_buffer():
    """mx_moe_linear_noalloc: the combine's per-slot sums must fit the
    library's 4 MiB buffer (T * topk * N <= 2^20 fp32), checked on the host
    before any device call; shape errors come first, as in mx_moe_linear."""
    L = mx.lib()
    f = C.c_float(1.0)
    # 512 tokens x top-8 x 3072 outputs x 4 bytes = 48 MiB
    assert L.mx_moe_linear_noalloc(1, 32, 3072, 3072, None, None, 512, 8, None, 3072, None,
                                   C.byref(f), None, None) == WS
    # exactly 2^20 floats would pass the size check (then fail on NULL pointers)
    assert L.mx_moe_linear_noalloc(1, 32, 4096, 3072, None, None, 32, 8, None, 3072, None,
                                   C.byref(f), None, None) == NULL
    assert L.mx_moe_linear_noalloc(1, 32, 4096, 3072, None, None, 33, 8, None, 3072, None,
                                   C.byref(f), None, None) == WS
    # per-slot mode uses no buffer: only the NULL pointers are refused
    assert L.mx_moe_linear_noalloc(1, 32, 3072, 3072, None, None, 512, 8, None, 3072, None,
                                   None, None, None) == NULL
    assert L.mx_moe_linear_noalloc(1, 32, 3072, 100, None, None, 16, 8, None, 3072, None,
                                   None, None, None) == SHAPE
