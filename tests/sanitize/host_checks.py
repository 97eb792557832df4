"""Drives every entry point of a host-only build of libmx (mx_api.cpp and
mx_plan.cpp with tests/sanitize/host_stubs.cpp standing in for the HIP
runtime and the kernel launchers) through valid and invalid arguments.

Run as a child process of tests/test_sanitizers.py, with the build made
under AddressSanitizer and UndefinedBehaviorSanitizer (any finding aborts
the process): python host_checks.py <path of the host build>.
Test infrastructure; the stubs never touch the fake device addresses."""
import ctypes as C
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import microscaling_quantized_linear_amd as mx  # noqa: E402

mx.LIB_PATH = sys.argv[1]
L = mx.lib()
launches = C.c_long.in_dll(L, "mx_stub_launches")

OK, NULL, SHAPE, ALIGN, VALUE, UNSUP, DEVICE, WS, LAUNCH = range(9)
E4M3, E2M1, ROW32, BLK32 = 0, 1, 0, 1
BF16, MXFP8, T16 = 0, 1, 2
calls = 0


def dev(i):
    """A distinct fake device address, 256-byte aligned."""
    return (i + 1) << 28


def expect(got, want, what):
    global calls
    calls += 1
    assert got == want, f"{what}: status {got}, expected {want}"


def sizes(elem, layout, E, N, K):
    wb, cb = C.c_size_t(), C.c_size_t()
    st = L.mx_packed_sizes(elem, layout, E, N, K, C.byref(wb), C.byref(cb))
    return st, wb.value, cb.value


# ---- status strings, arch gate, packed sizes
for s in range(12):
    assert L.mx_status_str(s)
for name in (b"gfx950", b"gfx950:xnack-", b"gfx942", b"", b"gfx9501"):
    L.mx_arch_supported(name)
for elem, layout, E, N, K in [(0, 0, 1, 256, 512), (0, 1, 1, 7168, 7168), (0, 0, 1, 4096, 1568),
                              (1, 0, 32, 3072, 3072), (1, 0, 2, 16, 160), (0, 1, 3, 64, 96)]:
    st, wb, cb = sizes(elem, layout, E, N, K)
    expect(st, OK, "packed sizes")
    assert wb == E * N * (K if elem == 0 else K // 2) and cb % 16 == 0
for args in [(0, 0, 1, 24, 512), (0, 1, 1, 48, 512), (0, 0, 1, 32, 100), (2, 0, 1, 32, 64),
             (0, 2, 1, 32, 64), (0, 0, 0, 32, 64)]:
    expect(sizes(*args)[0], SHAPE if args[0] < 2 and args[1] < 2 else UNSUP, f"sizes {args}")

# ---- pack
for elem, layout, E, N, K in [(0, 0, 1, 256, 512), (0, 1, 1, 64, 1568), (1, 0, 4, 32, 160)]:
    expect(L.mx_pack_weights(elem, layout, E, N, K, dev(1), dev(2), dev(3), dev(4), dev(5), 256,
                             None), OK, "pack")
expect(L.mx_pack_weights(0, 0, 1, 32, 64, dev(1), dev(2), dev(3), dev(4), dev(5), 255, None), WS,
       "pack ws")
expect(L.mx_pack_weights(0, 0, 1, 32, 64, dev(1) + 4, dev(2), dev(3), dev(4), dev(5), 256, None),
       ALIGN, "pack align")
expect(L.mx_pack_weights(0, 0, 1, 32, 64, None, dev(2), dev(3), dev(4), dev(5), 256, None), NULL,
       "pack null")

# ---- activation quantization
for M, K, rule in [(1, 32, 0), (16, 7168, 1), (4096, 7168, 0), (3, 1568, 1)]:
    expect(L.mx_quant_act(M, K, dev(1), K, dev(2), (K + 15) // 16 * 16, dev(3), K // 32, rule, None),
           OK, "quant")
    qb, cb = C.c_size_t(), C.c_size_t()
    expect(L.mx_act_t16_sizes(M, K, C.byref(qb), C.byref(cb)), OK, "t16 sizes")
    expect(L.mx_quant_act_t16(M, K, dev(1), K, dev(2), dev(3), rule, None), OK, "quant t16")
expect(L.mx_quant_act(4, 64, dev(1), 32, dev(2), 64, dev(3), 2, 0, None), SHAPE, "quant ldx")
expect(L.mx_quant_act(4, 64, dev(1), 64, dev(2), 64, dev(3), 2, 7, None), UNSUP, "quant rule")
expect(L.mx_quant_act_t16(4, 64, dev(1) + 2, 64, dev(2), dev(3), 0, None), ALIGN, "t16 align")


# ---- dense linear over the built combinations, decode and prefill sizes
def ws_bytes(elem, layout, N, K, M, act, preq):
    b = C.c_size_t()
    expect(L.mx_linear_workspace(elem, layout, N, K, M, act, preq, C.byref(b)), OK, "workspace")
    return b.value


COMBOS = [(E4M3, ROW32, BF16), (E4M3, BLK32, BF16), (E2M1, ROW32, BF16), (E4M3, ROW32, MXFP8),
          (E4M3, BLK32, MXFP8), (E4M3, ROW32, T16), (E4M3, BLK32, T16)]
SHAPES = [(1, 256, 512), (16, 7168, 7168), (8, 4096, 1568), (64, 512, 1024), (65, 512, 1024),
          (4096, 7168, 7168), (3, 64, 8320), (17, 96, 96)]
for invariant in (0, 1):
    L.mx_set_batch_invariant(invariant)
    for elem, layout, act in COMBOS:
        for M, N, K in SHAPES:
            if layout == BLK32 and N % 32:
                continue
            for preq in ((0, 1) if act == MXFP8 else (0,)):
                need = ws_bytes(elem, layout, N, K, M, act, preq)
                x = dev(1) if act == BF16 or (act == MXFP8 and not preq) else None
                xq = dev(2) if act == T16 or preq else None
                xc = dev(3) if act == T16 or preq else None
                ldq = (K + 15) // 16 * 16 if preq else 0
                st = L.mx_linear(elem, layout, N, K, dev(4), dev(5), M, act, 0, x, K if x else 0,
                                 xq, ldq, xc, K // 32 if preq else 0, dev(6) if M % 2 else None,
                                 dev(7), N, dev(8) if need else None, need, None)
                # T16 input is refused (UNSUP) where K is beyond the decode
                # GEMV's reach; everything else is served
                beyond = act == T16 and -(-K // 128) > 64 and (M <= 64 or invariant)
                expect(st, UNSUP if beyond else OK, f"linear {elem, layout, act, M, N, K, preq}")
                if need:
                    expect(L.mx_linear(elem, layout, N, K, dev(4), dev(5), M, act, 0, x,
                                       K if x else 0, xq, ldq, xc, K // 32 if preq else 0, None,
                                       dev(7), N, dev(8), need - 1, None), WS, "linear ws")
L.mx_set_batch_invariant(0)
expect(L.mx_linear(1, 1, 64, 64, dev(4), dev(5), 1, BF16, 0, dev(1), 64, None, 0, None, 0, None,
                   dev(7), 64, None, 0, None), UNSUP, "e2m1 blk32")
expect(L.mx_linear(0, 0, 64, 64, dev(4), dev(5), 1, BF16, 0, dev(1), 64, None, 0, None, 0, None,
                   dev(7), 32, None, 0, None), SHAPE, "ldy")
expect(L.mx_linear(0, 0, 64, 64, dev(4), dev(5), 1, BF16, 0, dev(1) + 8, 64, None, 0, None, 0,
                   None, dev(7), 64, None, 0, None), ALIGN, "x align")
expect(L.mx_linear(0, 0, 64, 64, dev(4), dev(5), 1, BF16, 0, None, 64, None, 0, None, 0, None,
                   dev(7), 64, None, 0, None), NULL, "x null")

# ---- MoE: grouped GEMV, the allocation-free variant, the block, ingest
for elem in (E2M1, E4M3):
    for (E, N, K, T, topk) in [(32, 3072, 3072, 16, 8), (6, 32, 256, 40, 2), (4, 48, 1568, 6, 2)]:
        for combine in (0, 1):
            b = C.c_size_t()
            expect(L.mx_moe_workspace(elem, E, N, K, T, topk, combine, C.byref(b)), OK, "moe ws")
            wts = dev(9) if combine else None
            expect(L.mx_moe_linear(elem, E, N, K, dev(1), dev(2), T, topk, dev(3), K, dev(4), wts,
                                   dev(5), dev(6) if b.value else None, b.value, None), OK, "moe")
            expect(L.mx_moe_linear_noalloc(elem, E, N, K, dev(1), dev(2), T, topk, dev(3), K,
                                           dev(4), wts, dev(5), None), OK, "moe noalloc")
    expect(L.mx_moe_gate_up(elem, 32, 1536, 3072, dev(1), dev(2), 16, 8, dev(3), 3072, dev(4),
                            dev(5), 1536, None), OK, "gate up")
    b = C.c_size_t()
    expect(L.mx_moe_workspace(elem, 32, 3072, 1536, 16, 8, 1, C.byref(b)), OK, "down ws")
    expect(L.mx_moe_down(elem, 32, 3072, 1536, dev(1), dev(2), 16, 8, dev(3), 1536, dev(4),
                         dev(9), dev(5), dev(6), b.value, None), OK, "down")
    expect(L.mx_moe_copies(elem, 8, 1600, 1536, 3072, 3072, dev(1), dev(2), dev(3), dev(4),
                           dev(5), dev(6), dev(7), dev(8), dev(9), 256, None), OK, "copies")
expect(L.mx_moe_linear(1, 4, 32, 256, dev(1), dev(2), 5, 5, dev(3), 256, dev(4), None, dev(5),
                       None, 0, None), SHAPE, "topk > E")
expect(L.mx_moe_linear_noalloc(1, 32, 3072, 3072, dev(1), dev(2), 512, 8, dev(3), 3072, dev(4),
                               dev(9), dev(5), None), WS, "noalloc beyond its buffer")
expect(L.mx_fold_row_codes(7168, 7168, dev(1), 224, dev(2), dev(3), 256, None), OK, "fold")
expect(L.mx_fold_row_codes(48, 64, dev(1), 2, dev(2), dev(3), 256, None), SHAPE, "fold N")
expect(L.mx_e4m3_from_dequant(1, 64, 256, dev(1), 256, dev(2), dev(3), dev(4), 256, None), OK,
       "from dequant")
expect(L.mx_fused_layout_permute(0, 0, 16 * 192, 512, 16, dev(1), dev(2), dev(3), dev(4), None),
       OK, "q rows")
expect(L.mx_fused_layout_permute(1, 1, 64, 8 * 512, 8, dev(1), dev(2), dev(3), dev(4), None), OK,
       "o cols")

assert launches.value > 100, launches.value
print(f"host checks ok: {calls} calls, {launches.value} stub launches", flush=True)
