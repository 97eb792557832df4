/*
 * mx_oracle.c -- plain, slow CPU reference ("oracle") for the block-scaled
 * (OCP microscaling) linear layer y = x . W^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or constant with the
 * HIP library; both sides are written independently from the definitions
 * below.
 *
 * Sources (web pages; cited by page title and section):
 *   [weights942]   vllm.models.deepseek_v41.amd.mono.weights942
 *   [rocm_native]  vllm.model_executor.kernels.linear.mxfp8.rocm_native
 *   [a16w4]        vllm.models.minimax_m3.amd.specialized_decode.mono.a16w4
 *   [fused_layout] vllm.models.deepseek_v41.common.ops.fused_layout
 *
 * Arithmetic: every real value is carried in IEEE binary64.  Decoding is
 * exact, products of decoded operands are exact in binary64, and sums are
 * taken in index order.  Nothing is fused, blocked or reordered.
 *
 * Readings taken where the pages leave a step open (each one is listed with
 * its justification in the design notes of the repository):
 *   R1  activation scale rule "ocp": shared exponent floor(log2 amax) - 8
 *       (8 = exponent of the largest e4m3 normal, 448 = 1.75 * 2^8); element
 *       conversion round-to-nearest-even with saturation to +-448.
 *   R2  activation scale rule "ceil448": the rule [rocm_native] _quant_mxfp8_tile
 *       states, ceil(log2(max(amax, TINY) / 448)) + 127 clamped to [0, 254],
 *       with TINY = 2^-126 and FP8_MAX = 448 (both undefined on the page).
 *   R3  a zero result keeps the sign of its input (-0 -> 0x80).
 *   R4  K is padded to a multiple of 128 with zero bytes and scale code 128
 *       ([weights942] dense_copy); padding never enters a sum.
 *   R5  MoE ids outside [0, E) give all-zero output rows.
 *   R18 the gated activation of the MoE up-gate product is SiLU.
 *   R20 a bf16-dequantized weight is recovered only when some e4m3 byte times
 *       its block's scale equals it exactly (a zero keeps its sign).
 *
 * Parity pins: every function here is checked in tests/test_oracle_*.py
 * against closed forms, brute force and exact rational arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_E4M3 = 0, ORC_E2M1 = 1 };
enum { ORC_ROW32 = 0, ORC_BLK32 = 1 };
enum { ORC_RULE_OCP = 0, ORC_RULE_CEIL448 = 1 };
enum { ORC_ACT_BF16 = 0, ORC_ACT_MXFP8 = 1 };

/* ------------------------------------------------------------------ */
/* Element and scale decoding                                          */
/* ------------------------------------------------------------------ */

/* OCP E4M3 byte: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal: 2^-6 * m/8.  0x7F and 0xFF are NaN; the
 * largest finite magnitude is 0x7E = 1.75 * 2^8 = 448.  ([weights942] module
 * notes on OCP bytes; [rocm_native] float8e4nv.) */
double orc_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* OCP E2M1 nibble: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
 * Exponent field 0 is subnormal: m/2.  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
 * ([a16w4] dequant: packed two per byte, low nibble first.) */
double orc_e2m1_value(int nibble)
{
    int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    double mag;
    if (e == 0)
        mag = (double)m / 2.0;
    else
        mag = ldexp(1.0 + (double)m / 2.0, e - 1);
    return s ? -mag : mag;
}

/* E8M0 scale code: the power of two 2^(code - 127); code 255 is NaN.
 * ([weights942] ocp_from_dequant: value = e4m3 value x 2^(code - 127).) */
double orc_e8m0_value(int code)
{
    if (code == 255)
        return NAN;
    return ldexp(1.0, code - 127);
}

/* A bfloat16 bit pattern is the upper half of a binary32 pattern. */
double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------ */
/* E4M3 rounding                                                       */
/* ------------------------------------------------------------------ */

/* Nearest finite E4M3 value to v, ties to the code whose mantissa LSB is 0,
 * saturating at +-448 (R1), zero keeping the sign of v (R3).  The 127
 * non-negative finite codes 0x00..0x7E are increasing in value, so the
 * nearest code is found by locating v between two neighbours. */
int orc_e4m3_round(double v)
{
    int sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    int lo, hi, mid, pick;
    double dlo, dhi;
    if (a >= 448.0)
        return sign | 0x7E;
    /* largest code lo with value(lo) <= a */
    lo = 0;
    hi = 0x7E;
    while (lo < hi) {
        mid = (lo + hi + 1) / 2;
        if (orc_e4m3_value(mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    if (orc_e4m3_value(lo) == a)
        return sign | lo;
    dlo = a - orc_e4m3_value(lo);
    dhi = orc_e4m3_value(lo + 1) - a;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = lo + 1;
    else
        pick = (lo & 1) ? lo + 1 : lo;
    return sign | pick;
}

/* ------------------------------------------------------------------ */
/* Activation quantization (per token, per 32-element K block)          */
/* ------------------------------------------------------------------ */

/* E8M0 code of a block whose largest magnitude is amax.
 *   ocp     (R1): code = floor(log2 amax) - 8 + 127, clamped to [0, 254];
 *                 amax == 0 gives code 0.
 *   ceil448 (R2): [rocm_native] _quant_mxfp8_tile -- the smallest n with
 *                 448 * 2^n >= max(amax, TINY); code = n + 127 clamped to
 *                 [0, 254].
 * Both exponents start from a log2 guess and are then settled by exact
 * comparisons against powers of two, so the guess's rounding cannot matter. */
int orc_act_code(double amax, int rule)
{
    int n;
    if (rule == ORC_RULE_OCP) {
        if (amax == 0.0)
            return 0;
        n = (int)floor(log2(amax));
        while (ldexp(1.0, n) > amax) /* largest n with 2^n <= amax */
            n--;
        while (ldexp(1.0, n + 1) <= amax)
            n++;
        n = n - 8 + 127;
    } else {
        double a = amax > ldexp(1.0, -126) ? amax : ldexp(1.0, -126);
        n = (int)ceil(log2(a / 448.0));
        while (ldexp(448.0, n - 1) >= a) /* smallest n with 448 * 2^n >= a */
            n--;
        while (ldexp(448.0, n) < a)
            n++;
        n = n + 127;
    }
    if (n < 0)
        n = 0;
    if (n > 254)
        n = 254;
    return n;
}

/* Quantize x (bf16 bits, [M, K] with row stride ldx) to e4m3 bytes xq
 * ([M, K], stride ldq) and row-major E8M0 codes ([M, K/32], stride ldc):
 * for each row m and block b, code = orc_act_code(max |x|), and each
 * element is RNE_e4m3(x * 2^(127 - code)), the product exact in binary64.
 * ([rocm_native] module notes: per-token quantization with row-major
 * [M, K/32] codes; _quant_mxfp8_tile for the per-block steps.) */
void orc_quant_act(int64_t M, int64_t K, const uint16_t *x, int64_t ldx,
                   uint8_t *xq, int64_t ldq, uint8_t *codes, int64_t ldc,
                   int rule)
{
    int64_t m, b, i;
    for (m = 0; m < M; m++) {
        for (b = 0; b < K / 32; b++) {
            double amax = 0.0;
            int code;
            double mul;
            for (i = 0; i < 32; i++) {
                double a = fabs(orc_bf16_value(x[m * ldx + 32 * b + i]));
                if (a > amax)
                    amax = a;
            }
            code = orc_act_code(amax, rule);
            mul = ldexp(1.0, 127 - code);
            codes[m * ldc + b] = (uint8_t)code;
            for (i = 0; i < 32; i++) {
                double v = orc_bf16_value(x[m * ldx + 32 * b + i]) * mul;
                xq[m * ldq + 32 * b + i] = (uint8_t)orc_e4m3_round(v);
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Packed weight and code layouts                                      */
/* ------------------------------------------------------------------ */
/*
 * Notation: E experts (1 for a dense layer), N rows per expert, K values per
 * row, Kp = K rounded up to 128 (R4), S = Kp / 128 "steps", T = N / 16
 * "tiles" of 16 rows, Q = ceil(S / 4) "quads" of four steps.  A lane index
 * l in [0, 64) of a 64-wide wavefront is split as l = 16 j + r.
 *
 * Weights W-T16.  For each (expert e, tile t, step s) a chunk of 16 rows x
 * 128 K values: 2048 bytes for E4M3, 1024 for E2M1.  Lane l reads 16-byte
 * pieces at 16 l (+ 1024 for the second E4M3 half), so every 16-byte load of
 * the wavefront reads 1 KB contiguous: the tile-major idea of [weights942]
 * dense_copy and fp4_tile_major.  When K % 128 != 0 the last step holds
 * TB = (K % 128) / 32 blocks; its valid bytes are exactly the first TB * 512
 * (E4M3) or TB * 256 (E2M1) bytes of the chunk, and the chunk is stored cut
 * to them, so a tile takes exactly 16 row lengths of bytes, TILEB = 16 K
 * (E4M3) or 8 K (E2M1): no padding is stored (reading R21).
 *   E4M3: lane l holds row 16 t + r, K 16 j .. 16 j + 15 of the step in its
 *         first half and K 64 + 16 j .. + 15 in its second half -- the K
 *         order in which a gfx950 16x16x128 scaled matrix-core operand lane
 *         holds its 32 bytes (lane group j's scale covers K block j).
 *   E2M1: lane l holds row 16 t + r, the whole 32-value block 4 s + j (one
 *         code group a lane), as in [a16w4] (module notes).
 *
 *   E4M3: wp[(e T + t) TILEB + 2048 s + 1024 h + 16 l + c]
 *           = w[e][16 t + r][128 s + 64 h + 16 j + c]      for K index < K
 *   E2M1: wp[(e T + t) TILEB + 1024 s + 16 l + c]
 *           = w[e][16 t + r][byte 64 s + 16 j + c]         for byte < K / 2
 *                                                      (low nibble = even K)
 *
 * Codes ROW32 ([E N, K/32] in) -> C-T16.  For each (expert, tile, quad) 256
 * bytes; lane l's dword holds the codes of its row for the blocks it owns in
 * the quad's four steps, step 4 q + u in byte u.  A lane group of 16 lanes
 * reads 64 contiguous bytes (the staging idea of [weights942]
 * codes_tile_rounds and the per-lane dwords of [a16w4] scale_loads).
 *
 *   cp[((e T + t) Q + q) 256 + 4 l + u] = codes[e N + 16 t + r][4 (4 q + u) + j]
 *
 * Codes BLK32 ([E N/32, K/32] in) -> [E N/32][Q][16]: for each 32-row group
 * and quad, 16 bytes; lane group j's dword (bytes 4 j .. 4 j + 3) holds the
 * group's codes of block 4 s + j for the quad's four steps s = 4 q + u in
 * byte u -- the same dword-per-lane-group, byte-per-step staging as C-T16.
 *
 *   cp[(R Q + q) 16 + 4 j + u] = codes[R][4 (4 q + u) + j]
 *
 * Every code of a block outside [0, K/32) is 128 (R4).
 */

int64_t orc_padded_k(int64_t K) { return (K + 127) / 128 * 128; }

/* 0 on success, 1 for a shape the layout does not cover. */
int orc_packed_sizes(int elem, int layout, int64_t E, int64_t N, int64_t K,
                     int64_t *w_bytes, int64_t *c_bytes)
{
    int64_t Kp = orc_padded_k(K), S = Kp / 128, Q = (S + 3) / 4;
    if (E < 1 || N < 1 || K < 32 || K % 32 != 0 || N % 16 != 0)
        return 1;
    if (layout == ORC_BLK32 && N % 32 != 0)
        return 1;
    *w_bytes = E * N * (elem == ORC_E4M3 ? K : K / 2);          /* no stored padding */
    (void)Kp;
    if (layout == ORC_ROW32)
        *c_bytes = E * (N / 16) * Q * 256;
    else
        *c_bytes = E * (N / 32) * Q * 16;
    *c_bytes += 16;                                /* the code-range trailer */
    return 0;
}

int orc_pack_weights(int elem, int layout, int64_t E, int64_t N, int64_t K,
                     const uint8_t *w, const uint8_t *codes, uint8_t *wp,
                     uint8_t *cp)
{
    int64_t Kp = orc_padded_k(K), S = Kp / 128, Q = (S + 3) / 4, T = N / 16;
    int64_t tileb = 16 * (elem == ORC_E4M3 ? K : K / 2);
    int64_t wb, cb, e, t, s, q, l, h, c, u;
    if (orc_packed_sizes(elem, layout, E, N, K, &wb, &cb))
        return 1;
    for (e = 0; e < E; e++)
        for (t = 0; t < T; t++)
            for (s = 0; s < S; s++)
                for (l = 0; l < 64; l++) {
                    int64_t r = l % 16, j = l / 16, row = 16 * t + r;
                    if (elem == ORC_E4M3) {
                        for (h = 0; h < 2; h++)
                            for (c = 0; c < 16; c++) {
                                int64_t k = 128 * s + 64 * h + 16 * j + c;
                                int64_t dst = (e * T + t) * tileb + 2048 * s + 1024 * h + 16 * l + c;
                                if (k < K)
                                    wp[dst] = w[(e * N + row) * K + k];
                            }
                    } else {
                        for (c = 0; c < 16; c++) {
                            int64_t byte = 64 * s + 16 * j + c;
                            int64_t dst = (e * T + t) * tileb + 1024 * s + 16 * l + c;
                            if (byte < K / 2)
                                wp[dst] = w[(e * N + row) * (K / 2) + byte];
                        }
                    }
                }
    if (layout == ORC_ROW32) {
        for (e = 0; e < E; e++)
            for (t = 0; t < T; t++)
                for (q = 0; q < Q; q++)
                    for (l = 0; l < 64; l++)
                        for (u = 0; u < 4; u++) {
                            int64_t r = l % 16, j = l / 16;
                            int64_t blk = 4 * (4 * q + u) + j;
                            int64_t dst = ((e * T + t) * Q + q) * 256 + 4 * l + u;
                            cp[dst] = blk < K / 32 ? codes[(e * N + 16 * t + r) * (K / 32) + blk] : 128;
                        }
    } else {
        int64_t R, jj;
        for (R = 0; R < E * N / 32; R++)
            for (q = 0; q < Q; q++)
                for (jj = 0; jj < 4; jj++)
                    for (u = 0; u < 4; u++) {
                        int64_t blk = 4 * (4 * q + u) + jj;
                        int64_t dst = (R * Q + q) * 16 + 4 * jj + u;
                        cp[dst] = blk < K / 32 ? codes[R * (K / 32) + blk] : 128;
                    }
    }
    /* trailer: the smallest and the largest of the given codes (padding not
     * counted), then 14 zero bytes */
    {
        int64_t n = (layout == ORC_ROW32 ? E * N : E * N / 32) * (K / 32), i;
        uint8_t lo = 255, hi = 0;
        for (i = 0; i < n; i++) {
            if (codes[i] < lo) lo = codes[i];
            if (codes[i] > hi) hi = codes[i];
        }
        memset(cp + cb - 16, 0, 16);
        cp[cb - 16] = lo;
        cp[cb - 15] = hi;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Dequantized operands                                                */
/* ------------------------------------------------------------------ */

/* Weight value Wf[e][n][k] = dec(w) * 2^(code - 127) from the standard
 * (unpacked) layouts: E4M3 bytes [E, N, K] or E2M1 bytes [E, N, K/2] (value
 * k in byte k/2, low nibble for even k); codes [E N, K/32] (ROW32) or
 * [E N/32, K/32] (BLK32).  ([weights942] ocp_from_dequant; [a16w4] dequant.) */
double orc_weight(int elem, int layout, int64_t E, int64_t N, int64_t K,
                  const uint8_t *w, const uint8_t *codes, int64_t e, int64_t n,
                  int64_t k)
{
    double v;
    int code;
    (void)E;
    if (elem == ORC_E4M3) {
        v = orc_e4m3_value(w[(e * N + n) * K + k]);
    } else {
        int byte = w[(e * N + n) * (K / 2) + k / 2];
        v = orc_e2m1_value(k % 2 == 0 ? (byte & 15) : (byte >> 4));
    }
    if (layout == ORC_ROW32)
        code = codes[(e * N + n) * (K / 32) + k / 32];
    else
        code = codes[((e * N + n) / 32) * (K / 32) + k / 32];
    return v * orc_e8m0_value(code);
}

/* Activation value a[m][k]: the bf16 value itself (A16), or the MXFP8 pair
 * dec(xq) * 2^(xcode - 127) with row-major codes (W8A8). */
double orc_activation(int act, const uint16_t *x, int64_t ldx, const uint8_t *xq,
                      int64_t ldq, const uint8_t *xc, int64_t ldc, int64_t m,
                      int64_t k)
{
    if (act == ORC_ACT_BF16)
        return orc_bf16_value(x[m * ldx + k]);
    return orc_e4m3_value(xq[m * ldq + k]) * orc_e8m0_value(xc[m * ldc + k / 32]);
}

/* ------------------------------------------------------------------ */
/* Linear layer                                                        */
/* ------------------------------------------------------------------ */

/* y[m][n] = sum_{k < K} a[m][k] Wf[n][k] (+ bias[n]), binary64, k ascending.
 * ([rocm_native] RocmDotScaledMxfp8LinearKernel.apply_weights: out = x W^T,
 * then + bias.)  Rows of Wf are decoded once per n; the sums are unchanged. */
void orc_linear(int elem, int layout, int64_t N, int64_t K, const uint8_t *w,
                const uint8_t *codes, int64_t M, int act, const uint16_t *x,
                int64_t ldx, const uint8_t *xq, int64_t ldq, const uint8_t *xc,
                int64_t ldc, const uint16_t *bias, double *y)
{
    double *a = (double *)malloc(sizeof(double) * (size_t)(M * K));
    int64_t m, k, n;
    for (m = 0; m < M; m++)
        for (k = 0; k < K; k++)
            a[m * K + k] = orc_activation(act, x, ldx, xq, ldq, xc, ldc, m, k);
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; n++) {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)K);
        int64_t mm, kk;
        for (kk = 0; kk < K; kk++)
            wrow[kk] = orc_weight(elem, layout, 1, N, K, w, codes, 0, n, kk);
        for (mm = 0; mm < M; mm++) {
            double s = 0.0;
            for (kk = 0; kk < K; kk++)
                s += a[mm * K + kk] * wrow[kk];
            if (bias)
                s += orc_bf16_value(bias[n]);
            y[mm * N + n] = s;
        }
        free(wrow);
    }
    free(a);
}

/* The same sums, for a list of (m, n) pairs only (large shapes). */
void orc_linear_pairs(int elem, int layout, int64_t N, int64_t K,
                      const uint8_t *w, const uint8_t *codes, int act,
                      const uint16_t *x, int64_t ldx, const uint8_t *xq,
                      int64_t ldq, const uint8_t *xc, int64_t ldc,
                      const uint16_t *bias, int64_t npairs, const int64_t *ms,
                      const int64_t *ns, double *out)
{
    int64_t p;
#pragma omp parallel for schedule(static)
    for (p = 0; p < npairs; p++) {
        double s = 0.0;
        int64_t kk;
        for (kk = 0; kk < K; kk++)
            s += orc_activation(act, x, ldx, xq, ldq, xc, ldc, ms[p], kk) *
                 orc_weight(elem, layout, 1, N, K, w, codes, 0, ns[p], kk);
        if (bias)
            s += orc_bf16_value(bias[ns[p]]);
        out[p] = s;
    }
}

/* ------------------------------------------------------------------ */
/* Grouped MoE linear                                                  */
/* ------------------------------------------------------------------ */

/* For every token t and slot k of its top-k routing, the row
 *   y[t][k][:] = x[t] . Wf[id[t][k]]^T                       (per slot), or
 *   out[t][:]  = sum_k weight[t][k] y[t][k][:], k ascending  (combined),
 * in binary64.  Expert weights are [E, N, K] in the standard layouts with
 * ROW32 codes [E N, K/32] ([weights942] moe_copies, expert tensors before
 * conversion).  An id outside [0, E) contributes a zero row (R5). */
void orc_moe_linear(int elem, int64_t E, int64_t N, int64_t K, const uint8_t *w,
                    const uint8_t *codes, int64_t T, int64_t topk,
                    const uint16_t *x, int64_t ldx, const int32_t *ids,
                    const float *weights, double *y)
{
    int64_t n;
    int64_t rows = weights ? T : T * topk;
    memset(y, 0, sizeof(double) * (size_t)(rows * N));
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; n++) {
        int64_t t, k, kk;
        for (t = 0; t < T; t++)
            for (k = 0; k < topk; k++) {
                int32_t e = ids[t * topk + k];
                double s = 0.0;
                if (e >= 0 && e < E)
                    for (kk = 0; kk < K; kk++)
                        s += orc_bf16_value(x[t * ldx + kk]) *
                             orc_weight(elem, ORC_ROW32, E, N, K, w, codes, e, n, kk);
                if (weights)
                    y[t * N + n] += (double)weights[t * topk + k] * s;
                else
                    y[(t * topk + k) * N + n] = s;
            }
    }
}

/* ------------------------------------------------------------------ */
/* The MoE block around the grouped linear                              */
/* ------------------------------------------------------------------ */

/* Load-time copies of the expert tensors ([weights942] moe_copies): the
 * input w13 holds, per expert, 2 Np rows -- the gate rows 0 .. inter - 1,
 * zero rows up to Np, the up rows Np .. Np + inter - 1, zero rows up to 2 Np
 * -- of rowb bytes each (K / 2 for e2m1, K for e4m3), with codes
 * [E, 2 Np, K / 32]; w2 is [E, H, Np] values (bytes per row Np / 2 or Np)
 * with codes [E, H, Np / 32].  The copies are
 *   out_w13[e][2 i][:]     = w13[e][i][:]        (gate row i)
 *   out_w13[e][2 i + 1][:] = w13[e][Np + i][:]   (up row i),   i < inter,
 * the codes alike, and w2 / its codes cut to the first inter values of each
 * row.  Returns 1, copying nothing, when a padding byte of the weights is
 * not zero (the page refuses it), 2 for shapes outside inter <= Np,
 * inter % 32 == 0, K % 32 == 0.  The gfx942 copy also rewrites -0 nibbles;
 * this one keeps every byte (-0 decodes equal to +0, reading R7). */
int orc_moe_copies(int elem, int64_t E, int64_t Np, int64_t inter, int64_t K,
                   int64_t H, const uint8_t *w13, const uint8_t *s13,
                   const uint8_t *w2, const uint8_t *s2, uint8_t *out_w13,
                   uint8_t *out_s13, uint8_t *out_w2, uint8_t *out_s2)
{
    const int64_t rowb = elem == ORC_E2M1 ? K / 2 : K;        /* w13 row bytes */
    const int64_t kb = K / 32;                                  /* w13 codes per row */
    const int64_t r2in = elem == ORC_E2M1 ? Np / 2 : Np;        /* w2 row bytes in */
    const int64_t r2out = elem == ORC_E2M1 ? inter / 2 : inter; /* w2 row bytes out */
    int64_t e, i, g, b, h;
    if (inter < 1 || inter > Np || inter % 32 != 0 || Np % 32 != 0 || K % 32 != 0)
        return 2;
    for (e = 0; e < E; e++) {
        for (g = 0; g < 2; g++)
            for (i = inter; i < Np; i++)
                for (b = 0; b < rowb; b++)
                    if (w13[(e * 2 * Np + g * Np + i) * rowb + b] != 0)
                        return 1;
        for (h = 0; h < H; h++)
            for (b = r2out; b < r2in; b++)
                if (w2[(e * H + h) * r2in + b] != 0)
                    return 1;
    }
    for (e = 0; e < E; e++) {
        for (i = 0; i < inter; i++)
            for (g = 0; g < 2; g++) {
                const int64_t src = e * 2 * Np + g * Np + i, dst = e * 2 * inter + 2 * i + g;
                memcpy(out_w13 + dst * rowb, w13 + src * rowb, (size_t)rowb);
                memcpy(out_s13 + dst * kb, s13 + src * kb, (size_t)kb);
            }
        for (h = 0; h < H; h++) {
            memcpy(out_w2 + (e * H + h) * r2out, w2 + (e * H + h) * r2in, (size_t)r2out);
            memcpy(out_s2 + (e * H + h) * (inter / 32), s2 + (e * H + h) * (Np / 32),
                   (size_t)(inter / 32));
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Ingest variants: row-expanded codes, bf16-dequantized weights        */
/* ------------------------------------------------------------------ */

/* [rocm_native] _as_block32_scale, [weights942] linear_copy: a checkpoint's
 * 32 x 32 block codes that the loader repeated over each block's 32 rows come
 * back as [N][KB]; folded, out[R][b] = codes_row[32 R][b], provided every one
 * of rows 32 R .. 32 R + 31 holds that same code in column b.  Returns 1,
 * writing nothing, when some block's rows disagree (the page raises, or keeps
 * the row codes); 2 when N is not a positive multiple of 32 or KB < 1. */
int orc_fold_row_codes(int64_t N, int64_t KB, const uint8_t *codes_row, uint8_t *codes_blk)
{
    int64_t R, i, b;
    if (N < 32 || N % 32 != 0 || KB < 1)
        return 2;
    for (R = 0; R < N / 32; R++)
        for (i = 1; i < 32; i++)
            for (b = 0; b < KB; b++)
                if (codes_row[(32 * R + i) * KB + b] != codes_row[32 * R * KB + b])
                    return 1;
    for (R = 0; R < N / 32; R++)
        memcpy(codes_blk + R * KB, codes_row + 32 * R * KB, (size_t)KB);
    return 0;
}

/* [weights942] ocp_from_dequant: the e4m3 bytes behind a weight the loader
 * dequantized to bf16, w[n][k] = dec(byte) * 2^(c - 127), c the code of the
 * weight's block (layout ROW32: codes [N][K/32]; BLK32: [N/32][K/32]).  The
 * page's steps: multiply w by 2^(127 - c), round to the nearest e4m3
 * (orc_e4m3_round: ties to even, sign of zero kept), scale the byte's value
 * back by 2^(c - 127) and require it to equal w.  Here both scalings are
 * exact (binary64), so "equal" is equality of the real values (reading R20).
 * A weight that does not come back -- not e4m3 x 2^(c - 127), NaN, infinite,
 * or under code 255, which is NaN (reading R6) -- gets the marker 0xFF in out
 * (a NaN byte, never a valid answer) and is counted.  Returns that count, or
 * -1 for a shape outside K % 32 == 0 (and N % 32 == 0 for BLK32). */
int64_t orc_e4m3_from_dequant(int layout, int64_t N, int64_t K, const uint16_t *w,
                              int64_t ldw, const uint8_t *codes, uint8_t *out)
{
    const int64_t KB = K / 32;
    int64_t n, k, bad = 0;
    if (N < 1 || K < 32 || K % 32 != 0 || ldw < K ||
        (layout == ORC_BLK32 && N % 32 != 0))
        return -1;
    for (n = 0; n < N; n++)
        for (k = 0; k < K; k++) {
            const double v = orc_bf16_value(w[n * ldw + k]);
            const int c = layout == ORC_BLK32 ? codes[(n / 32) * KB + k / 32]
                                              : codes[n * KB + k / 32];
            int byte = 0xFF;
            if (c != 255 && isfinite(v)) {
                const int q = orc_e4m3_round(ldexp(v, 127 - c));
                if (ldexp(orc_e4m3_value(q), c - 127) == v)
                    byte = q;
            }
            if (byte == 0xFF)
                bad++;
            out[n * K + k] = (uint8_t)byte;
        }
    return bad;
}

/* ------------------------------------------------------------------ */
/* Load-time layout permutations for the attention-adjacent linears     */
/* ------------------------------------------------------------------ */

/* [fused_layout] q_fused_permutation: the attention kernel reads Q with each
 * head's D values cut into 16-value chunks, chunk d/16 of every head side by
 * side: fused index (d / 16) H 16 + h 16 + d % 16 holds standard index
 * h D + d.  perm[f] = the standard index at fused index f (fused =
 * standard[perm]).  Returns 1 when D % 16 != 0. */
int orc_q_fused_perm(int64_t H, int64_t D, int64_t *perm)
{
    int64_t h, d;
    if (H < 1 || D < 16 || D % 16 != 0)
        return 1;
    for (h = 0; h < H; h++)
        for (d = 0; d < D; d++)
            perm[(d / 16) * H * 16 + h * 16 + d % 16] = h * D + d;
    return 0;
}

/* [fused_layout] o_fused_permutation: the kernel writes O for the G heads of
 * a group with each head's D values cut into 32-value chunks, chunk c of
 * every head side by side: fused index (c G + h) 32 + j holds standard index
 * h D + c 32 + j.  Returns 1 when D % 32 != 0. */
int orc_o_fused_perm(int64_t G, int64_t D, int64_t *perm)
{
    int64_t h, c, j;
    if (G < 1 || D < 32 || D % 32 != 0)
        return 1;
    for (h = 0; h < G; h++)
        for (c = 0; c < D / 32; c++)
            for (j = 0; j < 32; j++)
                perm[(c * G + h) * 32 + j] = h * D + c * 32 + j;
    return 0;
}

/* [fused_layout] permute_wq_b_: the rows of an MXFP8 weight [N, K] and of
 * its per-row codes [N, K/32] gathered by the Q permutation of `heads` heads
 * of D = N / heads rows: out row f = in row perm[f].  permute_wo_a_: the
 * input columns of [N, K] gathered by the O permutation of `heads` heads of
 * D = K / heads columns, and the code columns (one per 32 columns, layout
 * ROW32 [N, K/32] or BLK32 [N/32, K/32]) by its per-chunk form, perm[32 f] /
 * 32.  kind 0 = Q rows (ROW32 codes only: a 32-row block would straddle two
 * heads), 1 = O columns.  Returns 1 for shapes the permutation does not
 * divide, 2 for Q rows with BLK32 codes. */
int orc_fused_layout_permute(int kind, int layout, int64_t N, int64_t K, int64_t heads,
                             const uint8_t *w, const uint8_t *codes, uint8_t *w_out,
                             uint8_t *codes_out)
{
    const int64_t KB = K / 32;
    int64_t *perm, f, n;
    if (heads < 1 || K < 32 || K % 32 != 0 || N < 1)
        return 1;
    if (kind == 0) {
        if (layout != ORC_ROW32)
            return 2;
        if (N % heads != 0)
            return 1;
        perm = malloc((size_t)N * sizeof *perm);
        if (orc_q_fused_perm(heads, N / heads, perm)) {
            free(perm);
            return 1;
        }
        for (f = 0; f < N; f++) {
            memcpy(w_out + f * K, w + perm[f] * K, (size_t)K);
            memcpy(codes_out + f * KB, codes + perm[f] * KB, (size_t)KB);
        }
    } else {
        const int64_t crows = layout == ORC_BLK32 ? N / 32 : N;
        if (K % heads != 0 || (layout == ORC_BLK32 && N % 32 != 0))
            return 1;
        perm = malloc((size_t)K * sizeof *perm);
        if (orc_o_fused_perm(heads, K / heads, perm)) {
            free(perm);
            return 1;
        }
        for (n = 0; n < N; n++)
            for (f = 0; f < K; f++)
                w_out[n * K + f] = w[n * K + perm[f]];
        for (n = 0; n < crows; n++)
            for (f = 0; f < KB; f++)
                codes_out[n * KB + f] = codes[n * KB + perm[32 * f] / 32];
    }
    free(perm);
    return 0;
}

/* SiLU, v * sigmoid(v) = v / (1 + e^-v), in binary64.  The pages pair each
 * gate row with its up row (moe_copies) for the routed experts' up-gate
 * product; the gated activation they feed is read as SiLU, the activation of
 * the DeepSeek-family MoE these pages belong to (reading R18). */
double orc_silu(double v)
{
    return v / (1.0 + exp(-v));
}

/* Round a binary64 value to the nearest bf16 (ties to even), as bits.  The
 * MoE block hands its hidden activation h on in the activation dtype, bf16
 * ([rocm_native] apply_weights: outputs in the input dtype).  bf16 has 8
 * significant bits and binary32's exponent range: a value in [2^(x-1), 2^x)
 * lies on the grid 2^(x-8); below 2^-126 the grid is 2^-133 (subnormals). */
uint16_t orc_bf16_round(double v)
{
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v), step, q, r, res;
    float f;
    uint32_t u;
    int x;
    if (isnan(v))
        return 0x7FC0;
    if (a == 0.0)
        return sign;
    frexp(a, &x);                              /* a in [2^(x-1), 2^x) */
    step = x - 1 >= -126 ? ldexp(1.0, x - 8) : ldexp(1.0, -133);
    q = a / step;                              /* exact: step is a power of two */
    r = floor(q);
    if (q - r > 0.5 || (q - r == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    res = r * step;
    if (res > 3.3895313892515355e38)           /* above the largest bf16: Inf */
        return sign | 0x7F80;
    f = (float)res;                            /* exact: res is on the bf16 grid */
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/* The up-gate product of the routed experts over the interleaved copies:
 * for every token t, slot k with expert e = ids[t][k] in [0, E), and i < inter,
 *   g = x[t] . Wf[e][2 i]^T,  u = x[t] . Wf[e][2 i + 1]^T   (binary64 sums),
 *   h[t][k][i] = silu(g) * u;
 * zero rows for ids outside [0, E) (R5).  w13: [E, 2 inter, K(/2)] standard
 * layout with ROW32 codes [E 2 inter, K / 32]. */
void orc_moe_gate_up(int elem, int64_t E, int64_t inter, int64_t K, const uint8_t *w13,
                     const uint8_t *codes, int64_t T, int64_t topk, const uint16_t *x,
                     int64_t ldx, const int32_t *ids, double *h)
{
    const int64_t N = 2 * inter;
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < inter; i++) {
        int64_t t, k, kk;
        for (t = 0; t < T; t++)
            for (k = 0; k < topk; k++) {
                const int32_t e = ids[t * topk + k];
                double g = 0.0, u = 0.0;
                if (e >= 0 && e < E)
                    for (kk = 0; kk < K; kk++) {
                        const double a = orc_bf16_value(x[t * ldx + kk]);
                        g += a * orc_weight(elem, ORC_ROW32, E, N, K, w13, codes, e, 2 * i, kk);
                        u += a * orc_weight(elem, ORC_ROW32, E, N, K, w13, codes, e, 2 * i + 1, kk);
                    }
                h[(t * topk + k) * inter + i] = (e >= 0 && e < E) ? orc_silu(g) * u : 0.0;
            }
    }
}

/* The grouped linear with one activation row per routed slot (the down
 * projection of the MoE block reads the hidden row h[t][k] of its slot):
 *   y[t][k][:] = a[t topk + k] . Wf[ids[t][k]]^T             (per slot), or
 *   out[t][:]  = sum_k weight[t][k] y[t][k][:], k ascending  (combined),
 * binary64, zero rows for ids outside [0, E).  a: bf16 [T topk, lda]. */
void orc_moe_linear_rows(int elem, int64_t E, int64_t N, int64_t K, const uint8_t *w,
                         const uint8_t *codes, int64_t T, int64_t topk,
                         const uint16_t *a, int64_t lda, const int32_t *ids,
                         const float *weights, double *y)
{
    int64_t n;
    int64_t rows = weights ? T : T * topk;
    memset(y, 0, sizeof(double) * (size_t)(rows * N));
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; n++) {
        int64_t t, k, kk;
        for (t = 0; t < T; t++)
            for (k = 0; k < topk; k++) {
                int32_t e = ids[t * topk + k];
                double s = 0.0;
                if (e >= 0 && e < E)
                    for (kk = 0; kk < K; kk++)
                        s += orc_bf16_value(a[(t * topk + k) * lda + kk]) *
                             orc_weight(elem, ORC_ROW32, E, N, K, w, codes, e, n, kk);
                if (weights)
                    y[t * N + n] += (double)weights[t * topk + k] * s;
                else
                    y[(t * topk + k) * N + n] = s;
            }
    }
}

/* Threads the OpenMP loops above use (1 without OpenMP). */
int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of threads the OpenMP loops above use from now on (the
 * benchmark's CPU baseline times one thread and all of them); returns the
 * previous count.  Without OpenMP it does nothing and returns 1. */
int orc_set_threads(int n)
{
#ifdef _OPENMP
    const int prev = omp_get_max_threads();
    if (n > 0) omp_set_num_threads(n);
    return prev;
#else
    (void)n;
    return 1;
#endif
}
