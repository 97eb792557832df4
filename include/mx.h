/*
 * mx.h -- C ABI of libmx: the block-scaled (OCP microscaling, "MX") linear
 * layer y = x . W^T on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [weights942]   vllm.models.deepseek_v41.amd.mono.weights942
 *   [rocm_native]  vllm.model_executor.kernels.linear.mxfp8.rocm_native
 *   [a16w4]        vllm.models.minimax_m3.amd.specialized_decode.mono.a16w4
 *   [fused_layout] vllm.models.deepseek_v41.common.ops.fused_layout
 *
 * Number formats.
 *   E4M3   OCP fp8 byte (bias 7, max 448, 0x7F/0xFF NaN)        [weights942]
 *   E2M1   OCP fp4 nibble, two per byte, low nibble = even K       [a16w4] dequant
 *   E8M0   scale code c meaning 2^(c - 127), 255 = NaN            [weights942] ocp_from_dequant
 *   bf16   activations, bias and outputs
 * Every 32 consecutive K values of a weight row share one E8M0 code, laid out
 * either one code per row and block (ROW32, [E*N, K/32]) or one code per
 * 32 rows x 32 K block (BLK32, [E*N/32, K/32]) ([rocm_native]
 * process_weights_after_loading and _as_block32_scale).
 *
 * Conventions for every entry point.
 *   - Pointers marked (device) are device memory of the current HIP device;
 *     (host) are host memory.  The caller allocates and owns every buffer;
 *     the library never allocates device memory in these calls.
 *   - All device work is enqueued on `stream` (0 = the null stream) and the
 *     calls return without synchronizing, except the load-time calls that
 *     read back a validity flag: mx_pack_weights, mx_fold_row_codes,
 *     mx_e4m3_from_dequant and mx_moe_copies.
 *   - Arguments are validated on the host before anything is launched; on an
 *     error nothing is launched and outputs are untouched.
 *   - Each call checks that the current device is gfx950 (MX_ERR_DEVICE).
 *   - Inputs holding NaN or Inf give unspecified outputs.
 */
#ifndef MX_H
#define MX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *mx_stream_t; /* same type as hipStream_t */

typedef enum {
    MX_OK = 0,
    MX_ERR_NULL = 1,        /* a required pointer is NULL                      */
    MX_ERR_SHAPE = 2,       /* a size or leading dimension breaks the rules    */
    MX_ERR_ALIGN = 3,       /* a pointer or leading dimension is misaligned    */
    MX_ERR_VALUE = 4,       /* an E8M0 weight code 255 (NaN) was found at pack */
    MX_ERR_UNSUPPORTED = 5, /* a format / layout / mode combination not built  */
    MX_ERR_DEVICE = 6,      /* the current device is not gfx950 (or none)     */
    MX_ERR_WORKSPACE = 7,   /* the workspace is NULL or smaller than required  */
    MX_ERR_LAUNCH = 8       /* a HIP call or kernel launch failed              */
} mx_status;

typedef enum { MX_E4M3 = 0, MX_E2M1 = 1 } mx_elem;
typedef enum { MX_SCALE_ROW32 = 0, MX_SCALE_BLK32 = 1 } mx_scale_layout;
/* Activation scale rules ([rocm_native] _quant_mxfp8_tile and OCP MX v1.0):
 *   MX_RULE_OCP      code = clamp(floor(log2 amax) - 8 + 127, 0, 254); the
 *                    scaled elements are rounded to nearest-even e4m3 and
 *                    saturated to +-448.
 *   MX_RULE_CEIL448  code = clamp(ceil(log2(max(amax, 2^-126) / 448)) + 127,
 *                    0, 254); the scaled elements never exceed 448.
 * Either way a block whose amax is 0 gets code 0, and a zero element keeps
 * its sign (-0 -> 0x80). */
typedef enum { MX_RULE_OCP = 0, MX_RULE_CEIL448 = 1 } mx_quant_rule;
/* MX_ACT_BF16: activations stay bf16 (A16W8 / A16W4).
 * MX_ACT_MXFP8: activations are MXFP8, e4m3 bytes [M, K] with row-major
 * E8M0 codes [M, K/32] ([rocm_native] input_quant_key: row-major, not
 * swizzled), either given pre-quantized or quantized inside the call (W8A8).
 * MX_ACT_MXFP8_T16: MXFP8 activations pre-quantized by mx_quant_act_t16 into
 * the library's 16-token tile layout (below); the same values as
 * MX_ACT_MXFP8, stored the way the matrix cores read them, so a quantized
 * activation can be shared by several linears without re-reading it
 * row-major. */
typedef enum { MX_ACT_BF16 = 0, MX_ACT_MXFP8 = 1, MX_ACT_MXFP8_T16 = 2 } mx_act;

/*
 * T16 activation layout (this library's own; the values are those of
 * mx_quant_act).  S = ceil(K / 128) steps, Q = ceil(S / 4), MB = ceil(M / 16)
 * token tiles, lane l = 16 j + r:
 *   xq     MB * S * 2048 bytes: byte ((mb S + s) 2 + h) 1024 + 16 l + c is
 *          the e4m3 value of token 16 mb + r at K 128 s + 64 h + 16 j + c;
 *   xcodes MB * Q * 256 bytes: byte (mb Q + q) 256 + 4 l + u is the code of
 *          token 16 mb + r, block 4 (4 q + u) + j.
 * Tokens past M and K past the end hold byte 0 and code 127.
 */

/*
 * Packed weight layout ("W-T16", [weights942] dense_copy / fp4_tile_major
 * tile-major idea; [a16w4] module notes for E2M1).
 *   S = ceil(K / 128) steps, T = N / 16 tiles, Q = ceil(S / 4).  Lane
 *   l = 16 j + r.  A tile holds exactly 16 row lengths, TILEB = 16 K (E4M3)
 *   or 8 K (E2M1) bytes: no padding is stored.  When K % 128 != 0 the last
 *   step's chunk holds only its valid bytes, which are the chunk's first
 *   512 (E4M3) or 256 (E2M1) bytes per 32-K block present.
 *   E4M3: chunk (e, t, s) of 2048 bytes at (e T + t) TILEB + 2048 s;
 *         byte 1024 h + 16 l + c = W[e][16 t + r][128 s + 64 h + 16 j + c].
 *   E2M1: chunk (e, t, s) of 1024 bytes at (e T + t) TILEB + 1024 s;
 *         byte 16 l + c = packed byte 64 s + 16 j + c of row 16 t + r.
 *   Codes are padded to 4 Q steps per row (group) with code 128
 *   ([weights942] dense_copy pads its steps).
 * Packed codes:
 *   ROW32: 256 bytes per (e, t, q) at ((e T + t) Q + q) * 256;
 *          byte 4 l + u = code[e N + 16 t + r][4 (4 q + u) + j].
 *   BLK32: 16 bytes per (32-row group R, q) at (R Q + q) * 16, R < E N / 32;
 *          byte 4 j + u = code[R][4 (4 q + u) + j].
 *   Then a 16-byte trailer: byte 0 is the smallest and byte 1 the largest of
 *   the codes given to the pack (padding codes not counted), bytes 2..15
 *   are 0.  The bf16-activation products read it to learn whether every
 *   scaled weight is a normal bf16 number (below).
 * Each lane group j reads one dword per quad of steps, whose byte u is the
 * code of step 4 q + u: the scaled MFMA's byte select picks it directly.
 */

/* Sizes of the packed buffers for a weight of E experts x [N, K].
 * Rules: E >= 1, K >= 32 and K % 32 == 0, N % 16 == 0 (N % 32 == 0 for
 * BLK32).  w_bytes, code_bytes (host) receive the sizes.
 * Errors: MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_UNSUPPORTED (unknown enum). */
mx_status mx_packed_sizes(int elem, int layout, int64_t E, int64_t N, int64_t K,
                          size_t *w_bytes, size_t *code_bytes);

/* Load-time repack ([weights942] dense_copy, fp4_tile_major,
 * codes_tile_rounds; [rocm_native] process_weights_after_loading).
 *   w      (device) standard weight bytes: E4M3 [E, N, K], E2M1 [E, N, K/2]
 *   codes  (device) ROW32 [E N, K/32] or BLK32 [E N / 32, K / 32]
 *   w_packed, codes_packed (device) outputs of mx_packed_sizes' sizes
 *   ws     (device) at least 256 bytes of scratch
 * All device pointers 16-byte aligned.  This call synchronizes `stream`: it
 * reads back whether any code is 255 and returns MX_ERR_VALUE if so (the
 * packed outputs are then written but must not be used). */
mx_status mx_pack_weights(int elem, int layout, int64_t E, int64_t N, int64_t K,
                          const void *w, const void *codes, void *w_packed,
                          void *codes_packed, void *ws, size_t ws_bytes,
                          mx_stream_t stream);

/* ---- Ingest of checkpoint forms the packs do not take directly ---- */

/* Fold row-expanded codes back into 32 x 32 block codes ([rocm_native]
 * _as_block32_scale; [weights942] linear_copy): a loader that repeats each
 * 32 x 32 block's E8M0 code over the block's 32 rows hands back [N, K/32]
 * codes; the block codes are then BLK32 codes for mx_pack_weights.
 *   codes_row (device) [N, ldc] bytes, the first K/32 of each row used
 *   codes_blk (device) [N/32, K/32] output: codes_blk[R][b] = codes_row[32 R][b]
 *   ws        (device) at least 256 bytes of scratch, 16-byte aligned
 * Rules: N % 32 == 0, K % 32 == 0, ldc >= K/32.
 * Errors: MX_ERR_VALUE when some block's 32 rows do not all hold the same
 *   code (the output is still written as above but is not the block form;
 *   keep the row codes, ROW32).  Load-time: synchronizes `stream`. */
mx_status mx_fold_row_codes(int64_t N, int64_t K, const void *codes_row, int64_t ldc,
                            void *codes_blk, void *ws, size_t ws_bytes,
                            mx_stream_t stream);

/* The e4m3 bytes behind a weight the loader dequantized to bf16
 * ([weights942] ocp_from_dequant): w[n][k] = dec(byte) * 2^(c - 127), c the
 * code of the weight's block.
 *   layout  MX_SCALE_ROW32 (codes [N, K/32]) or MX_SCALE_BLK32 ([N/32, K/32])
 *   w_bf16  (device) [N, ldw] bf16, 16-byte aligned, ldw % 8 == 0
 *   codes   (device) the codes the weight was dequantized with
 *   w_out   (device) [N, K] e4m3 bytes, 16-byte aligned
 *   ws      (device) at least 256 bytes of scratch, 16-byte aligned
 * A weight is recovered only when some finite e4m3 byte times 2^(c - 127)
 * equals it exactly; a zero keeps its sign (-0 -> 0x80).
 * Errors: MX_ERR_VALUE when some weight is not recovered -- not of that
 *   form, NaN, infinite, or under code 255 (NaN).  Its output byte is then
 *   0xFF (an e4m3 NaN, never a recovered value); every other byte is still
 *   recovered.  Load-time: synchronizes `stream`. */
mx_status mx_e4m3_from_dequant(int layout, int64_t N, int64_t K, const void *w_bf16,
                               int64_t ldw, const void *codes, void *w_out, void *ws,
                               size_t ws_bytes, mx_stream_t stream);

/* Load-time permutations of an MXFP8 linear for an attention kernel's
 * layouts ([fused_layout]: applied once to the weights, so the linear itself
 * produces or consumes the kernel's layout).
 *   kind MX_PERM_Q_ROWS ([fused_layout] permute_wq_b_, q_fused_permutation):
 *     the weight's N = heads * D output rows, cut per head into 16-row chunks,
 *     reordered chunk-major: output row (d / 16) heads 16 + h 16 + d % 16 is
 *     input row h D + d; its ROW32 codes move with their rows (BLK32 codes
 *     cannot: a 32-row block would hold two heads -> MX_ERR_UNSUPPORTED).
 *     Rules: N % heads == 0, D % 16 == 0.
 *   kind MX_PERM_O_COLS ([fused_layout] permute_wo_a_, o_fused_permutation):
 *     the K = heads * D input columns (one group of heads), cut per head into
 *     32-column chunks, reordered chunk-major: output column (c heads + h) 32
 *     + j is input column h D + 32 c + j; each code column (ROW32 or BLK32)
 *     moves with its 32-column chunk.  Rules: K % heads == 0, D % 32 == 0.
 *   w, w_out       (device) E4M3 bytes [N, K], 16-byte aligned, distinct
 *   codes, codes_out (device) ROW32 [N, K/32] or BLK32 [N/32, K/32]
 * Out of place; pack the outputs with mx_pack_weights.  Asynchronous. */
typedef enum { MX_PERM_Q_ROWS = 0, MX_PERM_O_COLS = 1 } mx_perm_kind;
mx_status mx_fused_layout_permute(int kind, int layout, int64_t N, int64_t K, int64_t heads,
                                  const void *w, const void *codes, void *w_out,
                                  void *codes_out, mx_stream_t stream);

/* Per-token MXFP8 activation quantization ([rocm_native] _quant_mxfp8_tile;
 * rule as in mx_quant_rule).
 *   x      (device) bf16 [M, ldx], 16-byte aligned, ldx % 8 == 0, ldx >= K
 *   xq     (device) e4m3 [M, ldq], 16-byte aligned, ldq % 16 == 0, ldq >= K
 *   xcodes (device) E8M0 [M, ldc], ldc >= K / 32
 * Rules: M >= 1, K >= 32, K % 32 == 0.  Bytes and codes are bit-exact with
 * the rule's definition. */
mx_status mx_quant_act(int64_t M, int64_t K, const void *x, int64_t ldx,
                       void *xq, int64_t ldq, void *xcodes, int64_t ldc,
                       int rule, mx_stream_t stream);

/* Sizes (host) of the T16 quantized activation of M tokens x K.
 * Rules: M >= 1, K >= 32, K % 32 == 0. */
mx_status mx_act_t16_sizes(int64_t M, int64_t K, size_t *xq_bytes, size_t *xcodes_bytes);

/* Per-token MXFP8 quantization into the T16 layout: the same bytes and codes
 * as mx_quant_act, rearranged ([rocm_native] _quant_mxfp8_tile).
 *   x      (device) bf16 [M, ldx], 16-byte aligned, ldx % 8 == 0, ldx >= K
 *   xq, xcodes (device) outputs of mx_act_t16_sizes' sizes, 16-byte aligned
 * Every byte of both outputs is written. */
mx_status mx_quant_act_t16(int64_t M, int64_t K, const void *x, int64_t ldx, void *xq,
                           void *xcodes, int rule, mx_stream_t stream);

/* Workspace bytes mx_linear needs for these arguments (0 when none):
 *   act == MX_ACT_MXFP8 quantized inside the call (prequantized = 0): the
 *     T16 activation, round256(MB * S * 2048) + MB * Q * 256;
 *   act == MX_ACT_MXFP8 pre-quantized row-major with M > 64 (prefill GEMM):
 *     the same size: the GEMM reads the T16 layout, so the bytes and codes
 *     are restaged into it (0 in the batch-invariant mode, where the GEMV
 *     reads them as given: see mx_set_batch_invariant);
 *   otherwise 0 (MX_ACT_BF16, MX_ACT_MXFP8_T16, or pre-quantized M <= 64).
 * (K > 8192 with M <= 64 quantized inside the call is the exception: the
 * row-major staging round256(M * Kp) + round256(M * Kp / 32).)
 * E4M3 with M <= 64 quantized inside the call needs none when K % 128 == 0
 * and the decode GEMV's launch plan divides the shape evenly (eight
 * wavefronts of S / 8 steps each, S in {8, 16, 32, 56, 64}, whole tiles per
 * workgroup): the quantization then runs inside the GEMV, with the same bytes
 * and codes as mx_quant_act ([rocm_native] apply_weights fuses it at tiny
 * M).  The environment variable MX_FUSED_QUANT=0, read once per process,
 * turns that off; this function and mx_linear always agree. */
mx_status mx_linear_workspace(int elem, int layout, int64_t N, int64_t K,
                              int64_t M, int act, int prequantized,
                              size_t *bytes);

/* y[M, N] = a . Wf^T (+ bias), bf16 out, fp32 accumulation, one final
 * round to nearest-even bf16 ([rocm_native] apply_weights).
 * Every E8M0 code 0 .. 254 is served exactly on every path: products and
 * partial sums are formed without loss wherever they lie in fp32's normal
 * range.  With bf16 activations the weights are decoded to bf16 with their
 * scale; when a code lies outside 10 .. 246 (E4M3) or 2 .. 252 (E2M1), where
 * a scaled weight would leave bf16's normal range, that work is done on each
 * 32-K block's partial with the scale applied in fp32 instead (slower; such
 * codes mean weights beyond 2^120 or below 2^-117).
 *   Wf[n][k] = dec(W[n][k]) * 2^(code(n, k) - 127) from the packed buffers.
 *   a = x (bf16) when act == MX_ACT_BF16;
 *   a = dec(xq) * 2^(xcode - 127) when act == MX_ACT_MXFP8: if xq and xcodes
 *       are both non-NULL they are used as given (pre-quantized, row-major
 *       codes); otherwise x is quantized first with `rule` into ws;
 *   the same with xq, xcodes in the T16 layout when act == MX_ACT_MXFP8_T16
 *       (ldq, ldc, x and rule unused).
 *   w_packed, codes_packed (device) from mx_pack_weights with the same
 *       elem, layout, E = 1, N, K.
 *   x   (device) bf16 [M, ldx]: 16-byte aligned, ldx % 8 == 0, ldx >= K
 *   xq  (device) e4m3 [M, ldq]: 16-byte aligned, ldq % 16 == 0, ldq >= K
 *   xcodes (device) [M, ldc], ldc >= K / 32
 *   bias (device, nullable) bf16 [N]
 *   y   (device) bf16 [M, ldy]: 16-byte aligned, ldy % 8 == 0, ldy >= N
 *   ws  (device) at least mx_linear_workspace's bytes, 16-byte aligned
 *       (may be NULL when that is 0); its contents on return are unspecified
 * The call is asynchronous on `stream`, allocates nothing and may be
 * captured in a graph.
 * Size limit: every buffer a kernel reads or writes (x, xq, y, the packed
 * weights) must stay below 2 GiB (32-bit buffer offsets), else MX_ERR_SHAPE.
 * Built combinations: E4M3 x {ROW32, BLK32} x {BF16, MXFP8, MXFP8_T16};
 * E2M1 x ROW32 x BF16.  Others: MX_ERR_UNSUPPORTED. */
mx_status mx_linear(int elem, int layout, int64_t N, int64_t K,
                    const void *w_packed, const void *codes_packed, int64_t M,
                    int act, int rule, const void *x, int64_t ldx,
                    const void *xq, int64_t ldq, const void *xcodes,
                    int64_t ldc, const void *bias, void *y, int64_t ldy,
                    void *ws, size_t ws_bytes, mx_stream_t stream);

/* Workspace bytes mx_moe_linear needs: T * topk * N * 4 when topk_weights is
 * used (combine mode), else 0. */
mx_status mx_moe_workspace(int elem, int64_t E, int64_t N, int64_t K,
                           int64_t T, int64_t topk, int combine,
                           size_t *bytes);

/* Grouped MoE linear over routed experts ([weights942] moe_copies: expert
 * tensors [E, N, K(/2)] with codes [E N, K/32]; [a16w4] module notes):
 *   per slot (topk_weights == NULL): y[t][k][:] = x[t] . Wf[id[t][k]]^T,
 *       y bf16 [T, topk, N] contiguous;
 *   combined (topk_weights != NULL): y[t][:] = sum_k w[t][k] y_slot[t][k][:]
 *       summed in k order in fp32, y bf16 [T, N] contiguous.
 *   w_packed, codes_packed (device) from mx_pack_weights(elem, ROW32, E, N, K)
 *   x (device) bf16 [T, ldx], 16-byte aligned, ldx % 8 == 0, ldx >= K
 *   topk_ids (device) int32 [T, topk]; an id outside [0, E) gives a zero row
 *   topk_weights (device, nullable) fp32 [T, topk]
 * Rules: T >= 1, 1 <= topk <= E, T * topk <= 4096.  Experts that receive no
 * token read no weight bytes.  Built: E2M1 and E4M3 weights, bf16 x. */
mx_status mx_moe_linear(int elem, int64_t E, int64_t N, int64_t K,
                        const void *w_packed, const void *codes_packed,
                        int64_t T, int64_t topk, const void *x, int64_t ldx,
                        const int32_t *topk_ids, const float *topk_weights,
                        void *y, void *ws, size_t ws_bytes,
                        mx_stream_t stream);

/* mx_moe_linear for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same product with the same kernels and results, but no workspace
 * argument.  The combine's per-slot sums (T * topk * N fp32) go to a device
 * buffer the library holds (4 MiB per GPU, kept until the process ends), so
 * combine mode needs T * topk * N <= 1,048,576; per-slot mode uses no
 * buffer.  The call allocates nothing.  Every call on one GPU shares that
 * buffer: calls that overlap on one GPU (two streams, two threads) race and
 * must be ordered by the caller.  The buffer's contents need no clearing
 * (every value is written before it is read).
 * Errors: as mx_moe_linear; MX_ERR_WORKSPACE when the combine would need
 * more than 4 MiB (checked on the host before any device call). */
mx_status mx_moe_linear_noalloc(int elem, int64_t E, int64_t N, int64_t K,
                                const void *w_packed, const void *codes_packed,
                                int64_t T, int64_t topk, const void *x, int64_t ldx,
                                const int32_t *topk_ids, const float *topk_weights,
                                void *y, mx_stream_t stream);

/* ---- The MoE block around the grouped linear ---- */

/* Load-time expert copies ([weights942] moe_copies).  Input, as a model's
 * checkpoint holds the MoE experts (standard layouts, elem E2M1 or E4M3):
 *   w13 (device) [E, 2 Np, rowb] bytes, rowb = K/2 (E2M1) or K (E4M3): gate
 *       rows 0 .. inter-1, zero rows to Np, up rows Np .. Np+inter-1, zero
 *       rows to 2 Np;  s13 (device) codes [E, 2 Np, K/32];
 *   w2  (device) [E, H, Np values] (Np/2 or Np bytes a row), zero beyond
 *       inter;  s2 (device) codes [E, H, Np/32].
 * Output (device, caller-owned, 16-byte aligned):
 *   w13_out [E, 2 inter, rowb]: gate and up rows interleaved, the even row
 *       2 i holding gate row i and the odd row after it up row i,
 *   s13_out [E, 2 inter, K/32] alike, w2_out [E, H, inter values],
 *   s2_out [E, H, inter/32].
 * Bytes are copied verbatim (-0 nibbles kept).  Then pack them with
 * mx_pack_weights(elem, ROW32, E, 2 inter, K, ...) and
 * mx_pack_weights(elem, ROW32, E, H, inter, ...).
 * Rules: inter % 32 == 0, Np % 32 == 0, inter <= Np, K % 32 == 0, E, H >= 1;
 *   ws (device) at least 256 bytes of scratch.
 * Errors: MX_ERR_VALUE (nothing copied) when a padding byte of w13 or w2 is
 *   not zero, as the page refuses it.  Load-time: the call reads the padding
 *   check back and synchronizes `stream`. */
mx_status mx_moe_copies(int elem, int64_t E, int64_t Np, int64_t inter, int64_t K,
                        int64_t H, const void *w13, const void *s13, const void *w2,
                        const void *s2, void *w13_out, void *s13_out, void *w2_out,
                        void *s2_out, void *ws, size_t ws_bytes, mx_stream_t stream);

/* Up-gate product of the routed experts with the gated activation fused
 * ([weights942] moe_copies pairs each gate row with its up row; the
 * activation is read as SiLU):
 *   h[t k][i] = silu(x[t] . gate_e[i]^T) * (x[t] . up_e[i]^T),  e = id[t][k],
 * fp32 accumulation, silu in fp32, one bf16 rounding.
 *   w13_packed, codes_packed (device): mx_pack_weights(elem, ROW32, E,
 *       2 inter, K) of mx_moe_copies' w13_out / s13_out
 *   x (device) bf16 [T, ldx] as in mx_moe_linear
 *   h (device) bf16 [T topk, ldh], 16-byte aligned, ldh % 8 == 0, ldh >= inter;
 *       a slot whose id is outside [0, E) gets a zero row
 * Rules as mx_moe_linear, with N = 2 inter (inter % 8 == 0). */
mx_status mx_moe_gate_up(int elem, int64_t E, int64_t inter, int64_t K,
                         const void *w13_packed, const void *codes_packed,
                         int64_t T, int64_t topk, const void *x, int64_t ldx,
                         const int32_t *topk_ids, void *h, int64_t ldh,
                         mx_stream_t stream);

/* Down projection of the routed experts on the per-slot hidden rows:
 *   per slot: y[t][k][:] = h[t topk + k] . W2_e^T,  e = id[t][k];
 *   combined (topk_weights != NULL): y[t][:] = sum_k w[t][k] y_slot[t][k][:]
 * (as mx_moe_linear, whose workspace rule applies: mx_moe_workspace(elem, E,
 * H, inter, T, topk, combine)).
 *   w2_packed, codes_packed (device): mx_pack_weights(elem, ROW32, E, H,
 *       inter) of mx_moe_copies' w2_out / s2_out
 *   h (device) bf16 [T topk, ldh] (mx_moe_gate_up's output) */
mx_status mx_moe_down(int elem, int64_t E, int64_t H, int64_t inter,
                      const void *w2_packed, const void *codes_packed,
                      int64_t T, int64_t topk, const void *h, int64_t ldh,
                      const int32_t *topk_ids, const float *topk_weights,
                      void *y, void *ws, size_t ws_bytes, mx_stream_t stream);

/* Batch-invariant mode ([rocm_native] process_weights_after_loading: under
 * VLLM_BATCH_INVARIANT the page leaves its block-scaled GEMM, whose split of
 * K varies with M).  Here the decode GEMVs (every A16 call, W8A8 with
 * M <= 64, and the MoE) sum each output in an order fixed by K alone, so a
 * row's result does not depend on the number of rows in the call; W8A8 with
 * M > 64 runs the prefill GEMM, which sums in another order.  With the mode
 * on, W8A8 runs the GEMV for every M: every row's output is then bit-identical
 * to the same row computed in any other call, at the cost of re-reading the
 * weights once per 16 rows.  Process-wide and read at each call; set it before
 * sizing workspaces (mx_linear_workspace depends on it).  The environment
 * variable MX_BATCH_INVARIANT=1 turns it on at start-up.  Returns the previous
 * setting (0 or 1). */
int mx_set_batch_invariant(int on);

/* Static description of a status code (never NULL).
 * Dispatch trace: with the environment variable MX_LOG=1 (read once per
 * process) mx_linear and the MoE entry points write one line to stderr for
 * every kernel they launch, naming the kernel, its launch plan and the
 * shape. */
const char *mx_status_str(mx_status status);

/* Whether an architecture name (e.g. "gfx950:sramecc+:xnack-") is one the
 * kernels are built for; the same test every entry point applies to the
 * current device.  Host only, no device access. */
int mx_arch_supported(const char *gcn_arch_name);

#ifdef __cplusplus
}
#endif
#endif /* MX_H */
