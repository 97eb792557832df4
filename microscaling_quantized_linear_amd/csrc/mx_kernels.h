// mx_kernels.h -- internal interface between the host dispatcher (mx_api.cpp)
// and the gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// the enum values of include/mx.h
enum { E4M3 = 0, E2M1 = 1 };
enum { ROW32 = 0, BLK32 = 1 };
enum { RULE_OCP = 0, RULE_CEIL448 = 1 };
enum { ACT_BF16 = 0, ACT_MXFP8 = 1, ACT_MXFP8_T16 = 2 };

constexpr int kMoeMaxPairs = 4096;   // T * topk handled by one routing scan

struct GemvArgs {
    const uint8_t *w;        // packed W-T16 weights (all experts)
    const uint8_t *codes;    // packed codes
    int64_t E, N, K;
    int64_t rows;            // dense: M tokens; MoE: T tokens
    int64_t topk;            // MoE only
    int64_t xrows;           // rows of the activation buffer
    const void *x;           // bf16 [xrows, ldx] or e4m3 [xrows, ldx]
    int64_t ldx;             // elements
    const uint8_t *xcodes;   // MXFP8 codes [xrows, ldc]
    int64_t ldc;
    const int32_t *ids;      // MoE routing [T, topk]
    const uint16_t *bias;    // bf16 [N] or null
    uint16_t *y;             // bf16 output
    int64_t ldy;
    float *ws;               // MoE combine mode: fp32 per-slot rows [T*topk, N]
    int xslot;               // MoE: activation row of pair i is i (else i / topk)
    int epi;                 // MoE: 1 = silu(row 2i) * row 2i+1 -> output i (width N / 2)
};

struct GemmArgs {
    const uint8_t *w, *codes;
    int64_t N, K, M;
    const uint8_t *xq;       // activation bytes in the T16 data layout
    const uint8_t *xct;      // activation codes in the T16 code layout
    const uint16_t *bias;
    uint16_t *y;
    int64_t ldy;
};

// bytes of the XC-T16 activation-code staging for M rows
__host__ __device__ inline int64_t act_codes_t16_bytes(int64_t M, int64_t K) {
    const int64_t S = (K + 127) / 128, Q = (S + 3) / 4;
    return (M + 15) / 16 * Q * 256;
}
hipError_t launch_act_codes_t16(int64_t M, int64_t K, const void *xc, int64_t ldc, void *out,
                                hipStream_t stream);
// row-major e4m3 activations [M, ldq] restaged into the T16 data layout
hipError_t launch_act_data_t16(int64_t M, int64_t K, const void *xq, int64_t ldq, void *out,
                               hipStream_t stream);

// range: two unsigned counters the codes' smallest / largest value is folded
// into (atomic min / max); the caller sets them to 255 / 0 first
hipError_t launch_pack(int elem, int layout, int64_t E, int64_t N, int64_t K, const void *w,
                       const void *codes, void *wp, void *cp, int *bad, unsigned *range,
                       hipStream_t stream);

// Bytes of packed codes before the 16-byte code-range trailer (byte 0: the
// smallest given code, byte 1: the largest; padding codes not counted).
__host__ __device__ inline int64_t packed_code_body_bytes(int layout, int64_t E, int64_t N,
                                                          int64_t K) {
    const int64_t S = (K + 127) / 128, Q = (S + 3) / 4;
    return layout == 0 ? E * (N / 16) * Q * 256 : E * (N / 32) * Q * 16;
}
constexpr int64_t kCodeTrailer = 16;

// The fixed device buffer of mx_moe_linear_noalloc (mx_static.hip): its size,
// and the current device's address of it (looked up once per device;
// nullptr if the lookup fails).
constexpr int64_t kStaticScratchBytes = int64_t(4) << 20;
void *static_scratch();
// [weights942] moe_copies: the padding check (sets *bad), then the copies
hipError_t launch_moe_padding_check(int elem, int64_t E, int64_t Np, int64_t inter, int64_t K,
                                    int64_t H, const void *w13, const void *w2, int *bad,
                                    hipStream_t stream);
hipError_t launch_moe_copies(int elem, int64_t E, int64_t Np, int64_t inter, int64_t K,
                             int64_t H, const void *w13, const void *s13, const void *w2,
                             const void *s2, void *ow13, void *os13, void *ow2, void *os2,
                             hipStream_t stream);
hipError_t launch_fused_layout(int kind, int64_t N, int64_t K, int64_t heads, int64_t crows,
                               const void *w, const void *codes, void *wo, void *co,
                               hipStream_t st);
hipError_t launch_fold_codes(int64_t N, int64_t KB, int64_t ldc, const void *in, void *out,
                             int *bad, hipStream_t st);
hipError_t launch_e4m3_from_bf16(int layout, int64_t N, int64_t K, const void *w, int64_t ldw,
                                 const void *codes, void *out, int *bad, hipStream_t st);
hipError_t launch_quant(int64_t M, int64_t K, const void *x, int64_t ldx, void *xq, int64_t ldq,
                        void *xcodes, int64_t ldc, int rule, hipStream_t stream);
// Launch shape of the GEMV: nw wavefronts per workgroup (1, 2, 4, 8) split
// the 128-K steps; each issues the loads of `chunk` steps together (2, 4, 8);
// a workgroup owns `tiles` 16-row weight tiles (1, 2, 4) that share the
// activation loads.
struct GemvShape {
    int nw, chunk, tiles;
};
hipError_t launch_gemv(int elem, int layout, int act, bool moe, const GemvArgs &a,
                       const GemvShape &shape, hipStream_t stream);
hipError_t launch_moe_combine(int64_t T, int64_t topk, int64_t N, const float *ys,
                              const float *wts, void *y, hipStream_t stream);
hipError_t launch_gemm(int layout, const GemmArgs &a, hipStream_t stream);
int gemm_tile_n(int64_t N);

// W8A8 decode GEMV (mx_gemv_w8.hip).  Activations either row-major (xq
// [M, ldq], codes xc [M, ldc]) or in the T16 layout (xf, xct; mx_quant.hip).
struct GemvW8Args {
    const uint8_t *w, *codes;      // packed weights and codes (one expert)
    int64_t N, K, M;
    const uint8_t *xq;
    int64_t ldq;
    const uint8_t *xc;
    int64_t ldc;
    const uint8_t *xf, *xct;
    const uint16_t *xb;            // bf16 activations [M, ldx] (fused quantization)
    int64_t ldx;
    const uint16_t *bias;
    uint16_t *y;
    int64_t ldy;
};
// nw wavefronts per workgroup, each with at most spw steps; g tiles per
// workgroup; ok = false if the steps do not fit the register plan
struct GemvW8Plan {
    int nw, spw, g;
    bool ok;
};
GemvW8Plan plan_gemv_w8(int64_t T, int64_t S, int64_t MB, int nw_force, int g_force);
hipError_t launch_gemv_w8(int layout, bool xt16, const GemvW8Args &a, const GemvW8Plan &plan,
                          hipStream_t stream);
// True when the plan divides the shape evenly: eight wavefronts of exactly
// `spw` steps, whole tiles per workgroup.  Then T16 input runs the even-shape
// kernel, and bf16 input with K % 128 == 0 can be quantized inside the GEMV.
bool gemv_w8_even(int64_t N, int64_t K, const GemvW8Plan &plan);
// Per-token quantization fused into the GEMV (a.xb, a.ldx bf16 input; rule as
// in mx_quant_act); requires gemv_w8_even and K % 128 == 0.
hipError_t launch_gemv_w8_fused(int layout, int rule, const GemvW8Args &a,
                                const GemvW8Plan &plan, hipStream_t stream);

// per-token quantization into the T16 layout (mx_quant.hip)
hipError_t launch_quant_t16(int64_t M, int64_t K, const void *x, int64_t ldx, void *xq,
                            void *xc, int rule, hipStream_t stream);
inline int64_t act_t16_data_bytes(int64_t M, int64_t K) {
    return (M + 15) / 16 * ((K + 127) / 128) * 2048;
}

}  // namespace mx
