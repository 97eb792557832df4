// mx_ingest.hip -- load-time ingest of checkpoint forms the packs do not take
// directly.
//
// fold_codes_kernel ([rocm_native] _as_block32_scale, [weights942]
// linear_copy): a loader that repeated each 32 x 32 block's E8M0 code over
// the block's 32 rows hands back [N, K/32] codes; the block form is row 32 R
// of each group, valid when all 32 rows agree.
//
// e4m3_from_bf16_kernel ([weights942] ocp_from_dequant): a loader that
// dequantized e4m3 weights to bf16 (w = e4m3 x 2^(code - 127)) hands back
// bf16; the e4m3 byte is rebuilt from w's exponent and mantissa fields with
// integer arithmetic, and a weight no byte reproduces exactly is marked 0xFF.
//
// fused_q_rows_kernel, fused_o_cols_kernel ([fused_layout] permute_wq_b_,
// permute_wo_a_): an attention kernel's Q and O layouts applied once to the
// rows or input columns of the linears around it, codes moving with them.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

__global__ void __launch_bounds__(256) fold_codes_kernel(int64_t N, int64_t KB, int64_t ldc,
                                                         const uint8_t *__restrict__ in,
                                                         uint8_t *__restrict__ out,
                                                         int *__restrict__ bad) {
    const int64_t n = (N / 32) * KB;
    bool diff = false;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t R = q / KB, b = q % KB;
        const uint8_t c0 = in[32 * R * ldc + b];
#pragma unroll 8
        for (int i = 1; i < 32; ++i) diff |= in[(32 * R + i) * ldc + b] != c0;
        out[q] = c0;
    }
    if (diff) atomicOr(bad, 1);
}

// The finite e4m3 byte whose value times 2^(c - 127) equals the bf16 value
// `bits`, or -1.  Values: e4m3 normal (8 + m) 2^(E - 10), E in 1..15
// (E = 15, m = 7 is NaN); subnormal m 2^-9, m in 1..7; zero keeps its sign.
__device__ inline int e4m3_of_bf16(uint32_t bits, int c) {
    const int sign = (int)((bits >> 8) & 0x80u);
    const int ew = (int)((bits >> 7) & 0xFFu), mw = (int)(bits & 0x7Fu);
    if (c == 255 || ew == 0xFF) return -1;              // NaN scale, Inf, NaN
    if (ew == 0 && mw == 0) return sign;
    // w = M 2^X with an integer M; times 2^(127 - c)
    int M = ew ? (mw | 0x80) : mw;
    int X = (ew ? ew - 134 : -133) + 127 - c;
    const int tz = __builtin_ctz((unsigned)M);
    M >>= tz;
    X += tz;                                             // M odd
    if (M > 15) return -1;                               // more than 4 significant bits
    int s = 0;
    while ((M << s) < 8) ++s;
    const int F = M << s, Ep = X - s;                    // v = F 2^Ep, F in 8..15
    if (Ep > 5) return -1;
    if (Ep >= -9) {
        const int E = Ep + 10, m = F - 8;
        if (E == 15 && m == 7) return -1;
        return sign | (E << 3) | m;
    }
    const int sh = -9 - Ep;                              // subnormal: m = F / 2^sh
    if (sh > 3 || (F & ((1 << sh) - 1))) return -1;
    return sign | (F >> sh);
}

__global__ void __launch_bounds__(256) e4m3_from_bf16_kernel(
    int layout, int64_t N, int64_t K, const uint16_t *__restrict__ w, int64_t ldw,
    const uint8_t *__restrict__ codes, uint8_t *__restrict__ out, int *__restrict__ bad) {
    const int64_t per = K / 8, KB = K / 32, n8 = N * per;
    bool any = false;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n8;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = q / per, k0 = (q % per) * 8;
        const v4u v = *reinterpret_cast<const v4u *>(w + n * ldw + k0);
        const int c = layout == BLK32 ? codes[(n / 32) * KB + k0 / 32] : codes[n * KB + k0 / 32];
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int b = e4m3_of_bf16((v[i / 2] >> (16 * (i % 2))) & 0xFFFFu, c);
            if (b < 0) {
                any = true;
                b = 0xFF;
            }
            o[i / 4] |= (uint32_t)b << (8 * (i % 4));
        }
        *reinterpret_cast<v2u *>(out + n * K + k0) = v2u{o[0], o[1]};
    }
    if (any) atomicOr(bad, 1);
}

// [fused_layout] permute_wq_b_: output row f of the Q layout is standard row
// h D + d with f = (d / 16) H 16 + h 16 + d % 16; whole rows move, with their
// per-row codes.  One thread per 16-byte piece of a row, then per code byte.
__global__ void __launch_bounds__(256) fused_q_rows_kernel(
    int64_t N, int64_t K, int64_t H, const v4u *__restrict__ w,
    const uint8_t *__restrict__ codes, v4u *__restrict__ wo, uint8_t *__restrict__ co) {
    const int64_t D = N / H, P = K / 16, KB = K / 32;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < N * (P + KB);
         q += (int64_t)gridDim.x * blockDim.x) {
        const bool piece = q < N * P;
        const int64_t per = piece ? P : KB, qq = piece ? q : q - N * P;
        const int64_t f = qq / per, b = qq % per;
        const int64_t chunk = f / (H * 16), rem = f % (H * 16);
        const int64_t src = (rem / 16) * D + chunk * 16 + rem % 16;
        if (piece)
            wo[f * P + b] = w[src * P + b];
        else
            co[f * KB + b] = codes[src * KB + b];
    }
}

// [fused_layout] permute_wo_a_: output column chunk fc = c G + h (32 columns)
// is standard chunk h (D / 32) + c; each code column moves with its chunk.
__global__ void __launch_bounds__(256) fused_o_cols_kernel(
    int64_t N, int64_t K, int64_t G, int64_t crows, const v4u *__restrict__ w,
    const uint8_t *__restrict__ codes, v4u *__restrict__ wo, uint8_t *__restrict__ co) {
    const int64_t C = K / 32 / G, P = K / 16, KB = K / 32;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < N * P + crows * KB;
         q += (int64_t)gridDim.x * blockDim.x) {
        const bool piece = q < N * P;
        const int64_t qq = piece ? q : q - N * P;
        const int64_t per = piece ? P : KB, n = qq / per, b = qq % per;
        const int64_t fc = piece ? b / 2 : b;
        const int64_t sc = (fc % G) * C + fc / G;        // standard chunk
        if (piece)
            wo[n * P + b] = w[n * P + 2 * sc + b % 2];
        else
            co[n * KB + b] = codes[n * KB + sc];
    }
}

static unsigned ingest_grid(int64_t n) {
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < 1 ? 1 : (g > 16384 ? 16384 : g));
}

hipError_t launch_fold_codes(int64_t N, int64_t KB, int64_t ldc, const void *in, void *out,
                             int *bad, hipStream_t st) {
    hipLaunchKernelGGL(fold_codes_kernel, dim3(ingest_grid((N / 32) * KB)), dim3(256), 0, st, N,
                       KB, ldc, (const uint8_t *)in, (uint8_t *)out, bad);
    return hipGetLastError();
}

hipError_t launch_e4m3_from_bf16(int layout, int64_t N, int64_t K, const void *w, int64_t ldw,
                                 const void *codes, void *out, int *bad, hipStream_t st) {
    hipLaunchKernelGGL(e4m3_from_bf16_kernel, dim3(ingest_grid(N * (K / 8))), dim3(256), 0, st,
                       layout, N, K, (const uint16_t *)w, ldw, (const uint8_t *)codes,
                       (uint8_t *)out, bad);
    return hipGetLastError();
}

hipError_t launch_fused_layout(int kind, int64_t N, int64_t K, int64_t heads, int64_t crows,
                               const void *w, const void *codes, void *wo, void *co,
                               hipStream_t st) {
    if (kind == 0)
        hipLaunchKernelGGL(fused_q_rows_kernel, dim3(ingest_grid(N * (K / 16 + K / 32))),
                           dim3(256), 0, st, N, K, heads, (const v4u *)w, (const uint8_t *)codes,
                           (v4u *)wo, (uint8_t *)co);
    else
        hipLaunchKernelGGL(fused_o_cols_kernel,
                           dim3(ingest_grid(N * (K / 16) + crows * (K / 32))), dim3(256), 0, st,
                           N, K, heads, crows, (const v4u *)w, (const uint8_t *)codes, (v4u *)wo,
                           (uint8_t *)co);
    return hipGetLastError();
}

}  // namespace mx
