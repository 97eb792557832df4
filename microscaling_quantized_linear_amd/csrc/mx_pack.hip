// mx_pack.hip -- load-time repacks into the W-T16 weight layout and the
// C-T16 / padded BLK32 code layouts (layouts stated in include/mx.h).
//
// The tile-major weight copy follows the idea of [weights942] dense_copy and
// fp4_tile_major (16-row tiles x 128-K steps, each 16-byte load of a
// wavefront reading 1 KB that is contiguous); the code staging follows
// [weights942] codes_tile_rounds (a lane group reads its rows' codes from one
// line) with the per-lane dwords of [a16w4] scale_loads; BLK32 codes get the
// same dword-per-lane-group, byte-per-step staging.  Codes are padded to
// Kp = 128 * ceil(K / 128) with code 128 ([weights942] dense_copy pads its
// steps); weights store no padding: the valid bytes of a K % 128 tail step
// are a prefix of its chunk, and the chunk is stored cut to them, so a tile
// is exactly 16 row lengths.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

// One thread writes one 16-byte piece of the packed weights (a gather: every
// destination piece is read from exactly one source piece).  A tile holds
// 16 row lengths of bytes; piece o of it is in chunk o / CHUNK.
__global__ void __launch_bounds__(256) pack_weights_kernel(
    int elem, int64_t E, int64_t N, int64_t K, const uint8_t *__restrict__ w,
    uint8_t *__restrict__ wp, int64_t npieces) {
    int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= npieces) return;
    const int64_t T = N / 16;
    const int64_t row_bytes = elem == E4M3 ? K : K / 2;
    const int64_t tile_pieces = row_bytes;                 // 16 rows x row_bytes / 16
    const int64_t et = p / tile_pieces, o = p % tile_pieces;   // et = e * T + t
    int64_t s, lane, kbyte;
    if (elem == E4M3) {             // 128 pieces per 2 KB chunk
        s = o / 128;
        const int64_t h = (o % 128) / 64;
        lane = o % 64;
        kbyte = 64 * h + 16 * (lane / 16);
    } else {                        // 64 pieces per 1 KB chunk
        s = o / 64;
        lane = o % 64;
        kbyte = 16 * (lane / 16);
    }
    const int64_t e = et / T, t = et % T;
    const int64_t row = e * N + 16 * t + lane % 16;
    const int64_t step_bytes = elem == E4M3 ? 128 : 64;
    const int64_t off = s * step_bytes + kbyte;           // byte within the row, < row_bytes
    *reinterpret_cast<v4u *>(wp + p * 16) =
        *reinterpret_cast<const v4u *>(w + row * row_bytes + off);
}

// ROW32: one thread writes one dword (4 codes) of C-T16.  BLK32: one byte.
// Any code 255 sets *bad; range[0] / range[1] collect the smallest and the
// largest given code (padding not counted) for the trailer.
__global__ void __launch_bounds__(256) pack_codes_kernel(
    int layout, int64_t E, int64_t N, int64_t K, const uint8_t *__restrict__ codes,
    uint8_t *__restrict__ cp, int64_t nunits, int *__restrict__ bad,
    unsigned *__restrict__ range) {
    int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t KB = K / 32, Kp = (K + 127) / 128 * 128, S = Kp / 128, Q = (S + 3) / 4;
    const int64_t T = N / 16;
    int found = 0;
    unsigned lo = 255, hi = 0;
    if (p < nunits) {
    if (layout == ROW32) {
        const int64_t lane = p % 64, etq = p / 64;
        const int64_t q = etq % Q, et = etq / Q;
        const int64_t row = (et / T) * N + 16 * (et % T) + lane % 16;
        uint32_t dw = 0;
        for (int u = 0; u < 4; ++u) {
            const int64_t blk = 4 * (4 * q + u) + lane / 16;
            uint32_t c = 128;
            if (blk < KB) {
                c = codes[row * KB + blk];
                found |= c == 255;
                lo = c < lo ? c : lo;
                hi = c > hi ? c : hi;
            }
            dw |= c << (8 * u);
        }
        reinterpret_cast<uint32_t *>(cp)[p] = dw;
    } else {
        // BLK32: per 32-row group and quad, 16 bytes; byte 4 j + u holds
        // block 4 (4 q + u) + j
        const int64_t R = p / (Q * 16), rem = p % (Q * 16);
        const int64_t q = rem / 16, jj = (rem % 16) / 4, u = rem % 4;
        const int64_t b = 4 * (4 * q + u) + jj;
        uint32_t c = 128;
        if (b < KB) {
            c = codes[R * KB + b];
            found = c == 255;
            lo = hi = c;
        }
        cp[p] = (uint8_t)c;
    }
    }
    if (found) atomicOr(bad, 1);
    // the wavefront's range, then one pair of atomics per wavefront
#pragma unroll
    for (int d = 32; d >= 1; d /= 2) {
        const unsigned olo = (unsigned)__shfl_xor((int)lo, d), ohi = (unsigned)__shfl_xor((int)hi, d);
        lo = olo < lo ? olo : lo;
        hi = ohi > hi ? ohi : hi;
    }
    if (threadIdx.x % 64 == 0 && lo <= hi) {
        atomicMin(&range[0], lo);
        atomicMax(&range[1], hi);
    }
}

// Row-major activation codes [M, ldc] -> XC-T16: per 16-row tile and quad of
// four 128-K steps, 256 bytes; lane l = 16 j + r's dword holds row r's code
// of block 4 (4 q + u) + j in byte u (the lane order of the scaled MFMA's
// B-operand scales).  Rows past M and blocks past K/32 get code 127.
__global__ void __launch_bounds__(256) act_codes_t16_kernel(int64_t M, int64_t K,
                                                            const uint8_t *__restrict__ xc,
                                                            int64_t ldc, uint32_t *__restrict__ out,
                                                            int64_t ndw) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= ndw) return;
    const int64_t S = (K + 127) / 128, Q = (S + 3) / 4, KB = K / 32;
    const int64_t lane = p % 64, mq = p / 64, q = mq % Q, mt = mq / Q;
    const int64_t row = 16 * mt + lane % 16, j = lane / 16;
    uint32_t dw = 0;
    for (int u = 0; u < 4; ++u) {
        const int64_t b = 4 * (4 * q + u) + j;
        const uint32_t c = (row < M && b < KB) ? xc[row * ldc + b] : 127u;
        dw |= c << (8 * u);
    }
    out[p] = dw;
}

hipError_t launch_act_codes_t16(int64_t M, int64_t K, const void *xc, int64_t ldc, void *out,
                                hipStream_t stream) {
    const int64_t S = (K + 127) / 128, Q = (S + 3) / 4;
    const int64_t ndw = (M + 15) / 16 * Q * 64;
    hipLaunchKernelGGL(act_codes_t16_kernel, dim3((unsigned)((ndw + 255) / 256)), dim3(256), 0,
                       stream, M, K, (const uint8_t *)xc, ldc, (uint32_t *)out, ndw);
    return hipGetLastError();
}

// Row-major e4m3 activations [M, ldq] -> the T16 data layout: 2,048 bytes
// per (16-token tile mb, 128-K step s); byte 1024 h + 16 l + c (l = 16 j + r)
// holds xq[16 mb + r][128 s + 64 h + 16 j + c].  One thread per 16-byte
// piece; tokens past M and K past the end read as zeros (K is a multiple of
// 32, so a piece is wholly inside or outside).
__global__ void __launch_bounds__(256) act_data_t16_kernel(int64_t M, int64_t K,
                                                           const uint8_t *__restrict__ xq,
                                                           int64_t ldq, v4u *__restrict__ out,
                                                           int64_t npieces) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= npieces) return;
    const int64_t S = (K + 127) / 128;
    const int64_t l = p % 64, blk = p / 64, h = blk % 2, ms = blk / 2, s = ms % S, mb = ms / S;
    const int64_t row = 16 * mb + l % 16, k = 128 * s + 64 * h + 16 * (l / 16);
    out[p] = (row < M && k < K) ? *reinterpret_cast<const v4u *>(xq + row * ldq + k)
                                : v4u{0u, 0u, 0u, 0u};
}

hipError_t launch_act_data_t16(int64_t M, int64_t K, const void *xq, int64_t ldq, void *out,
                               hipStream_t stream) {
    const int64_t npieces = act_t16_data_bytes(M, K) / 16;
    hipLaunchKernelGGL(act_data_t16_kernel, dim3((unsigned)((npieces + 255) / 256)), dim3(256), 0,
                       stream, M, K, (const uint8_t *)xq, ldq, (v4u *)out, npieces);
    return hipGetLastError();
}

hipError_t launch_pack(int elem, int layout, int64_t E, int64_t N, int64_t K, const void *w,
                       const void *codes, void *wp, void *cp, int *bad, unsigned *range,
                       hipStream_t stream) {
    const int64_t Kp = (K + 127) / 128 * 128, S = Kp / 128, Q = (S + 3) / 4;
    const int64_t wbytes = E * N * (elem == E4M3 ? K : K / 2);
    const int64_t npieces = wbytes / 16;
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((npieces + 255) / 256)), dim3(256), 0,
                       stream, elem, E, N, K, (const uint8_t *)w, (uint8_t *)wp, npieces);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t nunits = layout == ROW32 ? E * (N / 16) * Q * 64 : E * (N / 32) * Q * 16;
    hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((nunits + 255) / 256)), dim3(256), 0,
                       stream, layout, E, N, K, (const uint8_t *)codes, (uint8_t *)cp, nunits,
                       bad, range);
    return hipGetLastError();
}

// ---- expert copies for the MoE block ([weights942] moe_copies) ----
// w13 [E, 2 Np, rowb]: gate rows 0 .. inter - 1, zero rows to Np, up rows
// Np .. Np + inter - 1, zero rows to 2 Np.  Copies: row 2 i <- gate row i,
// row 2 i + 1 <- up row i; w2 [E, H, Np values] cut to inter values.  rowb,
// the w2 row bytes and their padding are multiples of 16 (K, inter, Np are
// multiples of 32), so everything but the codes moves in 16-byte pieces.

// one 16-byte piece of padding per thread: w13's zero rows, then w2's zero
// columns; any non-zero byte sets *bad
__global__ void __launch_bounds__(256) moe_padding_kernel(
    const v4u *__restrict__ w13, const v4u *__restrict__ w2, int64_t E, int64_t Np,
    int64_t inter, int64_t rowb16, int64_t r2in16, int64_t r2out16, int64_t H,
    int *__restrict__ bad) {
    const int64_t pad13 = E * 2 * (Np - inter) * rowb16;   // pieces in w13's padding rows
    const int64_t pad2 = E * H * (r2in16 - r2out16);       // pieces in w2's padding columns
    bool found = false;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < pad13 + pad2;
         q += (int64_t)gridDim.x * blockDim.x) {
        v4u v;
        if (q < pad13) {
            const int64_t b = q % rowb16, row = q / rowb16;
            const int64_t per = 2 * (Np - inter), e = row / per, pr = row % per;
            const int64_t src = e * 2 * Np + (pr < Np - inter ? inter + pr : Np + inter + (pr - (Np - inter)));
            v = w13[src * rowb16 + b];
        } else {
            const int64_t q2 = q - pad13, w = r2in16 - r2out16;
            v = w2[(q2 / w) * r2in16 + r2out16 + q2 % w];
        }
        found |= (v[0] | v[1] | v[2] | v[3]) != 0u;
    }
    if (found) atomicOr(bad, 1);
}

__global__ void __launch_bounds__(256) moe_copy_kernel(
    const v4u *__restrict__ w13, const v4u *__restrict__ w2, v4u *__restrict__ ow13,
    v4u *__restrict__ ow2, int64_t E, int64_t Np, int64_t inter, int64_t rowb16,
    int64_t r2in16, int64_t r2out16, int64_t H) {
    const int64_t n13 = E * 2 * inter * rowb16, n2 = E * H * r2out16;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n13 + n2;
         q += (int64_t)gridDim.x * blockDim.x) {
        if (q < n13) {
            const int64_t b = q % rowb16, row = q / rowb16;    // output row e 2 inter + 2 i + g
            const int64_t e = row / (2 * inter), rr = row % (2 * inter);
            const int64_t src = e * 2 * Np + (rr % 2) * Np + rr / 2;
            ow13[q] = w13[src * rowb16 + b];
        } else {
            const int64_t q2 = q - n13;
            ow2[q2] = w2[(q2 / r2out16) * r2in16 + q2 % r2out16];
        }
    }
}

// the codes, one byte per thread: s13 [E, 2 Np, kb] interleaved like the
// rows, s2 [E, H, Np / 32] cut to inter / 32
__global__ void __launch_bounds__(256) moe_copy_codes_kernel(
    const uint8_t *__restrict__ s13, const uint8_t *__restrict__ s2, uint8_t *__restrict__ os13,
    uint8_t *__restrict__ os2, int64_t E, int64_t Np, int64_t inter, int64_t kb, int64_t H) {
    const int64_t n13 = E * 2 * inter * kb, c2in = Np / 32, c2out = inter / 32;
    const int64_t n2 = E * H * c2out;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n13 + n2;
         q += (int64_t)gridDim.x * blockDim.x) {
        if (q < n13) {
            const int64_t b = q % kb, row = q / kb;
            const int64_t e = row / (2 * inter), rr = row % (2 * inter);
            os13[q] = s13[(e * 2 * Np + (rr % 2) * Np + rr / 2) * kb + b];
        } else {
            const int64_t q2 = q - n13;
            os2[q2] = s2[(q2 / c2out) * c2in + q2 % c2out];
        }
    }
}

static unsigned grid_for(int64_t n) {
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

hipError_t launch_moe_padding_check(int elem, int64_t E, int64_t Np, int64_t inter, int64_t K,
                                    int64_t H, const void *w13, const void *w2, int *bad,
                                    hipStream_t st) {
    const int64_t rowb16 = (elem == E2M1 ? K / 2 : K) / 16;
    const int64_t r2in16 = (elem == E2M1 ? Np / 2 : Np) / 16;
    const int64_t r2out16 = (elem == E2M1 ? inter / 2 : inter) / 16;
    const int64_t n = E * 2 * (Np - inter) * rowb16 + E * H * (r2in16 - r2out16);
    hipLaunchKernelGGL(moe_padding_kernel, dim3(grid_for(n)), dim3(256), 0, st,
                       (const v4u *)w13, (const v4u *)w2, E, Np, inter, rowb16, r2in16,
                       r2out16, H, bad);
    return hipGetLastError();
}

hipError_t launch_moe_copies(int elem, int64_t E, int64_t Np, int64_t inter, int64_t K,
                             int64_t H, const void *w13, const void *s13, const void *w2,
                             const void *s2, void *ow13, void *os13, void *ow2, void *os2,
                             hipStream_t st) {
    const int64_t rowb16 = (elem == E2M1 ? K / 2 : K) / 16;
    const int64_t r2in16 = (elem == E2M1 ? Np / 2 : Np) / 16;
    const int64_t r2out16 = (elem == E2M1 ? inter / 2 : inter) / 16;
    const int64_t n = E * 2 * inter * rowb16 + E * H * r2out16;
    hipLaunchKernelGGL(moe_copy_kernel, dim3(grid_for(n)), dim3(256), 0, st, (const v4u *)w13,
                       (const v4u *)w2, (v4u *)ow13, (v4u *)ow2, E, Np, inter, rowb16, r2in16,
                       r2out16, H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nc = E * 2 * inter * (K / 32) + E * H * (inter / 32);
    hipLaunchKernelGGL(moe_copy_codes_kernel, dim3(grid_for(nc)), dim3(256), 0, st,
                       (const uint8_t *)s13, (const uint8_t *)s2, (uint8_t *)os13, (uint8_t *)os2,
                       E, Np, inter, K / 32, H);
    return hipGetLastError();
}

}  // namespace mx
