// mx_quant.hip -- per-token MXFP8 activation quantization.
//
// For every row m and 32-value K block b ([rocm_native] _quant_mxfp8_tile):
//   amax  = max |x| over the block
//   code  = E8M0 code of the block, by one of two rules (include/mx.h):
//             OCP      floor(log2 amax) - 8 + 127
//             CEIL448  ceil(log2(max(amax, 2^-126) / 448)) + 127
//           clamped to [0, 254]
//   xq    = e4m3(x * 2^(127 - code)), nearest-even, saturated to +-448
// The codes are computed from the bits of amax (exact: amax is a bf16 value),
// the multiply by a power of two is exact in fp32 (results below 2^-126 are
// far under half the smallest e4m3 subnormal and round to a signed zero
// either way), and the hardware convert rounds to nearest even.
//
// Work split: four lanes per block, eight bf16 values (one 16-byte load) per
// lane, so a wavefront reads 1 KB of contiguous activations; the block
// maximum is combined across the four lanes with DPP quad permutes.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

__device__ inline uint32_t quad_max(uint32_t v) {
    // DPP quad_perm [1,0,3,2] then [2,3,0,1]: max over the 4 lanes of a quad
    uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
    v = v > o ? v : o;
    o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
    return v > o ? v : o;
}

template <int RULE>
__global__ void __launch_bounds__(256) quant_act_kernel(
    int64_t M, int64_t K, const uint16_t *__restrict__ x, int64_t ldx,
    uint8_t *__restrict__ xq, int64_t ldq, uint8_t *__restrict__ xcodes, int64_t ldc) {
    const int64_t nb = K / 32;
    const int64_t blk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 4;
    const int q = threadIdx.x % 4;
    const bool valid = blk < M * nb;
    const int64_t m = valid ? blk / nb : 0, b = valid ? blk % nb : 0;
    v4u v = {0u, 0u, 0u, 0u};
    if (valid) v = *reinterpret_cast<const v4u *>(x + m * ldx + 32 * b + 8 * q);
    // |x| as fp32 bits: bf16 bits << 16 with the sign cleared; integer order
    // equals numeric order for non-negative finite values
    uint32_t amax = 0;
    for (int i = 0; i < 4; ++i) {
        uint32_t lo = (v[i] & 0x7FFFu) << 16, hi = (v[i] >> 16 & 0x7FFFu) << 16;
        amax = amax > lo ? amax : lo;
        amax = amax > hi ? amax : hi;
    }
    amax = quad_max(amax);
    const uint32_t code = act_code<RULE>(amax);
    // 2^(127 - code) as an fp32 bit pattern; code <= 247 for any bf16 amax,
    // so the exponent field 254 - code stays within [7, 254]
    const float mul = __uint_as_float((254u - code) << 23);
    uint32_t out[2];
    for (int d = 0; d < 2; ++d) {
        float f[4];
        for (int i = 0; i < 2; ++i) {
            uint32_t w = v[2 * d + i];
            f[2 * i] = __uint_as_float(w << 16) * mul;
            f[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u) * mul;
        }
        for (int i = 0; i < 4; ++i) f[i] = __builtin_fminf(__builtin_fmaxf(f[i], -448.0f), 448.0f);
        int packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], packed, true);
        out[d] = (uint32_t)packed;
    }
    if (valid) {
        v2u o = {out[0], out[1]};
        *reinterpret_cast<v2u *>(xq + m * ldq + 32 * b + 8 * q) = o;
        if (q == 0) xcodes[m * ldc + b] = (uint8_t)code;
    }
}

// 16-token tile ("T16") layout of a quantized activation, S = ceil(K / 128)
// steps, Q = ceil(S / 4), MB = ceil(M / 16) tiles, lane l = 16 j + r:
//   xq byte ((mb S + s) 2 + h) 1024 + 16 l + c
//         = e4m3 of token 16 mb + r, K 128 s + 64 h + 16 j + c
//           (one 1 KB block per step half, in the scaled MFMA's operand lane
//           order: a lane's two blocks of a step are its 32 operand bytes);
//   xc byte (mb Q + q) 256 + 4 l + u
//         = code of token 16 mb + r, block 4 (4 q + u) + j
//           (a lane's dword holds its codes of four steps, byte u = step 4 q + u).
// Tokens past M, K past the end and blocks past K/32 read as byte 0 and code
// 127, so every byte of both buffers is defined.
//
// One wavefront per (token tile mb, quad q of four steps): for each of the
// quad's steps s and halves h, lane (r, j) converts 16 values, half of the
// 32-value block 4 s + 2 h + j / 2 (the block maximum is taken with the
// partner lane 16 apart, j xor 1), and the wavefront writes the 1 KB block
// contiguously; then each lane writes its own code dword of the quad (token
// r, block 4 (4 q + u) + j in byte u), gathered from the lanes that computed
// those codes.  All of a lane's loads are issued before its first convert.
template <int RULE>
__global__ void __launch_bounds__(256) quant_act_t16_kernel(
    int64_t M, int64_t K, const uint16_t *__restrict__ x, int64_t ldx,
    uint8_t *__restrict__ xq, uint8_t *__restrict__ xc, int64_t nunits) {
    const int64_t wid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
    if (wid >= nunits) return;                       // whole wavefronts
    const int lane = threadIdx.x % 64, r = lane % 16, j = lane / 16;
    const int64_t S = (K + 127) / 128, Q = (S + 3) / 4, KB = K / 32;
    const int64_t q = wid % Q, mb = wid / Q;
    const int64_t m = 16 * mb + r;
    v4u v[4][2][2];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t k0 = 128 * (4 * q + u) + 64 * h + 16 * j;
            // K % 32 == 0: the lane's 16 values are all inside K or all past it
            const bool ok = m < M && k0 < K;
            v[u][h][0] = ok ? *reinterpret_cast<const v4u *>(x + m * ldx + k0) : v4u{0u, 0u, 0u, 0u};
            v[u][h][1] = ok ? *reinterpret_cast<const v4u *>(x + m * ldx + k0 + 8)
                            : v4u{0u, 0u, 0u, 0u};
        }
    uint32_t code[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t s = 4 * q + u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const v4u o = quant_half_block<RULE>(v[u][h][0], v[u][h][1], code[u][h]);
            if (s < S) *reinterpret_cast<v4u *>(xq + ((mb * S + s) * 2 + h) * 1024 + 16 * lane) = o;
        }
    }
    // lane (r, j) owns block 4 s + j of each step: half j / 2, computed by
    // the lanes 16 (2 (j % 2)) + r and 16 (2 (j % 2) + 1) + r of that half
    const int src = 32 * (j % 2) + r;
    uint32_t dw = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t c0 = (uint32_t)__shfl((int)code[u][0], src);
        const uint32_t c1 = (uint32_t)__shfl((int)code[u][1], src);
        const int64_t blk = 4 * (4 * q + u) + j;
        const uint32_t c = (m < M && blk < KB) ? (j / 2 ? c1 : c0) : 127u;
        dw |= c << (8 * u);
    }
    reinterpret_cast<uint32_t *>(xc)[(mb * Q + q) * 64 + lane] = dw;
}

hipError_t launch_quant(int64_t M, int64_t K, const void *x, int64_t ldx, void *xq, int64_t ldq,
                        void *xcodes, int64_t ldc, int rule, hipStream_t stream) {
    const int64_t threads = M * (K / 32) * 4;
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (rule == RULE_OCP)
        hipLaunchKernelGGL(quant_act_kernel<RULE_OCP>, grid, block, 0, stream, M, K,
                           (const uint16_t *)x, ldx, (uint8_t *)xq, ldq, (uint8_t *)xcodes, ldc);
    else
        hipLaunchKernelGGL(quant_act_kernel<RULE_CEIL448>, grid, block, 0, stream, M, K,
                           (const uint16_t *)x, ldx, (uint8_t *)xq, ldq, (uint8_t *)xcodes, ldc);
    return hipGetLastError();
}

hipError_t launch_quant_t16(int64_t M, int64_t K, const void *x, int64_t ldx, void *xq,
                            void *xc, int rule, hipStream_t stream) {
    const int64_t S = (K + 127) / 128, Q = (S + 3) / 4, nunits = (M + 15) / 16 * Q;
    const dim3 grid((unsigned)((nunits + 3) / 4)), block(256);
    if (rule == RULE_OCP)
        hipLaunchKernelGGL(quant_act_t16_kernel<RULE_OCP>, grid, block, 0, stream, M, K,
                           (const uint16_t *)x, ldx, (uint8_t *)xq, (uint8_t *)xc, nunits);
    else
        hipLaunchKernelGGL(quant_act_t16_kernel<RULE_CEIL448>, grid, block, 0, stream, M, K,
                           (const uint16_t *)x, ldx, (uint8_t *)xq, (uint8_t *)xc, nunits);
    return hipGetLastError();
}

}  // namespace mx
