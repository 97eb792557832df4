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
__device__ inline uint32_t act_code(uint32_t amax_bits /* fp32 bits, sign 0 */) {
    const int e = (int)(amax_bits >> 23);          // exponent field; 0 for 0 and subnormals
    int c;
    if (RULE == RULE_OCP) {
        c = e - 8;                                 // floor(log2 amax) - 8 + 127
    } else {
        c = e - 8 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);   // mantissa > 1.75
    }
    if (e == 0) c = 0;                             // amax < 2^-126 -> code 0 (both rules)
    c = c < 0 ? 0 : c;
    return (uint32_t)(c > 254 ? 254 : c);
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

}  // namespace mx
