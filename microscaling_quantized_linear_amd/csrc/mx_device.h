// mx_device.h -- device helpers shared by the gfx950 kernels of libmx.
//
// gfx950 facts the kernels rely on (established with one-instruction probes
// of the hardware and fixed by the parity tests):
//  * v_mfma_scale_f32_16x16x128_f8f6f4 (fp8 operands): lane l = 16 j + r
//    supplies row r; operand bytes 0..15 are K 16 j .. 16 j + 15 of the
//    128-K step and bytes 16..31 are K 64 + 16 j .. + 15; the lane's E8M0
//    scale (byte `opsel` of the scale register) covers K block j of row r.
//  * v_mfma_f32_16x16x32_bf16: lane l supplies row r, K 8 j .. 8 j + 7.
//  * both return D[4 j + i][r] in element i of lane l (16 x 16 tile).
//  * v_cvt_scalef32_pk_* read the scale's exponent field as the E8M0 code,
//    so a code c is passed as the float bit pattern c << 23 (code 0 is
//    2^-127, 255 is NaN).
//  * v_cvt_pk_fp8_f32 rounds to nearest even but does not saturate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding and leaves the export and LDS/scalar counters alone
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
__host__ __device__ constexpr int vmcnt_only(int n) {
    return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 0x3) << 14);
}

// Cache-policy bits of buffer instructions on gfx950: nt (streamed once).
constexpr int kNT = 2;

// Buffer resource over [base, base + bytes): loads past the end return 0,
// so ragged tails need no branches and a wrong offset cannot fault.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Byte offset that is always out of range of a resource (reads give 0).
constexpr uint32_t kOOB = 0x80000000u;

template <int AUX = 0>
__device__ inline v4u load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}
template <int AUX = 0>
__device__ inline uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, AUX);
}
template <int AUX = 0>
__device__ inline uint32_t load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, AUX);
}

// E8M0 code -> the float operand of v_cvt_scalef32_* (exponent field = code).
__device__ inline float code_as_scale(uint32_t code) { return __uint_as_float(code << 23); }

__device__ inline uint32_t byte_of(uint32_t w, uint32_t i) { return (w >> (8 * i)) & 0xFFu; }

// 8 e4m3 bytes (two dwords) x 2^(code-127) -> 8 bf16: exact while every
// product is a normal bf16 number (codes 10 .. 246); callers apply the rest
// of a code outside that range in fp32 (a16_exact_tile).
__device__ inline v8bf dec8_e4m3(uint32_t w0, uint32_t w1, float scale) {
    v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
    v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
    v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
    v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
    v8bf r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

// 8 e2m1 nibbles (one dword, low nibble first) x 2^(code-127) -> 8 bf16
// ([a16w4] dequant: four scaled pair conversions); exact for codes 2 .. 252.
__device__ inline v8bf dec8_e2m1(uint32_t w, float scale) {
    v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    v8bf r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

__device__ inline v8bf as_bf16x8(v4u v) { return __builtin_bit_cast(v8bf, v); }

__device__ inline v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp8 x fp8 with per-lane E8M0 scales taken from byte 0 of sa / sb.
__device__ inline v4f mfma_fp8_scaled(v8i a, v8i b, v4f c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// the same with the scale bytes picked by opsel (byte U of sa and of sb)
template <int U>
__device__ inline v4f mfma_fp8_scaled_sel(v8i a, v8i b, v4f c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, U, sa, U, sb);
}

__device__ inline v8i cat8(v4u lo, v4u hi) {
    v8i r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return r;
}

// bf16 round-to-nearest-even of an fp32 value, as bits.
__device__ inline uint32_t bf16_bits(float f) {
    __bf16 h = (__bf16)f;
    return (uint32_t)__builtin_bit_cast(unsigned short, h);
}

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// ---- per-token MXFP8 quantization of one 32-value block ----
// ([rocm_native] _quant_mxfp8_tile: per token and 32-value K block, amax ->
// E8M0 code -> e4m3 of x * 2^(127 - code))

// E8M0 code of a block from the fp32 bits of its amax (sign 0), by rule
// (0 = OCP: floor(log2 amax) - 8 + 127; 1 = CEIL448: ceil(log2(amax / 448))
// + 127), clamped to [0, 254]; amax below 2^-126 gives code 0.  Exact: amax
// is a bf16 value, and the ceiling adds one exactly when the mantissa is
// above 1.75 (448 = 1.75 * 2^8).
template <int RULE>
__device__ inline uint32_t act_code(uint32_t amax_bits) {
    const int e = (int)(amax_bits >> 23);          // exponent field; 0 for 0 and subnormals
    int c = e - 8;
    if (RULE != 0) c += (amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0;
    if (e == 0) c = 0;
    c = c < 0 ? 0 : c;
    return (uint32_t)(c > 254 ? 254 : c);
}

// Half of a block per lane: the 16 bf16 values v0, v1 (8 each, in K order)
// are one half of a 32-value block whose other half is held by the lane 16
// apart (lane xor 16).  Returns the 16 e4m3 bytes in K order and the block's
// code.  Each value is multiplied by the exact power 2^(127 - code) (results
// below 2^-126 round to a signed zero either way), clamped to +-448 and
// converted with round to nearest even.
template <int RULE>
__device__ inline v4u quant_half_block(v4u v0, v4u v1, uint32_t &code) {
    // |x| as fp32 bits (bf16 bits << 16, sign cleared): integer order is
    // numeric order for non-negative finite values
    uint32_t amax = 0;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = a ? v1[i] : v0[i];
            const uint32_t lo = (w & 0x7FFFu) << 16, hi = (w >> 16 & 0x7FFFu) << 16;
            amax = amax > lo ? amax : lo;
            amax = amax > hi ? amax : hi;
        }
    const uint32_t other = (uint32_t)__shfl_xor((int)amax, 16);
    amax = amax > other ? amax : other;
    code = act_code<RULE>(amax);
    // 2^(127 - code) as fp32 bits; code <= 247 for any bf16 amax, so the
    // exponent field 254 - code stays within [7, 254]
    const float mul = __uint_as_float((254u - code) << 23);
    v4u out;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            float f[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t w = a ? v1[2 * d + i] : v0[2 * d + i];
                f[2 * i] = __uint_as_float(w << 16) * mul;
                f[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u) * mul;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) f[i] = __builtin_fminf(__builtin_fmaxf(f[i], -448.0f), 448.0f);
            int packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
            packed = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], packed, true);
            out[2 * a + d] = (uint32_t)packed;
        }
    return out;
}

// The same quantization of a half block through the gfx950 scaled convert:
// v_cvt_scalef32_pk_fp8_bf16 divides two bf16 values by the scale whose
// exponent field is the code and rounds to nearest even, which on gfx950
// gives the bytes of quant_half_block exactly (checked over every finite bf16
// value for codes 0 .. 247) except that a quotient that rounds above 448
// (possible under the OCP rule, whose block maximum scales into [256, 512))
// becomes the NaN code 0x7F / 0xFF instead of +-448; those bytes are moved to
// 0x7E / 0xFE.  The block maximum uses packed 16-bit integer maxima on the
// magnitudes (integer order of bf16 magnitudes is numeric order).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <int RULE>
__device__ inline v4u quant_half_block_cvt(v4u v0, v4u v1, uint32_t &code) {
    u16x2 m = __builtin_bit_cast(u16x2, v0[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (a == 0 && i == 0) continue;
            const uint32_t w = (a ? v1[i] : v0[i]) & 0x7FFF7FFFu;
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w));
        }
    uint32_t amax = (uint32_t)(m[0] > m[1] ? m[0] : m[1]) << 16;
    const uint32_t other = (uint32_t)__shfl_xor((int)amax, 16);
    amax = amax > other ? amax : other;
    code = act_code<RULE>(amax);
    const float scale = __uint_as_float(code << 23);
    v4u out;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo = d < 2 ? v0[2 * d] : v1[2 * d - 4];
        const uint32_t hi = d < 2 ? v0[2 * d + 1] : v1[2 * d - 3];
        v2s r = {0, 0};
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, lo), scale, false);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, hi), scale, true);
        uint32_t w = __builtin_bit_cast(uint32_t, r);
        if (RULE == 0) {
            // bytes whose low seven bits are all ones: 0x7F / 0xFF -> 0x7E / 0xFE
            const uint32_t nan = ((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
            w -= nan >> 7;
        }
        out[d] = w;
    }
    return out;
}

}  // namespace mx
