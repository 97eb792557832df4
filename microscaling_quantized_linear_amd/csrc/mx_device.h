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

// 8 e4m3 bytes (two dwords) x 2^(code-127) -> 8 bf16 (exact for codes whose
// products stay inside bf16's normal range; rounded to nearest otherwise).
__device__ inline v8bf dec8_e4m3(uint32_t w0, uint32_t w1, float scale) {
    v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
    v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
    v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
    v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
    v8bf r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

// 8 e2m1 nibbles (one dword, low nibble first) x 2^(code-127) -> 8 bf16
// ([a16w4] dequant: four scaled pair conversions).
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

}  // namespace mx
