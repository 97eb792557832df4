// mx_gemv.hip -- decode-time GEMV and grouped MoE GEMV, M <= 16 per batch.
//
// y[m][n] = sum_k a[m][k] * dec(W[n][k]) * 2^(code(n,k) - 127)
// ([rocm_native] apply_weights: out = x W^T; [a16w4] step_mfma for the
// in-register decode feeding bf16 matrix cores).
//
// One workgroup owns one 16-row weight tile of one expert and one batch of up
// to 16 token "slots"; its NW wavefronts split the tile's 128-K steps into
// contiguous ranges and reduce their partial tiles in LDS in a fixed order,
// so results do not depend on timing.  Per step each lane loads its weight
// piece(s) of the W-T16 chunk (16-byte buffer loads, 1 KB contiguous per
// wavefront, marked non-temporal: weights are streamed once), its code(s),
// and the activation values of its slot; tokens are the 16-wide N side of
// the matrix-core tile, weight rows its M side, so a step is
//   W8A8  (e4m3 x MXFP8):  one v_mfma_scale_f32_16x16x128_f8f6f4 with the
//                          weight and activation E8M0 codes as lane scales;
//   A16W8 (e4m3 x bf16):   32 bytes decoded with their scale to bf16 by
//                          v_cvt_scalef32_pk_bf16_fp8, four bf16 16x16x32;
//   A16W4 (e2m1 x bf16):   16 bytes decoded by v_cvt_scalef32_pk_bf16_fp4,
//                          four bf16 16x16x32 ([a16w4] dequant / step_mfma).
// The MFMA accumulates in fp32; the single bf16 rounding happens at the store.
//
// Grouped MoE: a workgroup first collects the (token, slot) pairs routed to
// its expert with a wavefront ballot (in pair order) and exits before reading
// any weight byte if there are none.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

struct StepW8A8 {
    v4u a0, a1, b0, b1;
    uint32_t cw, cx;
};
struct StepA16 {
    v4u a0, a1;           // e4m3: two halves; e2m1: a0 only
    v4u x0, x1, x2, x3;   // bf16 activations of the four MFMAs
    uint32_t cw;
};

template <int ELEM, int LAYOUT, int ACT, bool MOE, int NW>
__global__ void __launch_bounds__(NW * 64) gemv_kernel(GemvArgs p) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const int r = lane % 16, j = lane / 16;
    const int64_t Kp = (p.K + 127) / 128 * 128, S = Kp / 128, T = p.N / 16, Q = (S + 3) / 4;
    const int64_t KB = p.K / 32;
    const int64_t unit = blockIdx.x;                 // e * T + t
    const int64_t e = MOE ? unit / T : 0, t = MOE ? unit % T : unit;
    constexpr int CHUNK = ELEM == E4M3 ? 2048 : 1024;

    __shared__ uint16_t slots[MOE ? kMoeMaxPairs : 1];
    __shared__ int nslots_sh;
    __shared__ v4f red[NW > 1 ? NW : 1][64];

    int64_t nslots;
    if (MOE) {
        const int64_t P = p.rows * p.topk;
        if (wave == 0) {
            int running = 0;
            for (int64_t base = 0; base < P; base += 64) {
                const int64_t i = base + lane;
                // unit e == E collects the pairs whose id is out of range
                const int32_t id = i < P ? p.ids[i] : 0;
                const bool hit = i < P && (e < p.E ? id == (int32_t)e : (id < 0 || id >= p.E));
                const uint64_t mask = __ballot(hit);
                const int rank = running + __popcll(mask & ((1ull << lane) - 1ull));
                if (hit) slots[rank] = (uint16_t)i;
                running += __popcll(mask);
            }
            if (lane == 0) nslots_sh = running;
        }
        __syncthreads();
        nslots = nslots_sh;
        if (nslots == 0) return;                     // no token: no weight bytes read
        if (e == p.E) {                              // out-of-range ids: zero rows
            for (int64_t idx = threadIdx.x; idx < nslots * 16; idx += NW * 64) {
                const int64_t pair = slots[idx / 16], n = 16 * t + idx % 16;
                if (p.ws)
                    p.ws[pair * p.N + n] = 0.f;
                else
                    p.y[pair * p.ldy + n] = 0;
            }
            return;
        }
    } else {
        nslots = p.rows;
    }

    // resources: the tile's weight chunks, its codes, the activations
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(p.w + unit * S * CHUNK, (uint32_t)(S * CHUNK));
    __amdgpu_buffer_rsrc_t cr;
    if (LAYOUT == ROW32)
        cr = make_rsrc(p.codes + unit * Q * 256, (uint32_t)(Q * 256));
    else
        cr = make_rsrc(p.codes + ((e * p.N + 16 * t) / 32) * (Kp / 32), (uint32_t)(Kp / 32));
    const int64_t xelt = ACT == ACT_MXFP8 ? 1 : 2;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, (uint32_t)(p.xrows * p.ldx * xelt));
    const __amdgpu_buffer_rsrc_t xcr =
        make_rsrc(p.xcodes, ACT == ACT_MXFP8 ? (uint32_t)(p.xrows * p.ldc) : 0u);

    const int64_t s0 = (wave * S) / NW, s1 = ((wave + 1) * S) / NW;
    const int64_t batches = (nslots + 15) / 16;
    const int64_t b_first = MOE ? 0 : blockIdx.y, b_last = MOE ? batches : blockIdx.y + 1;

    for (int64_t bi = b_first; bi < b_last; ++bi) {
        // this lane's slot: activation row and output row (or -1)
        const int64_t slot = 16 * bi + r;
        int64_t xrow = -1, yrow = -1;
        if (slot < nslots) {
            if (MOE) {
                const int64_t pair = slots[slot];
                xrow = pair / p.topk;
                yrow = pair;
            } else {
                xrow = slot;
                yrow = slot;
            }
        }
        const bool live = xrow >= 0;
        const uint32_t xbase = live ? (uint32_t)(xrow * p.ldx * xelt) : 0u;
        const uint32_t cxbase = live ? (uint32_t)(xrow * p.ldc) : 0u;

        v4f acc = {0.f, 0.f, 0.f, 0.f};

        if (ACT == ACT_MXFP8) {
            // ---- W8A8: e4m3 weights x MXFP8 activations, scaled MFMA ----
            auto load = [&](int64_t s) {
                StepW8A8 st;
                st.a0 = load16<kNT>(wr, (uint32_t)(s * 2048 + 16 * lane));
                st.a1 = load16<kNT>(wr, (uint32_t)(s * 2048 + 1024 + 16 * lane));
                const int64_t k0 = 128 * s + 16 * j, k1 = k0 + 64;   // K of each 16-byte half
                st.b0 = load16(xr, live && k0 < p.K ? xbase + (uint32_t)k0 : kOOB);
                st.b1 = load16(xr, live && k1 < p.K ? xbase + (uint32_t)k1 : kOOB);
                const int64_t blk = 4 * s + j;                       // scale block of lane group j
                st.cx = load1(xcr, live && blk < KB ? cxbase + (uint32_t)blk : kOOB);
                if (LAYOUT == ROW32)
                    st.cw = load4(cr, (uint32_t)((s / 4) * 256 + 4 * lane));
                else
                    st.cw = load4(cr, (uint32_t)(4 * s));
                return st;
            };
            auto compute = [&](const StepW8A8 &st, int64_t s, v4f c) {
                const uint32_t sw = LAYOUT == ROW32 ? byte_of(st.cw, (uint32_t)(s % 4))
                                                    : byte_of(st.cw, (uint32_t)j);
                return mfma_fp8_scaled(cat8(st.a0, st.a1), cat8(st.b0, st.b1), c, (int)sw,
                                       (int)st.cx);
            };
            int64_t s = s0;
            for (; s + 4 <= s1; s += 4) {
                StepW8A8 st[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) st[u] = load(s + u);
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = compute(st[u], s + u, acc);
            }
            for (; s < s1; ++s) acc = compute(load(s), s, acc);
        } else {
            // ---- A16: bf16 activations, weights decoded in registers ----
            auto load = [&](int64_t s) {
                StepA16 st;
                if (ELEM == E4M3) {
                    st.a0 = load16<kNT>(wr, (uint32_t)(s * 2048 + 16 * lane));
                    st.a1 = load16<kNT>(wr, (uint32_t)(s * 2048 + 1024 + 16 * lane));
                    // MFMA d covers K 16 j + 8 d (d < 2) and 64 + 16 j + 8 (d - 2)
                    const int64_t k0 = 128 * s + 16 * j, k1 = k0 + 64;
                    const bool v0 = live && k0 < p.K, v1 = live && k1 < p.K;
                    st.x0 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0) : kOOB);
                    st.x1 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0 + 16) : kOOB);
                    st.x2 = load16(xr, v1 ? xbase + (uint32_t)(2 * k1) : kOOB);
                    st.x3 = load16(xr, v1 ? xbase + (uint32_t)(2 * k1 + 16) : kOOB);
                } else {
                    st.a0 = load16<kNT>(wr, (uint32_t)(s * 1024 + 16 * lane));
                    const int64_t k0 = 128 * s + 32 * j;            // the lane's whole block
                    const bool v0 = live && k0 < p.K;
                    st.x0 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0) : kOOB);
                    st.x1 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0 + 16) : kOOB);
                    st.x2 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0 + 32) : kOOB);
                    st.x3 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0 + 48) : kOOB);
                }
                if (LAYOUT == ROW32)
                    st.cw = load4(cr, (uint32_t)((s / 4) * 256 + 4 * lane));
                else
                    st.cw = load4(cr, (uint32_t)(4 * s));
                return st;
            };
            auto compute = [&](const StepA16 &st, int64_t s, v4f c) {
                if (ELEM == E4M3) {
                    // codes of the blocks holding K 16 j.. (block j/2) and 64 + 16 j..
                    // (block 2 + j/2) of this lane's row
                    uint32_t c0, c1;
                    if (LAYOUT == ROW32) {
                        const uint32_t u = (uint32_t)(s % 4);
                        c0 = byte_of((uint32_t)__shfl((int)st.cw, 16 * (j / 2) + r), u);
                        c1 = byte_of((uint32_t)__shfl((int)st.cw, 16 * (2 + j / 2) + r), u);
                    } else {
                        c0 = byte_of(st.cw, (uint32_t)(j / 2));
                        c1 = byte_of(st.cw, (uint32_t)(2 + j / 2));
                    }
                    const float f0 = code_as_scale(c0), f1 = code_as_scale(c1);
                    c = mfma_bf16(dec8_e4m3(st.a0[0], st.a0[1], f0), as_bf16x8(st.x0), c);
                    c = mfma_bf16(dec8_e4m3(st.a0[2], st.a0[3], f0), as_bf16x8(st.x1), c);
                    c = mfma_bf16(dec8_e4m3(st.a1[0], st.a1[1], f1), as_bf16x8(st.x2), c);
                    c = mfma_bf16(dec8_e4m3(st.a1[2], st.a1[3], f1), as_bf16x8(st.x3), c);
                } else {
                    const uint32_t cc = LAYOUT == ROW32 ? byte_of(st.cw, (uint32_t)(s % 4))
                                                        : byte_of(st.cw, (uint32_t)j);
                    const float f = code_as_scale(cc);
                    c = mfma_bf16(dec8_e2m1(st.a0[0], f), as_bf16x8(st.x0), c);
                    c = mfma_bf16(dec8_e2m1(st.a0[1], f), as_bf16x8(st.x1), c);
                    c = mfma_bf16(dec8_e2m1(st.a0[2], f), as_bf16x8(st.x2), c);
                    c = mfma_bf16(dec8_e2m1(st.a0[3], f), as_bf16x8(st.x3), c);
                }
                return c;
            };
            int64_t s = s0;
            for (; s + 4 <= s1; s += 4) {
                StepA16 st[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) st[u] = load(s + u);
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = compute(st[u], s + u, acc);
            }
            for (; s < s1; ++s) acc = compute(load(s), s, acc);
        }

        // ---- reduce the NW partial tiles in wave order, then store ----
        if (NW > 1) {
            red[wave][lane] = acc;
            __syncthreads();
            if (wave == 0) {
#pragma unroll
                for (int w2 = 1; w2 < NW; ++w2) acc += red[w2][lane];
            }
        }
        if (wave == 0 && yrow >= 0) {
            // lane (r, j) holds rows 4 j .. 4 j + 3 of the tile for slot r
            const int64_t n0 = 16 * t + 4 * j;
            if (p.ws) {
                float *dst = p.ws + yrow * p.N + n0;
                *reinterpret_cast<v4f *>(dst) = acc;
            } else {
                float v[4] = {acc[0], acc[1], acc[2], acc[3]};
                if (p.bias) {
                    const uint16_t *bb = p.bias + n0;
                    for (int i = 0; i < 4; ++i) v[i] += bf16_to_f32(bb[i]);
                }
                v2u o = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                         bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
                *reinterpret_cast<v2u *>(p.y + yrow * p.ldy + n0) = o;
            }
        }
        if (NW > 1) __syncthreads();                 // red[] is reused by the next batch
    }
}

// Deterministic top-k combine: y[t][n] = sum_k w[t][k] * ys[t*topk + k][n],
// k ascending, fp32, one bf16 rounding.
__global__ void __launch_bounds__(256) moe_combine_kernel(int64_t T, int64_t topk, int64_t N,
                                                          const float *__restrict__ ys,
                                                          const float *__restrict__ wts,
                                                          uint16_t *__restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * N) return;
    const int64_t t = i / N, n = i % N;
    float s = 0.f;
    for (int64_t k = 0; k < topk; ++k) s += wts[t * topk + k] * ys[(t * topk + k) * N + n];
    y[i] = (uint16_t)bf16_bits(s);
}

template <int ELEM, int LAYOUT, int ACT, bool MOE>
static hipError_t launch_nw(const GemvArgs &a, int nw, dim3 grid, hipStream_t st) {
    switch (nw) {
    case 1: hipLaunchKernelGGL((gemv_kernel<ELEM, LAYOUT, ACT, MOE, 1>), grid, dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<ELEM, LAYOUT, ACT, MOE, 2>), grid, dim3(128), 0, st, a); break;
    case 8: hipLaunchKernelGGL((gemv_kernel<ELEM, LAYOUT, ACT, MOE, 8>), grid, dim3(512), 0, st, a); break;
    default: hipLaunchKernelGGL((gemv_kernel<ELEM, LAYOUT, ACT, MOE, 4>), grid, dim3(256), 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv(int elem, int layout, int act, bool moe, const GemvArgs &a, int nw,
                       hipStream_t st) {
    const int64_t T = a.N / 16;
    // MoE: one extra group of T workgroups (unit e == E) zero-fills the rows of
    // out-of-range ids; it exits at once when there are none
    const dim3 grid = moe ? dim3((unsigned)((a.E + 1) * T))
                          : dim3((unsigned)T, (unsigned)((a.rows + 15) / 16));
#define MX_GEMV_CASE(EL, LA, AC, MO)                                                     \
    if (elem == EL && layout == LA && act == AC && moe == MO)                              \
        return launch_nw<EL, LA, AC, MO>(a, nw, grid, st);
    MX_GEMV_CASE(E4M3, ROW32, ACT_MXFP8, false)
    MX_GEMV_CASE(E4M3, BLK32, ACT_MXFP8, false)
    MX_GEMV_CASE(E4M3, ROW32, ACT_BF16, false)
    MX_GEMV_CASE(E4M3, BLK32, ACT_BF16, false)
    MX_GEMV_CASE(E2M1, ROW32, ACT_BF16, false)
    MX_GEMV_CASE(E2M1, ROW32, ACT_BF16, true)
    MX_GEMV_CASE(E4M3, ROW32, ACT_BF16, true)
#undef MX_GEMV_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_moe_combine(int64_t T, int64_t topk, int64_t N, const float *ys,
                              const float *wts, void *y, hipStream_t st) {
    const int64_t n = T * N;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, T,
                       topk, N, ys, wts, (uint16_t *)y);
    return hipGetLastError();
}

}  // namespace mx
