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
// its expert with a wavefront ballot (in pair order) and exits if there are
// none (before reading any weight byte, except for the first chunk the
// two-wavefront A16W4 form requests ahead of the scan).  Two runtime modes serve the MoE block:
// `xslot` reads one activation row per slot (the down projection of the
// hidden rows), `epi` turns interleaved (gate, up) row pairs into
// silu(gate) * up, one output per pair ([weights942] moe_copies interleaves
// the two halves: even rows gate, odd rows up).
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

template <int G>
struct StepW8A8 {
    v4u a0[G], a1[G], b0, b1;
    uint32_t cw[G], cx;
};
template <int G>
struct StepA16 {
    v4u a0[G], a1[G];     // e4m3: two halves; e2m1: a0 only
    v4u x0, x1, x2, x3;   // bf16 activations of the four MFMAs
    uint32_t cw[G], cw2[G];
};

// One tile's step of the A16 product in exact form, for steps holding an E8M0
// code outside kLo .. kHi (the range where every scaled weight is a normal
// bf16 number): decode with the code clamped into that range, take each
// 32-K block's partial on its own (the operands of the lane groups that do
// not hold the block are zero), multiply the partial by the remaining power
// of two 2^(code - clamped) in fp32 and add it to acc.  Output row 4 j + i of
// a lane takes the factor of that row's block, read from the lanes whose
// weight row it is.  Lane (r, j) holds, for its row r: E4M3 a0 = K 16 j ..
// (block j / 2, code c0) and a1 = K 64 + 16 j .. (block 2 + j / 2, code c1);
// E2M1 a0 = block j (code c0).  All 64 lanes must be active.
template <int ELEM>
__device__ inline v4f a16_exact_tile(v4f acc, v4u a0, v4u a1, v4u x0, v4u x1,
                                                       v4u x2, v4u x3, uint32_t c0, uint32_t c1,
                                                       int j) {
    constexpr uint32_t kLo = ELEM == E4M3 ? 10u : 2u, kHi = ELEM == E4M3 ? 246u : 252u;
    const uint32_t k0 = c0 < kLo ? kLo : (c0 > kHi ? kHi : c0);
    const uint32_t k1 = c1 < kLo ? kLo : (c1 > kHi ? kHi : c1);
    const int d0 = (int)c0 - (int)k0, d1 = (int)c1 - (int)k1;
    const float f0 = code_as_scale(k0), f1 = code_as_scale(k1);
    const v4u xx[4] = {x0, x1, x2, x3};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        // E4M3: block b sits in operands 2 (b / 2), + 1 of lane groups
        // 2 (b % 2), + 1 (half b / 2: code c0 or c1); E2M1: in all four
        // operands of lane group b
        v4f t = {0.f, 0.f, 0.f, 0.f};
        int delta;
        if (ELEM == E4M3) {
            const bool mine = j / 2 == b % 2;
            const int h = b / 2;
            const v4u a = h ? a1 : a0;
            const float f = h ? f1 : f0;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const uint32_t lo = mine ? a[2 * q] : 0u, hi = mine ? a[2 * q + 1] : 0u;
                t = mfma_bf16(dec8_e4m3(lo, hi, f), as_bf16x8(xx[2 * h + q]), t);
            }
            delta = h ? d1 : d0;
        } else {
            const bool mine = j == b;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                t = mfma_bf16(dec8_e2m1(mine ? a0[d] : 0u, f0), as_bf16x8(xx[d]), t);
            delta = d0;
        }
        const int src0 = ELEM == E4M3 ? 32 * (b % 2) : 16 * b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int di = __shfl(delta, src0 + 4 * j + i);
            acc[i] += t[i] * __uint_as_float((uint32_t)(127 + di) << 23);
        }
        __builtin_amdgcn_sched_barrier(0);      // one block's temporaries at a time
    }
    return acc;
}

// G: weight tiles per workgroup.  A wavefront's activation fragment of a step
// is loaded once and feeds the G tiles' matrix-core operations.
// The A16W4 MoE launches hold about 1,500 workgroups of NW = 4 wavefronts:
// with chunks of two steps the kernel fits the register budget of four
// wavefronts per SIMD without spilling, which keeps them all resident at once
// (measured on MI355X: 29.8-30.3 against 32.1-33.3 us at E = 32, N = K = 3072).
// With NW = 2 (the K = 1536 down projection) three wavefronts per SIMD keep
// its ~1,500 workgroups resident too, and leave the registers that sharing
// the code dwords of a chunk needs (47.2 against 48.1 us for the MoE block).
template <int ELEM, int LAYOUT, int ACT, bool MOE, int NW, int P, int G>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(MOE && ELEM == E2M1 && P <= 2 ? (NW >= 4 ? 4 : 3) : 1)))
gemv_kernel(GemvArgs p) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const int r = lane % 16, j = lane / 16;
    const int64_t Kp = (p.K + 127) / 128 * 128, S = Kp / 128, T = p.N / 16, Q = (S + 3) / 4;
    const int64_t KB = p.K / 32;
    const int64_t TG = (T + G - 1) / G;              // tile groups per expert
    const int64_t unit = blockIdx.x;                 // e * TG + tg
    const int64_t e = MOE ? unit / TG : 0, tg = MOE ? unit % TG : unit;
    const int64_t t0 = tg * G;
    const int ntiles = (int)(T - t0 < G ? T - t0 : G);
    constexpr int CHUNK = ELEM == E4M3 ? 2048 : 1024;

    __shared__ uint16_t slots[MOE ? kMoeMaxPairs : 1];
    __shared__ int nslots_sh;
    __shared__ v4f red[NW > 1 ? NW : 1][G][64];

    // resources: the group's weight chunks, codes, the activations
    // a tile is 16 row lengths: S - 1 whole chunks, then the last step's
    // valid prefix of tailb bytes (no padding stored)
    const int64_t TILEB = 16 * (ELEM == E4M3 ? p.K : p.K / 2);
    const uint32_t tailb = (uint32_t)(TILEB - (S - 1) * CHUNK);
    // kPre (below): the MoE unit e == E reads no weights, an empty resource
    constexpr bool kPre = MOE && ELEM == E2M1 && ACT == ACT_BF16 && NW == 2 && P == 2;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(
        p.w + (e * T + t0) * TILEB, kPre && e >= p.E ? 0u : (uint32_t)(ntiles * TILEB));
    __amdgpu_buffer_rsrc_t cr;
    if (LAYOUT == ROW32)
        cr = make_rsrc(p.codes + (e * T + t0) * Q * 256, (uint32_t)(ntiles * Q * 256));
    else
        cr = make_rsrc(p.codes, (uint32_t)(p.E * (p.N / 32) * Q * 16));
    uint32_t crow[G];                                // BLK32: code offset of each tile's row group
#pragma unroll
    for (int g = 0; g < G; ++g) crow[g] = (uint32_t)(((e * p.N + 16 * (t0 + g)) / 32) * Q * 16);
    const int64_t xelt = ACT == ACT_MXFP8 ? 1 : 2;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, (uint32_t)(p.xrows * p.ldx * xelt));
    const __amdgpu_buffer_rsrc_t xcr =
        make_rsrc(p.xcodes, ACT == ACT_MXFP8 ? (uint32_t)(p.xrows * p.ldc) : 0u);

    // Grouped A16 with chunks of two steps: wavefront ranges start on even
    // steps, so both steps of a chunk lie in one quad and share its code
    // dwords (loaded once a chunk instead of once a step).
    constexpr bool kPairCodes = MOE && ACT == ACT_BF16 && P == 2 && NW >= 2;
    const int64_t b0 = (wave * S) / NW, b1 = ((wave + 1) * S) / NW;
    const int64_t s0 = kPairCodes ? (b0 & ~int64_t(1)) : b0;
    const int64_t s1 = kPairCodes && wave + 1 < NW ? (b1 & ~int64_t(1)) : b1;

    // A16: is any weight code outside kLo .. kHi?  The register-tight grouped
    // A16W4 GEMV reads the tensor's code range from the packed codes' trailer
    // (one scalar load; its wait lands ahead of the first loads, which that
    // kernel's routing scan pays anyway); the others note the codes of their
    // own steps as the loop meets them.
    constexpr uint32_t kLo = ELEM == E4M3 ? 10u : 2u, kHi = ELEM == E4M3 ? 246u : 252u;
    constexpr bool kRangeTrailer = MOE && ELEM == E2M1;
    uint32_t crange = 0;
    if (ACT == ACT_BF16 && kRangeTrailer)
        crange = *reinterpret_cast<const uint32_t *>(
            p.codes + packed_code_body_bytes(LAYOUT, p.E, p.N, p.K));

    // weight and code offsets of tile g at step s (out of range beyond s1,
    // and past the last step's valid prefix); half 1 is an E4M3 chunk's
    // second 1 KB
    auto woff = [&](int g, int64_t s, bool in, int half) -> uint32_t {
        const uint32_t o = (uint32_t)(1024 * half + 16 * lane);
        if (!in || (s == S - 1 && o >= tailb)) return kOOB;
        return (uint32_t)(g * TILEB + s * CHUNK) + o;
    };
    // the dword holding this step's code of the lane's row r for the block
    // of lane group jj (byte s % 4 of it): ROW32 the C-T16 dword of lane
    // 16 jj + r (only the A16 e4m3 form asks for jj != j; the others read the
    // lane's own), BLK32 dword jj of the row group's 16-byte quad
    auto coff = [&](int g, int64_t s, bool in, int jj) -> uint32_t {
        if (!in) return kOOB;
        if (LAYOUT == ROW32)
            return (uint32_t)((g * Q + s / 4) * 256 +
                              (ELEM == E4M3 && ACT == ACT_BF16 ? 4 * (16 * jj + r) : 4 * lane));
        return crow[g] + (uint32_t)((s / 4) * 16 + 4 * jj);
    };

    // A16 weights and codes of step s (out of range beyond s1), requested
    // before the step's activations
    auto loadw = [&](int64_t s, bool codes = true) {
        StepA16<G> st;
        const bool in = s < s1;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            st.a0[g] = load16<kNT>(wr, woff(g, s, in, 0));
            if (ELEM == E4M3) st.a1[g] = load16<kNT>(wr, woff(g, s, in, 1));
        }
        if (!codes) return st;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (ELEM == E4M3) {
                // codes of the blocks holding K 16 j.. (block j / 2) and
                // 64 + 16 j.. (block 2 + j / 2) of this lane's row, loaded
                // directly (no lane exchange in the loop)
                st.cw[g] = load4(cr, coff(g, s, in, j / 2));
                st.cw2[g] = load4(cr, coff(g, s, in, 2 + j / 2));
            } else {
                st.cw[g] = load4(cr, coff(g, s, in, j));
            }
        }
        return st;
    };
    // the E2M1 codes of step s alone (the prefetched chunk's, after the scan)
    auto loadc_e2m1 = [&](StepA16<G> &st, int64_t s) {
        const bool in = s < s1;
#pragma unroll
        for (int g = 0; g < G; ++g) st.cw[g] = load4(cr, coff(g, s, in, j));
    };

    // Two-wavefront grouped A16W4 (the short-K down projection): the first
    // chunk's weight bytes are requested before the routing scan is known
    // (its codes after it), so the weight stream starts at once.  Every
    // wavefront requests them right behind the first 128 pairs' ids loads
    // (loads complete in issue order: wavefront 0's scan waits for the ids
    // only, not for the weight bytes).
    static_assert(!kPre || kPairCodes, "the prefetch takes a chunk of two steps");
    StepA16<G> pre[kPre ? P : 1];
    auto prefetch = [&]() {
        pre[0] = loadw(s0, false);
        pre[1] = loadw(s0 + 1, false);
    };

    int64_t nslots;
    if (MOE) {
        const int64_t npairs = p.rows * p.topk;
        // the first 128 pairs' ids, then the prefetch: every wavefront issues
        // both, unconditionally (ids past the pairs read 0 through the
        // resource bounds), so nothing waits on them before the scan
        int32_t id0[2] = {0, 0};
        if constexpr (kPre) {
            const __amdgpu_buffer_rsrc_t ir = make_rsrc(p.ids, (uint32_t)(npairs * 4));
#pragma unroll
            for (int h = 0; h < 2; ++h) id0[h] = (int32_t)load4(ir, (uint32_t)(4 * (64 * h + lane)));
            prefetch();
        }
        if (wave == 0) {
            int running = 0;
            // 128 pairs an iteration: both ids loads go out before the first
            // ballot, so the scan waits for one load round trip, not two
            for (int64_t base = 0; base < npairs; base += 128) {
                int32_t id[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t i = base + 64 * h + lane;
                    id[h] = kPre && base == 0 ? id0[h] : (i < npairs ? p.ids[i] : 0);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t i = base + 64 * h + lane;
                    // unit e == E collects the pairs whose id is out of range
                    const bool hit = i < npairs && (e < p.E ? id[h] == (int32_t)e
                                                            : (id[h] < 0 || id[h] >= p.E));
                    const uint64_t mask = __ballot(hit);
                    const int rank = running + __popcll(mask & ((1ull << lane) - 1ull));
                    if (hit) slots[rank] = (uint16_t)i;
                    running += __popcll(mask);
                }
            }
            if (lane == 0) nslots_sh = running;
        }
        __syncthreads();
        nslots = nslots_sh;
        // no token: no further weight bytes read (the two-wavefront form
        // has requested its first chunk already)
        if (nslots == 0) return;
        if (e == p.E) {                              // out-of-range ids: zero rows
            // (with the SiLU epilogue a 16-row tile gives 8 outputs)
            const int64_t per = p.epi ? 8 : 16;
            for (int64_t idx = threadIdx.x; idx < nslots * per * ntiles; idx += NW * 64) {
                const int64_t pair = slots[idx / (per * ntiles)];
                const int64_t n = per * t0 + idx % (per * ntiles);
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

    const int64_t batches = (nslots + 15) / 16;
    const int64_t b_first = MOE ? 0 : blockIdx.y, b_last = MOE ? batches : blockIdx.y + 1;

    for (int64_t bi = b_first; bi < b_last; ++bi) {
        // this lane's slot: activation row and output row (or -1)
        const int64_t slot = 16 * bi + r;
        int64_t xrow = -1, yrow = -1;
        if (slot < nslots) {
            if (MOE) {
                const int64_t pair = slots[slot];
                // one activation row per slot, or per token (kPre: 32-bit
                // division, pair < kMoeMaxPairs, to stay within its registers)
                xrow = p.xslot ? pair
                               : (kPre ? (uint32_t)pair / (uint32_t)p.topk : pair / p.topk);
                yrow = pair;
            } else {
                xrow = slot;
                yrow = slot;
            }
        }
        const bool live = xrow >= 0;
        const uint32_t xbase = live ? (uint32_t)(xrow * p.ldx * xelt) : 0u;
        const uint32_t cxbase = live ? (uint32_t)(xrow * p.ldc) : 0u;

        v4f acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};

        if (ACT == ACT_MXFP8) {
            // ---- W8A8: e4m3 weights x MXFP8 activations, scaled MFMA ----
            // a step outside [s0, s1) reads only zeros (out-of-range offsets)
            auto load = [&](int64_t s) {
                StepW8A8<G> st;
                const bool in = s < s1;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    st.a0[g] = load16<kNT>(wr, woff(g, s, in, 0));
                    st.a1[g] = load16<kNT>(wr, woff(g, s, in, 1));
                }
                const int64_t k0 = 128 * s + 16 * j, k1 = k0 + 64;   // K of each 16-byte half
                st.b0 = load16(xr, in && live && k0 < p.K ? xbase + (uint32_t)k0 : kOOB);
                st.b1 = load16(xr, in && live && k1 < p.K ? xbase + (uint32_t)k1 : kOOB);
                const int64_t blk = 4 * s + j;                       // scale block of lane group j
                st.cx = load1(xcr, in && live && blk < KB ? cxbase + (uint32_t)blk : kOOB);
#pragma unroll
                for (int g = 0; g < G; ++g) st.cw[g] = load4(cr, coff(g, s, in, j));
                return st;
            };
            auto compute = [&](const StepW8A8<G> &st, int64_t s) {
                const v8i b = cat8(st.b0, st.b1);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const uint32_t sw = byte_of(st.cw[g], (uint32_t)(s % 4));
                    acc[g] = mfma_fp8_scaled(cat8(st.a0[g], st.a1[g]), b, acc[g], (int)sw,
                                             (int)st.cx);
                }
            };
            // all loads of a chunk of P steps are issued before its first MFMA
            for (int64_t c = s0; c < s1; c += P) {
                StepW8A8<G> st[P];
#pragma unroll
                for (int u = 0; u < P; ++u) st[u] = load(c + u);
                // keep the scheduler from pulling MFMAs (and their waits) up
                // between the loads: all P steps stay in flight together
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < P; ++u) compute(st[u], c + u);
            }
        } else {
            // ---- A16: bf16 activations, weights decoded in registers ----
            auto loadx = [&](auto &st, int64_t s) {
                const bool in = s < s1;
                if (ELEM == E4M3) {
                    // MFMA d covers K 16 j + 8 d (d < 2) and 64 + 16 j + 8 (d - 2)
                    const int64_t k0 = 128 * s + 16 * j, k1 = k0 + 64;
                    const bool v0 = in && live && k0 < p.K, v1 = in && live && k1 < p.K;
                    st.x0 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0) : kOOB);
                    st.x1 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0 + 16) : kOOB);
                    st.x2 = load16(xr, v1 ? xbase + (uint32_t)(2 * k1) : kOOB);
                    st.x3 = load16(xr, v1 ? xbase + (uint32_t)(2 * k1 + 16) : kOOB);
                } else {
                    const int64_t k0 = 128 * s + 32 * j;            // the lane's whole block
                    const bool v0 = in && live && k0 < p.K;
                    st.x0 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0) : kOOB);
                    st.x1 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0 + 16) : kOOB);
                    st.x2 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0 + 32) : kOOB);
                    st.x3 = load16(xr, v0 ? xbase + (uint32_t)(2 * k0 + 48) : kOOB);
                }
            };
            auto load = [&](int64_t s, bool codes = true) {
                StepA16<G> st = loadw(s, codes);
                loadx(st, s);
                return st;
            };
            // Each lane's weight bytes belong to one 32-K block per 16-byte
            // half (E4M3: K 16 j .. is block j / 2, K 64 + 16 j .. block
            // 2 + j / 2; E2M1: the lane's 16 bytes are block j), so one code
            // per half scales them.  Decoded with that code the bf16 operand
            // is exact while every e4m3 / e2m1 value times 2^(code - 127)
            // stays in bf16's normal range (codes kLo .. kHi).  The loop
            // assumes so; when a code leaves kLo .. kHi (see kRangeTrailer)
            // the wavefront's range is done again in the exact form
            // (a16_exact_tile) after the loop.
            auto codes_of = [&](uint32_t cw, uint32_t cw2, int64_t s, uint32_t &c0,
                                uint32_t &c1) {
                const uint32_t u = (uint32_t)(s % 4);
                c0 = byte_of(cw, u);
                c1 = ELEM == E4M3 ? byte_of(cw2, u) : c0;
            };
            bool outside = false;             // a code of this lane's steps outside kLo .. kHi
            auto compute = [&](const StepA16<G> &st, int64_t s) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    uint32_t c0, c1;
                    codes_of(st.cw[g], st.cw2[g], s, c0, c1);
                    // (steps past s1 read code 0 and zero bytes: not counted)
                    if (!kRangeTrailer)
                        outside = outside ||
                                  (s < s1 && (c0 - kLo > kHi - kLo || c1 - kLo > kHi - kLo));
                    const float f0 = code_as_scale(c0), f1 = code_as_scale(c1);
                    v4f c = acc[g];
                    if (ELEM == E4M3) {
                        c = mfma_bf16(dec8_e4m3(st.a0[g][0], st.a0[g][1], f0), as_bf16x8(st.x0), c);
                        c = mfma_bf16(dec8_e4m3(st.a0[g][2], st.a0[g][3], f0), as_bf16x8(st.x1), c);
                        c = mfma_bf16(dec8_e4m3(st.a1[g][0], st.a1[g][1], f1), as_bf16x8(st.x2), c);
                        c = mfma_bf16(dec8_e4m3(st.a1[g][2], st.a1[g][3], f1), as_bf16x8(st.x3), c);
                    } else {
                        c = mfma_bf16(dec8_e2m1(st.a0[g][0], f0), as_bf16x8(st.x0), c);
                        c = mfma_bf16(dec8_e2m1(st.a0[g][1], f0), as_bf16x8(st.x1), c);
                        c = mfma_bf16(dec8_e2m1(st.a0[g][2], f0), as_bf16x8(st.x2), c);
                        c = mfma_bf16(dec8_e2m1(st.a0[g][3], f0), as_bf16x8(st.x3), c);
                    }
                    acc[g] = c;
                }
            };
            int64_t c0 = s0;
            if constexpr (kPre) {
                // the first batch's first chunk: weights and codes prefetched
                if (bi == b_first && c0 < s1) {
                    StepA16<G> st[P];
                    // the codes of the chunk's quad, then the activations
                    st[0] = pre[0];
                    loadc_e2m1(st[0], c0);
                    loadx(st[0], c0);
                    st[1] = pre[1];
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        st[1].cw[g] = st[0].cw[g];
                        st[1].cw2[g] = st[0].cw2[g];
                    }
                    loadx(st[1], c0 + 1);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int u = 0; u < P; ++u) compute(st[u], c0 + u);
                    c0 += P;
                }
            }
            for (int64_t c = c0; c < s1; c += P) {
                StepA16<G> st[P];
#pragma unroll
                for (int u = 0; u < P; ++u) {
                    if (kPairCodes && u == 1) {
                        // c is even: step c + 1 is in step c's quad
                        st[1] = load(c + 1, false);
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            st[1].cw[g] = st[0].cw[g];
                            st[1].cw2[g] = st[0].cw2[g];
                        }
                    } else {
                        st[u] = load(c + u);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < P; ++u) compute(st[u], c + u);
            }
            const bool exact = kRangeTrailer
                                   ? (crange & 0xFFu) < kLo || ((crange >> 8) & 0xFFu) > kHi
                                   : __any(outside);
            if (exact) {
                // exact form, one tile and step at a time on reloaded
                // operands; the partial tiles live in this wavefront's slot
                // of the reduction buffer meanwhile (fewer registers)
                v4f *part = red[NW > 1 ? wave : 0][0] + lane;      // tile g at part[64 g]
#pragma unroll
                for (int g = 0; g < G; ++g) part[64 * g] = v4f{0.f, 0.f, 0.f, 0.f};
                for (int64_t s = s0; s < s1; ++s) {
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        StepA16<1> one;
                        one.a0[0] = load16<kNT>(wr, woff(g, s, true, 0));
                        one.a1[0] = ELEM == E4M3 ? load16<kNT>(wr, woff(g, s, true, 1)) : v4u{};
                        if (ELEM == E4M3) {
                            one.cw[0] = load4(cr, coff(g, s, true, j / 2));
                            one.cw2[0] = load4(cr, coff(g, s, true, 2 + j / 2));
                        } else {
                            one.cw[0] = load4(cr, coff(g, s, true, j));
                            one.cw2[0] = 0;
                        }
                        loadx(one, s);
                        uint32_t c0, c1;
                        codes_of(one.cw[0], one.cw2[0], s, c0, c1);
                        part[64 * g] = a16_exact_tile<ELEM>(part[64 * g], one.a0[0],
                                                            ELEM == E4M3 ? one.a1[0] : one.a0[0],
                                                            one.x0, one.x1, one.x2, one.x3, c0, c1, j);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g] = part[64 * g];
            }
        }

        // ---- the NW partial tiles, summed over the wavefronts in order
        // 0 .. NW - 1 (the result does not depend on timing), then stored.
        // Wavefront w finishes tiles w, w + NW, ...  The two-wavefront
        // grouped launch (the down projection) keeps wavefront 0 finishing
        // every tile, with its epilogue written out in place: measured on
        // MI355X, both forms of it that went through store_tile ran 0.2-0.5 us
        // slower. ----
        auto store_tile = [&](int g, const v4f a) {
            // lane (r, j) holds rows 4 j .. 4 j + 3 of tile t0 + g for slot r
            const int64_t n0 = 16 * (t0 + g) + 4 * j;
            if (MOE && p.epi) {
                // rows 4 j .. 4 j + 3 are (gate, up) of outputs n0 / 2 and
                // n0 / 2 + 1 (interleaved copies): silu(gate) * up
                const float h0 = a[0] / (1.f + __expf(-a[0])) * a[1];
                const float h1 = a[2] / (1.f + __expf(-a[2])) * a[3];
                *reinterpret_cast<uint32_t *>(p.y + yrow * p.ldy + n0 / 2) =
                    bf16_bits(h0) | (bf16_bits(h1) << 16);
            } else if (p.ws) {
                *reinterpret_cast<v4f *>(p.ws + yrow * p.N + n0) = a;
            } else {
                float v[4] = {a[0], a[1], a[2], a[3]};
                if (!MOE && p.bias) {                // (the MoE entry points take no bias)
                    const uint16_t *bb = p.bias + n0;
                    for (int i = 0; i < 4; ++i) v[i] += bf16_to_f32(bb[i]);
                }
                v2u o = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                         bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
                *reinterpret_cast<v2u *>(p.y + yrow * p.ldy + n0) = o;
            }
        };
        constexpr bool kSpread = NW > 1 && (NW >= 4 || !MOE);
        if (NW > 1) {
#pragma unroll
            for (int g = 0; g < G; ++g) red[wave][g][lane] = acc[g];
            __syncthreads();
        }
        if (kSpread) {
#pragma unroll
            for (int g0 = 0; g0 < G; g0 += NW) {
                const int g = g0 + wave;
                if (g >= ntiles) break;
                v4f a = red[0][g][lane];
#pragma unroll
                for (int w2 = 1; w2 < NW; ++w2) a += red[w2][g][lane];
                if (yrow >= 0) store_tile(g, a);
            }
        } else {
            if (NW > 1 && wave == 0) {
#pragma unroll
                for (int w2 = 1; w2 < NW; ++w2)
#pragma unroll
                    for (int g = 0; g < G; ++g) acc[g] += red[w2][g][lane];
            }
            if (wave == 0 && yrow >= 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    if (g >= ntiles) break;
                    // lane (r, j) holds rows 4 j .. 4 j + 3 of tile t0 + g for slot r
                    const int64_t n0 = 16 * (t0 + g) + 4 * j;
                    const v4f a = acc[g];
                    if (MOE && p.epi) {
                        const float h0 = a[0] / (1.f + __expf(-a[0])) * a[1];
                        const float h1 = a[2] / (1.f + __expf(-a[2])) * a[3];
                        *reinterpret_cast<uint32_t *>(p.y + yrow * p.ldy + n0 / 2) =
                            bf16_bits(h0) | (bf16_bits(h1) << 16);
                    } else if (p.ws) {
                        *reinterpret_cast<v4f *>(p.ws + yrow * p.N + n0) = a;
                    } else {
                        float v[4] = {a[0], a[1], a[2], a[3]};
                        if (p.bias) {
                            const uint16_t *bb = p.bias + n0;
                            for (int i = 0; i < 4; ++i) v[i] += bf16_to_f32(bb[i]);
                        }
                        v2u o = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                                 bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
                        *reinterpret_cast<v2u *>(p.y + yrow * p.ldy + n0) = o;
                    }
                }
            }
        }
        if (NW > 1) __syncthreads();                 // red[] is reused by the next batch
    }
}

// Deterministic top-k combine: y[t][n] = sum_k w[t][k] * ys[t*topk + k][n],
// k ascending, fp32, one bf16 rounding.  A thread owns 4 consecutive outputs
// (N % 16 == 0) and issues the loads of 8 slots before summing them in order.
// One-wavefront workgroups spread the launch over as many CUs as it has
// wavefronts (192 at T = 16, N = 3072; measured on MI355X: MoE block step
// 46.77 against 46.92 us with 256-thread workgroups).
__global__ void __launch_bounds__(256) moe_combine_kernel(int64_t T, int64_t topk, int64_t N,
                                                          const float *__restrict__ ys,
                                                          const float *__restrict__ wts,
                                                          uint16_t *__restrict__ y) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= T * N) return;
    const int64_t t = i / N, n = i % N;
    v4f s = {0.f, 0.f, 0.f, 0.f};
    for (int64_t k0 = 0; k0 < topk; k0 += 8) {
        v4f v[8];
        float w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t k = k0 + u < topk ? k0 + u : topk - 1;   // in bounds; unused
            v[u] = *reinterpret_cast<const v4f *>(ys + (t * topk + k) * N + n);
            w[u] = wts[t * topk + k];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (k0 + u < topk) s += w[u] * v[u];
    }
    const v2u o = {bf16_bits(s[0]) | (bf16_bits(s[1]) << 16),
                   bf16_bits(s[2]) | (bf16_bits(s[3]) << 16)};
    *reinterpret_cast<v2u *>(y + i) = o;
}

template <int ELEM, int LAYOUT, int ACT, bool MOE, int NW, int G>
static hipError_t launch_p(const GemvArgs &a, int chunk, dim3 grid, hipStream_t st) {
    switch (chunk) {
    case 2: hipLaunchKernelGGL((gemv_kernel<ELEM, LAYOUT, ACT, MOE, NW, 2, G>), grid, dim3(NW * 64), 0, st, a); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<ELEM, LAYOUT, ACT, MOE, NW, 4, G>), grid, dim3(NW * 64), 0, st, a); break;
    default: hipLaunchKernelGGL((gemv_kernel<ELEM, LAYOUT, ACT, MOE, NW, 8, G>), grid, dim3(NW * 64), 0, st, a); break;
    }
    return hipGetLastError();
}

template <int ELEM, int LAYOUT, int ACT, bool MOE, int G>
static hipError_t launch_nw(const GemvArgs &a, int nw, int chunk, dim3 grid, hipStream_t st) {
    switch (nw) {
    case 1: return launch_p<ELEM, LAYOUT, ACT, MOE, 1, G>(a, chunk, grid, st);
    case 2: return launch_p<ELEM, LAYOUT, ACT, MOE, 2, G>(a, chunk, grid, st);
    case 8: return launch_p<ELEM, LAYOUT, ACT, MOE, 8, G>(a, chunk, grid, st);
    default: return launch_p<ELEM, LAYOUT, ACT, MOE, 4, G>(a, chunk, grid, st);
    }
}

template <int ELEM, int LAYOUT, int ACT, bool MOE>
static hipError_t launch_g(const GemvArgs &a, const GemvShape &sh, hipStream_t st) {
    const int64_t T = a.N / 16;
    const int64_t TG = (T + sh.tiles - 1) / sh.tiles;
    // MoE: one extra group of TG workgroups (unit e == E) zero-fills the rows of
    // out-of-range ids; it exits at once when there are none
    const dim3 grid = MOE ? dim3((unsigned)((a.E + 1) * TG))
                          : dim3((unsigned)TG, (unsigned)((a.rows + 15) / 16));
    switch (sh.tiles) {
    case 2: return launch_nw<ELEM, LAYOUT, ACT, MOE, 2>(a, sh.nw, sh.chunk, grid, st);
    case 4: return launch_nw<ELEM, LAYOUT, ACT, MOE, 4>(a, sh.nw, sh.chunk, grid, st);
    default: return launch_nw<ELEM, LAYOUT, ACT, MOE, 1>(a, sh.nw, sh.chunk, grid, st);
    }
}

hipError_t launch_gemv(int elem, int layout, int act, bool moe, const GemvArgs &a,
                       const GemvShape &sh, hipStream_t st) {
#define MX_GEMV_CASE(EL, LA, AC, MO)                                                     \
    if (elem == EL && layout == LA && act == AC && moe == MO)                              \
        return launch_g<EL, LA, AC, MO>(a, sh, st);
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
    const int64_t n = T * N / 4;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((n + 63) / 64)), dim3(64), 0, st, T,
                       topk, N, ys, wts, (uint16_t *)y);
    return hipGetLastError();
}

}  // namespace mx
