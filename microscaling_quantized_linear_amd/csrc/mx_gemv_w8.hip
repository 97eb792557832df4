// mx_gemv_w8.hip -- W8A8 decode GEMV: e4m3 weights x MXFP8 activations,
// 16 tokens per grid row.
//
// y[m][n] = sum_k dec(xq[m][k]) 2^(xc(m,k)-127) dec(W[n][k]) 2^(c(n,k)-127)
// ([rocm_native] apply_weights: fp8 operands and E8M0 block scales go to
// the microscaling matrix cores directly; the pages quantize the activation
// per token ahead of the small-M product).
//
// A workgroup owns G weight tiles of 16 rows; its NW wavefronts split the
// 128-K steps into contiguous ranges.  Per step a wavefront does one
// v_mfma_scale_f32_16x16x128_f8f6f4 per tile: weights as the A operand (a
// W-T16 chunk is one operand in lane order), the 16 tokens as B, both E8M0
// codes as lane scales.
//
// Load order, per wavefront, everything issued before the first wait:
//  1. the activation fragments of its own steps, copied straight into its
//     private LDS region by buffer loads with an LDS destination;
//  2. the activation and weight scale dwords (one per four steps, byte u =
//     step 4 q + u);
//  3. every weight chunk of its steps (16-byte non-temporal loads, 1 KB
//     contiguous per wavefront).
// The activations arrive either in fragment order (written by the in-call
// quantization: every copy is 1 KB contiguous) or row-major as the caller
// gave them.  Measured on MI355X, reading the activations per wavefront into
// registers interleaved with the weights cost several microseconds per
// launch; issued first, into LDS, they cost a fraction of one.
//
// The NW partial tiles are summed in LDS in wavefront order (the result
// does not depend on timing), then the bias is added and y rounded to bf16
// once.
#include "mx_device.h"
#include "mx_kernels.h"

#include <type_traits>

namespace mx {

typedef __attribute__((address_space(3))) void lds_void_w8;

// f(integral_constant<I>) for I = B .. E - 1, each a compile-time constant
template <int B, int E, class F>
__device__ inline void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// XFRAG: activations in fragment order (xf, xct); else row-major (xq, xc).
// G tiles per workgroup, SPW = the most steps one wavefront owns.
template <int LAYOUT, bool XFRAG, int G, int SPW>
__global__ void __launch_bounds__(512) gemv_w8_kernel(GemvW8Args p) {
    constexpr int NQ = (SPW + 6) / 4;                   // quads SPW steps can span
    __shared__ __attribute__((aligned(1024))) uint8_t xs[8][SPW * 2048];
    __shared__ v4f red[8][G][64];

    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int nw = blockDim.x / 64;
    const int r = lane % 16, j = lane / 16;
    const int64_t S = (p.K + 127) / 128, T = p.N / 16, Q = (S + 3) / 4, KB = p.K / 32;
    const int64_t t0 = (int64_t)blockIdx.x * G;
    const int ntiles = (int)(T - t0 < G ? T - t0 : G);
    const int64_t mb = blockIdx.y, row = 16 * mb + r;
    const bool live = row < p.M;
    const int64_t s0 = (wave * S) / nw, s1 = ((wave + 1) * S) / nw;
    const int n = (int)(s1 - s0);                       // <= SPW (host plan)
    const int64_t qa = s0 / 4;                          // first quad of the range

    // ---- 1. activation fragments of steps s0 .. s1 - 1 -> LDS ----
    uint8_t *myx = xs[wave];
    const __amdgpu_buffer_rsrc_t xr =
        XFRAG ? make_rsrc(p.xf, (uint32_t)(((p.M + 15) / 16) * S * 2048))
              : make_rsrc(p.xq, (uint32_t)(p.M * p.ldq));
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t s = s0 + i, k = 128 * s + 64 * h + 16 * j;
            uint32_t off = kOOB;
            if (i < n && live && k < p.K)
                off = XFRAG ? (uint32_t)(((mb * S + s) * 2 + h) * 1024 + 16 * lane)
                            : (uint32_t)(row * p.ldq + k);
            if (i < n)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (lds_void_w8 *)(myx + (2 * i + h) * 1024), 16, (int)off, 0, 0, 0);
        }

    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. scale codes ----
    // activation: fragment order gives one dword per quad (byte u = step
    // 4 q + u); row-major gives one byte per step.  Tokens past M and blocks
    // past K/32 get code 127 (their bytes are zero).
    uint32_t cxq[XFRAG ? NQ : 1];
    uint32_t cxs[XFRAG ? 1 : SPW];
    if constexpr (XFRAG) {
        const __amdgpu_buffer_rsrc_t xcr =
            make_rsrc(p.xct, (uint32_t)(((p.M + 15) / 16) * Q * 256));
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const int64_t q = qa + c;
            cxq[c] = load4(xcr, q < Q && live ? (uint32_t)((mb * Q + q) * 256 + 4 * lane) : kOOB);
        }
    } else {
        const __amdgpu_buffer_rsrc_t xcr = make_rsrc(p.xc, (uint32_t)(p.M * p.ldc));
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int64_t blk = 4 * (s0 + i) + j;
            cxs[i] = load1(xcr, i < n && live && blk < KB ? (uint32_t)(row * p.ldc + blk) : kOOB);
        }
    }
    // weights: one dword per tile and quad (packed codes are padded with 128)
    const __amdgpu_buffer_rsrc_t cr =
        make_rsrc(p.codes, LAYOUT == ROW32 ? (uint32_t)(T * Q * 256)
                                           : (uint32_t)((p.N / 32) * Q * 16));
    uint32_t cwq[G][NQ];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const int64_t t = t0 + g, q = qa + c;
            uint32_t off = kOOB;
            if (g < ntiles && q < Q)
                off = LAYOUT == ROW32 ? (uint32_t)((t * Q + q) * 256 + 4 * lane)
                                      : (uint32_t)(((16 * t) / 32 * Q + q) * 16 + 4 * j);
            cwq[g][c] = load4(cr, off);
        }
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. every weight chunk of the range ----
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w + t0 * S * 2048, (uint32_t)(ntiles * S * 2048));
    v4u wv[SPW][G][2];
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t base = i < n && g < ntiles
                                      ? (uint32_t)((g * S + s0 + i) * 2048 + 16 * lane)
                                      : kOOB;
            wv[i][g][0] = load16<kNT>(wr, base);
            wv[i][g][1] = load16<kNT>(wr, base == kOOB ? kOOB : base + 1024u);
        }
    __builtin_amdgcn_sched_barrier(0);

    // The copies into LDS were issued before every other load of this
    // wavefront, and every later load is issued unconditionally, so waiting
    // until at most that many loads are outstanding means the copies have
    // landed (memory loads complete in issue order).  The compiler does not
    // track copies issued under a condition, hence the explicit wait.
    constexpr int kLater = (XFRAG ? NQ : SPW) + G * NQ + 2 * SPW * G;
    static_assert(kLater < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt(vmcnt_only(kLater));
    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. one scaled MFMA per tile and step ----
    // The range starts at quad offset A = s0 % 4: step i is byte (A + i) % 4 of
    // quad slot (A + i) / 4.  One code path per A keeps every slot and byte
    // select a compile-time constant (a runtime index would put the small
    // arrays in scratch memory).
    v4f acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};
    auto run = [&](auto aconst) {
        constexpr int A = decltype(aconst)::value;
        static_for<0, SPW>([&](auto iconst) {
            constexpr int i = decltype(iconst)::value;
            constexpr int c = (A + i) / 4, u = (A + i) % 4;
            if (i >= n) return;                         // uniform
            const v4u b0 = *reinterpret_cast<const v4u *>(myx + (2 * i) * 1024 + 16 * lane);
            const v4u b1 = *reinterpret_cast<const v4u *>(myx + (2 * i + 1) * 1024 + 16 * lane);
            const v8i bf = cat8(b0, b1);
            uint32_t cx;
            if constexpr (XFRAG) {
                cx = cxq[c];
                // tokens past M and blocks past K/32: code 127 (zero bytes)
                if (!live || 4 * (s0 + i) + j >= KB) cx = 0x7F7F7F7Fu;
            } else {
                cx = cxs[i] << (8 * u);
            }
#pragma unroll
            for (int g = 0; g < G; ++g)
                acc[g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    cat8(wv[i][g][0], wv[i][g][1]), bf, acc[g], 0, 0, u, (int)cwq[g][c], u,
                    (int)cx);
        });
    };
    switch ((int)(s0 % 4)) {
    case 0: run(std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    default: run(std::integral_constant<int, 3>{}); break;
    }

    // ---- 5. wavefront-order reduction; wavefront g finishes tile g ----
#pragma unroll
    for (int g = 0; g < G; ++g) red[wave][g][lane] = acc[g];
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (wave != g % nw || g >= ntiles) continue;
        v4f a = red[0][g][lane];
        for (int w2 = 1; w2 < nw; ++w2) a += red[w2][g][lane];
        if (!live) continue;
        // lane (r, j) holds rows 4 j .. 4 j + 3 of the tile for token r
        const int64_t n0 = 16 * (t0 + g) + 4 * j;
        float v[4] = {a[0], a[1], a[2], a[3]};
        if (p.bias)
            for (int e = 0; e < 4; ++e) v[e] += bf16_to_f32(p.bias[n0 + e]);
        v2u o = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                 bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
        *reinterpret_cast<v2u *>(p.y + row * p.ldy + n0) = o;
    }
}

template <int LAYOUT, bool XFRAG, int G>
static hipError_t launch_w8_spw(const GemvW8Args &a, const GemvW8Plan &pl, hipStream_t st) {
    const dim3 grid((unsigned)((a.N / 16 + G - 1) / G), (unsigned)((a.M + 15) / 16));
    const dim3 block((unsigned)(pl.nw * 64));
    switch (pl.spw) {
    case 1: hipLaunchKernelGGL((gemv_w8_kernel<LAYOUT, XFRAG, G, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((gemv_w8_kernel<LAYOUT, XFRAG, G, 2>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((gemv_w8_kernel<LAYOUT, XFRAG, G, 4>), grid, block, 0, st, a); break;
    case 7:
        if constexpr (G * 7 <= 16)
            hipLaunchKernelGGL((gemv_w8_kernel<LAYOUT, XFRAG, G, 7>), grid, block, 0, st, a);
        else
            return hipErrorInvalidValue;
        break;
    default:
        // the plan keeps G * SPW <= 16 (registers)
        if constexpr (G * 8 <= 16)
            hipLaunchKernelGGL((gemv_w8_kernel<LAYOUT, XFRAG, G, 8>), grid, block, 0, st, a);
        else
            return hipErrorInvalidValue;
        break;
    }
    return hipGetLastError();
}

template <int LAYOUT, bool XFRAG>
static hipError_t launch_w8_g(const GemvW8Args &a, const GemvW8Plan &pl, hipStream_t st) {
    switch (pl.g) {
    case 1: return launch_w8_spw<LAYOUT, XFRAG, 1>(a, pl, st);
    case 4: return launch_w8_spw<LAYOUT, XFRAG, 4>(a, pl, st);
    default: return launch_w8_spw<LAYOUT, XFRAG, 2>(a, pl, st);
    }
}

hipError_t launch_gemv_w8(int layout, bool xfrag, const GemvW8Args &a, const GemvW8Plan &pl,
                          hipStream_t st) {
    if (layout == ROW32)
        return xfrag ? launch_w8_g<ROW32, true>(a, pl, st) : launch_w8_g<ROW32, false>(a, pl, st);
    return xfrag ? launch_w8_g<BLK32, true>(a, pl, st) : launch_w8_g<BLK32, false>(a, pl, st);
}

// Launch plan for T tiles, S steps and MB 16-token grid rows: tiles per
// workgroup G in {4, 2, 1} (the largest that still gives about one
// workgroup per compute unit, measured best on MI355X), up to eight
// wavefronts per workgroup, each with at most SPW in {1, 2, 4, 7, 8} steps.
// ok = false when S needs more than 64 steps' worth of registers.  nw_force
// and g_force (0 = none) override the choice, for tuning sweeps.
GemvW8Plan plan_gemv_w8(int64_t T, int64_t S, int64_t MB, int nw_force, int g_force) {
    GemvW8Plan pl{};
    int nw = S >= 8 ? 8 : (int)S;
    if (nw_force >= 1 && nw_force <= 8) nw = nw_force;
    const int64_t per = (S + nw - 1) / nw;
    pl.nw = nw;
    pl.spw = per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per == 7 ? 7 : 8;
    pl.ok = per <= 8;
    pl.g = 1;
    for (int g : {4, 2}) {
        if (g * pl.spw > 16) continue;                   // register budget
        if ((T + g - 1) / g * MB >= 224) {
            pl.g = g;
            break;
        }
    }
    if ((g_force == 1 || g_force == 2 || g_force == 4) && g_force * pl.spw <= 16) pl.g = g_force;
    return pl;
}

}  // namespace mx
