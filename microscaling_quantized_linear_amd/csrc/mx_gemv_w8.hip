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
    // a tile is 16 K bytes: S - 1 whole chunks, then the last step's valid
    // prefix of tailb bytes (no padding stored)
    const int64_t TILEB = 16 * p.K;
    const uint32_t tailb = (uint32_t)(TILEB - (S - 1) * 2048);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w + t0 * TILEB, (uint32_t)(ntiles * TILEB));
    v4u wv[SPW][G][2];
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t s = s0 + i;
                const uint32_t o = (uint32_t)(1024 * h + 16 * lane);
                const bool in = i < n && g < ntiles && (s < S - 1 || o < tailb);
                wv[i][g][h] = load16<kNT>(wr, in ? (uint32_t)(g * TILEB + s * 2048) + o : kOOB);
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

// The same product when the shape divides evenly and the activations come
// in the T16 layout: every wavefront owns exactly SPW steps and every
// workgroup G whole tiles, so no load needs a guard (T16 pads tokens past M
// and K past its end with zero bytes and code 127).  What differs is the
// front of the kernel: offsets are 32-bit with their uniform parts in scalar
// registers, and the first step's weight chunks are requested before
// anything else, so the weight stream starts at the top of the kernel; the
// activation copies and both codes follow, then the remaining weight chunks.
// Measured on MI355X, every cycle between the start of a wavefront and its
// weight requests adds to the time of this HBM-bound kernel.
template <int LAYOUT, int G, int SPW, int NW>
__global__ void __launch_bounds__(NW * 64) gemv_w8_even_kernel(GemvW8Args p) {
    constexpr int NQ = (SPW + 6) / 4;                   // quads SPW steps can span
    static_assert(2 * G * (SPW - 1) < 64, "vmcnt holds 6 bits");
    __shared__ __attribute__((aligned(1024))) uint8_t xs[NW][SPW * 2048];
    __shared__ v4f red[NW][G][64];

    const int lane = threadIdx.x % 64;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int r = lane % 16, j = lane / 16;
    const uint32_t S = (uint32_t)((p.K + 127) / 128), Q = (S + 3) / 4;
    const uint32_t MB = gridDim.y, mb = blockIdx.y;
    const uint32_t t0 = blockIdx.x * G;
    const uint32_t s0 = wave * SPW, qa = s0 / 4;
    const uint32_t lo = 16 * lane;

    // ---- 1. the first step's weight chunks ----
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w + (size_t)t0 * S * 2048, G * S * 2048);
    v4u wv[SPW][G][2];
    auto wload = [&](int i) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                wv[i][g][h] = __builtin_amdgcn_raw_buffer_load_b128(
                    wr, lo, (int)((g * S + s0 + i) * 2048 + h * 1024), kNT);
    };
    wload(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. activation fragments of the wavefront's steps -> its LDS ----
    uint8_t *myx = xs[wave];
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xf, MB * S * 2048);
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (lds_void_w8 *)(myx + (2 * i + h) * 1024), 16, (int)lo,
                (int)(((mb * S + s0 + i) * 2 + h) * 1024), 0, 0);

    // ---- 3. codes: one dword per quad of steps (byte u = step 4 q + u) ----
    // A quad past the last one reads zero through the resource bounds and is
    // never used.
    const __amdgpu_buffer_rsrc_t xcr = make_rsrc(p.xct, MB * Q * 256);
    uint32_t cxq[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c)
        cxq[c] = __builtin_amdgcn_raw_buffer_load_b32(xcr, 4 * lane, (int)((mb * Q + qa + c) * 256), 0);
    uint32_t cwq[G][NQ];
    if constexpr (LAYOUT == BLK32) {
        // tiles 2 R and 2 R + 1 share the codes of row group R
        const __amdgpu_buffer_rsrc_t cr = make_rsrc(p.codes, (uint32_t)(p.N / 32) * Q * 16);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                if (G % 2 == 0 && g % 2 == 1) {
                    cwq[g][c] = cwq[g - 1][c];
                    continue;
                }
                cwq[g][c] = __builtin_amdgcn_raw_buffer_load_b32(
                    cr, 4 * j, (int)((((t0 + g) / 2) * Q + qa + c) * 16), 0);
            }
    } else {
        const __amdgpu_buffer_rsrc_t cr = make_rsrc(p.codes, (uint32_t)(p.N / 16) * Q * 256);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < NQ; ++c)
                cwq[g][c] = __builtin_amdgcn_raw_buffer_load_b32(
                    cr, 4 * lane, (int)(((t0 + g) * Q + qa + c) * 256), 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. the remaining weight chunks ----
#pragma unroll
    for (int i = 1; i < SPW; ++i) wload(i);
    __builtin_amdgcn_sched_barrier(0);

    // Everything before the remaining weight chunks has landed once at most
    // that many loads are outstanding (in-order completion); the compiler
    // does not count the copies into LDS, hence the explicit wait.
    __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * G * (SPW - 1)));
    __builtin_amdgcn_sched_barrier(0);

    // ---- 5. one scaled MFMA per tile and step ----
    v4f acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};
    auto run = [&](auto aconst) {
        constexpr int A = decltype(aconst)::value;
        static_for<0, SPW>([&](auto iconst) {
            constexpr int i = decltype(iconst)::value;
            constexpr int c = (A + i) / 4, u = (A + i) % 4;
            const v4u b0 = *reinterpret_cast<const v4u *>(myx + (2 * i) * 1024 + 16 * lane);
            const v4u b1 = *reinterpret_cast<const v4u *>(myx + (2 * i + 1) * 1024 + 16 * lane);
            const v8i bf = cat8(b0, b1);
#pragma unroll
            for (int g = 0; g < G; ++g)
                acc[g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    cat8(wv[i][g][0], wv[i][g][1]), bf, acc[g], 0, 0, u, (int)cwq[g][c], u,
                    (int)cxq[c]);
        });
    };
    switch (s0 % 4) {
    case 0: run(std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    default: run(std::integral_constant<int, 3>{}); break;
    }

    // ---- 6. wavefront-order reduction; wavefront g finishes tile g ----
#pragma unroll
    for (int g = 0; g < G; ++g) red[wave][g][lane] = acc[g];
    __syncthreads();
    if (wave >= G) return;
    const int g = wave;
    v4f a = red[0][g][lane];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) a += red[w2][g][lane];
    const int64_t row = 16 * (int64_t)mb + r;
    if (row >= p.M) return;
    // lane (r, j) holds rows 4 j .. 4 j + 3 of the tile for token r
    const int64_t n0 = 16 * (int64_t)(t0 + g) + 4 * j;
    float v[4] = {a[0], a[1], a[2], a[3]};
    if (p.bias)
        for (int e = 0; e < 4; ++e) v[e] += bf16_to_f32(p.bias[n0 + e]);
    v2u o = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16), bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
    *reinterpret_cast<v2u *>(p.y + row * p.ldy + n0) = o;
}

// The even-shape GEMV with the per-token MXFP8 quantization of the bf16
// activations done inside it ([rocm_native] apply_weights: at tiny M the
// quantization is fused into the product).  Each wavefront quantizes exactly
// the activation fragment it multiplies.  Lane (r, j) must end with token
// 16 mb + r, K 128 s + 16 j + [0, 16) and 128 s + 64 + 16 j + [0, 16): two
// halves of two 32-value blocks, whose other halves sit in the lane 16 apart.
//
// Loads: per step, four 1 KB loads of 4 tokens x 256 contiguous bytes (lane
// l reads token 4 u + l / 16, bytes 16 (l % 16) of the step).  Reading 16
// tokens x 64 bytes per load instead, with the caller's row stride, measured
// about 4 us slower per launch on MI355X.  Whole token tiles (M % 16 == 0,
// four or more steps a wavefront) copy them straight into a ring of four
// 4 KB LDS slots per wavefront (buffer loads with an LDS destination): each
// lane fetches the piece whose 16-byte position in its token's 256-byte row
// is piece ^ token, so the fragment reads are free of bank conflicts, and a
// wait counted from the fixed issue order (loads complete in issue order)
// precedes each step's reads.  Measured on MI355X: M = 16 11.05 against
// 11.08 us (five alternations, every pair lower), with 69 instead of 132
// VGPRs.  Partial tiles go through registers, skipping the loads of token
// groups past M, and a padded 16 x 272-byte LDS tile per wavefront turns
// them into the fragment order (rows 272 bytes apart keep both the writes
// and the 16-byte reads free of bank conflicts).
//
// Quantization: quant_half_block_cvt, the scaled hardware convert, which
// gives the bytes of mx_quant_act.  The MFMA's activation scale for lane
// (r, j) is the code of block j of the step, which a lane pair computes; one
// lane permute brings it to the lane that needs it.
//
// Order: the raw activations of the wavefront's first (up to) four steps
// first (L2 hits, they arrive long before the weights), then the weight
// chunks of the first step and the weight codes; each step is quantized just
// before its MFMAs (its LDS transpose one step earlier), after which the
// activations of the step four ahead and the next step's weight chunks are
// requested.  One step of weight chunks in flight per wavefront (1,792
// wavefronts, 7 MB in flight) measured fastest on MI355X: deeper windows,
// and activations requested with the weights of their own step, were
// slower.  Results are
// identical to mx_quant_act_t16 followed by the even-shape kernel: the same
// bytes, codes and MFMA order.
template <int LAYOUT, int RULE, int G, int SPW, int NW, bool FULL>
__global__ void __launch_bounds__(NW * 64) gemv_w8_fused_kernel(GemvW8Args p) {
    constexpr int XA = SPW > 4 ? 4 : SPW;              // steps of activations requested first
    constexpr int WIN = 1;                             // steps of weight chunks in flight
    constexpr int XROW = 272;                          // padded LDS row of one token
    __shared__ v4f red[NW][G][64];
    // whole tiles: activations straight into a ring of four 4 KB LDS slots
    constexpr bool kXD = FULL && XA == 4;
    __shared__ __attribute__((aligned(16))) uint8_t xt[kXD ? 1 : NW][16 * XROW];
    __shared__ __attribute__((aligned(1024))) uint8_t xd[kXD ? NW : 1][kXD ? 4 * 4096 : 16];

    const int lane = threadIdx.x % 64;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int r = lane % 16, j = lane / 16;
    const uint32_t S = (uint32_t)(p.K / 128), Q = (S + 3) / 4;
    const uint32_t mb = blockIdx.y;
    const uint32_t t0 = blockIdx.x * G;
    const uint32_t s0 = wave * SPW;
    const uint32_t lo = 16 * lane;

    // ---- 1. raw bf16 activations of the wavefront's steps ----
    // load u of a step: token 16 mb + 4 u + j, bytes 16 r of the step's 256;
    // tokens past M read zeros through the resource bounds
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xb, (uint32_t)(p.M * p.ldx * 2));
    uint32_t xo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t tok = 16 * (int64_t)mb + 4 * u + j;
        xo[u] = tok < p.M ? (uint32_t)(tok * p.ldx * 2) + 16 * r : kOOB;
    }
    v4u xv[SPW][4];
    // FULL: every token tile of the call is whole (M % 16 == 0).  Otherwise
    // a load whose four tokens all lie past M is not issued (a uniform
    // branch): its registers hold zeros, what the resource bounds would give.
    // Measured on MI355X: M = 1 9.77 against 10.15 us and M = 4 9.90 against
    // 10.18 us; the branches cost M = 16 about 0.2 us, hence the two forms.
    const int64_t mrem = p.M - 16 * (int64_t)mb;       // tokens of this tile
    // LDS-destination form: copy u lands lane (r, j)'s 16 bytes at position
    // r of token 4 u + j's 256-byte row in the slot, so the lane fetches the
    // piece r ^ (4 u + j): piece p of token n sits at position p ^ n
    uint32_t xod[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t tok = 16 * (int64_t)mb + 4 * u + j;
        xod[u] = tok < p.M ? (uint32_t)(tok * p.ldx * 2) + 16 * (r ^ (4 * u + j)) : kOOB;
    }
    uint8_t *const myd = xd[kXD ? wave : 0];
    auto xload = [&](int i) {
        if constexpr (kXD) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (lds_void_w8 *)(myd + (i % 4) * 4096 + u * 1024), 16, (int)xod[u],
                    (int)(256 * (s0 + i)), 0, 0);
            return;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (FULL || 4 * u < mrem)
                xv[i][u] =
                    __builtin_amdgcn_raw_buffer_load_b128(xr, xo[u], (int)(256 * (s0 + i)), 0);
            else
                xv[i][u] = v4u{0u, 0u, 0u, 0u};
        }
    };
    // The first XA steps' activations go out before any weight request;
    // step i + XA's go out in step i, ahead of that step's weight refill.
    // Measured on MI355X (M = 16, N = K = 7168, seven steps a wavefront):
    // all seven up front 11.23 us, four 11.07 us, five 11.17, six 11.14,
    // three 11.19, two 11.42; M = 1 and 4: 10.26 against 10.68-10.70 us.
    // Fewer up front lets the first weight requests of all eight
    // wavefronts out sooner (a CU's address unit takes each wavefront's
    // activation loads in turn); too few put the later ones in the chain.
#pragma unroll
    for (int i = 0; i < XA; ++i) xload(i);
    // Whole tiles run at wave priority 1 except while issuing activation
    // loads, so the compute unit serves those behind everything else:
    // measured on MI355X, M = 16 11.07 against 11.09 us (five alternations,
    // every pair lower).
    if constexpr (FULL) __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. the first WIN steps of weight chunks ----
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w + (size_t)t0 * S * 2048, G * S * 2048);
    v4u wv[SPW][G][2];
    auto wload = [&](int i) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                wv[i][g][h] = __builtin_amdgcn_raw_buffer_load_b128(
                    wr, lo, (int)((g * S + s0 + i) * 2048 + h * 1024), kNT);
    };
#pragma unroll
    for (int i = 0; i < WIN; ++i) wload(i);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. weight codes: the dwords of the quads the wavefront's steps
    // span (byte u of a dword is step 4 q + u; a quad past the last one
    // reads zeros through the resource bounds or codes that go unused).  Each
    // step's byte is picked by a wavefront-uniform select and shift: an array
    // indexed by the runtime quad offset would go to LDS (measured: byte
    // loads per step instead cost 0.13 us at M = 1) ----
    constexpr int NQ = (SPW + 6) / 4;
    const uint32_t qa = s0 / 4, a0 = s0 % 4;
    uint32_t cwd[G][NQ];
    if constexpr (LAYOUT == BLK32) {
        // tiles 2 R and 2 R + 1 share the codes of row group R
        const __amdgpu_buffer_rsrc_t cr = make_rsrc(p.codes, (uint32_t)(p.N / 32) * Q * 16);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                if (G % 2 == 0 && g % 2 == 1) {
                    cwd[g][c] = cwd[g - 1][c];
                    continue;
                }
                cwd[g][c] = __builtin_amdgcn_raw_buffer_load_b32(
                    cr, 4 * j, (int)((((t0 + g) / 2) * Q + qa + c) * 16), 0);
            }
    } else {
        const __amdgpu_buffer_rsrc_t cr = make_rsrc(p.codes, (uint32_t)(p.N / 16) * Q * 256);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < NQ; ++c)
                cwd[g][c] = __builtin_amdgcn_raw_buffer_load_b32(
                    cr, 4 * lane, (int)(((t0 + g) * Q + qa + c) * 256), 0);
    }
    auto wcode = [&](int g, int i) -> uint32_t {
        const uint32_t k = a0 + (uint32_t)i;            // uniform: step s0 + i is quad qa + k / 4
        uint32_t d = cwd[g][0];
#pragma unroll
        for (int c = 1; c < NQ; ++c) d = k >= 4u * c ? cwd[g][c] : d;
        return (d >> (8 * (k & 3u))) & 0xFFu;
    };
    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. per step: transpose, quantize, one scaled MFMA per tile, refill ----
    // Lane j computes the codes of blocks j/2 (first half) and 2 + j/2
    // (second half); the MFMA wants block j: lanes j = 0 and 3 hold it, lane
    // j = 1 takes the first-half code of lane j = 2, lane j = 2 the
    // second-half code of lane j = 1.
    uint8_t *tile = xt[wave];
    const int src = j == 1 ? lane + 16 : (j == 2 ? lane - 16 : lane);
    v4f acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};
    // The transpose runs one step ahead: step i + 1's tile write is queued
    // behind step i's operand reads (a wavefront's LDS operations run in
    // order) and its operand reads go out before step i's MFMAs, so the LDS
    // round trip overlaps the quantization and the matrix cores.
    const uint8_t *mine = tile + r * XROW + 32 * j;
    auto put = [&](int i) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<v4u *>(tile + (4 * u + j) * XROW + 16 * r) = xv[i][u];
    };
    v4u f[4], fn[4];
    auto get = [&](v4u (&d)[4]) {
        d[0] = *reinterpret_cast<const v4u *>(mine);
        d[1] = *reinterpret_cast<const v4u *>(mine + 16);
        d[2] = *reinterpret_cast<const v4u *>(mine + 128);
        d[3] = *reinterpret_cast<const v4u *>(mine + 144);
    };
    // DMA form: step k's fragment straight from its LDS slot (pieces at
    // position piece ^ token), after a wait that leaves outstanding only the
    // loads issued after step k's copies
    constexpr int NCODE = LAYOUT == BLK32 ? (G % 2 == 0 ? G / 2 : G) * NQ : G * NQ;
    auto nafter = [](int k) constexpr {
        // loads issued after step k's four copies, up to the read of step k
        // (issue order: X_0 .. X_{XA-1} (four each), W_0 .. W_{WIN-1},
        // codes; then step i issues X_{i+XA} and W_{i+WIN} after reading
        // step i + 1's fragment)
        int n = 0;
        bool seen = false;
        for (int i = 0; i < XA; ++i) {
            if (seen) n += 4;
            if (i == k) seen = true;
        }
        if (seen) n += WIN * 2 * G + NCODE;
        if (k == 0) return n;
        for (int i = 0; i + 1 < k; ++i) {
            if (i + XA < SPW) {
                if (seen) n += 4;
                if (i + XA == k) seen = true;
            }
            if (i + WIN < SPW && seen) n += 2 * G;
        }
        return n;
    };
    auto getd = [&](v4u (&d)[4], auto kconst) {
        constexpr int k = decltype(kconst)::value;
        constexpr int n = nafter(k);
        static_assert(n >= 0 && n < 64, "vmcnt holds 6 bits");
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_only(n));
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t *row = myd + (k % 4) * 4096 + r * 256;
        d[0] = *reinterpret_cast<const v4u *>(row + 16 * ((2 * j) ^ r));
        d[1] = *reinterpret_cast<const v4u *>(row + 16 * ((2 * j + 1) ^ r));
        d[2] = *reinterpret_cast<const v4u *>(row + 16 * ((8 + 2 * j) ^ r));
        d[3] = *reinterpret_cast<const v4u *>(row + 16 * ((9 + 2 * j) ^ r));
    };
    if constexpr (kXD) {
        getd(f, std::integral_constant<int, 0>{});
    } else {
        put(0);
        get(f);
    }
    static_for<0, SPW>([&](auto iconst) {
        constexpr int i = decltype(iconst)::value;
        if constexpr (!kXD && i + 1 < SPW) put(i + 1);
        const v4u f0 = f[0], f1 = f[1], f2 = f[2], f3 = f[3];
        if constexpr (i + 1 < SPW) {
            if constexpr (kXD)
                getd(fn, std::integral_constant<int, i + 1>{});
            else
                get(fn);
        }
        uint32_t c0, c1;
        const v4u q0 = quant_half_block_cvt<RULE>(f0, f1, c0);
        const v4u q1 = quant_half_block_cvt<RULE>(f2, f3, c1);
        const v8i bq = cat8(q0, q1);
        const uint32_t got = (uint32_t)__shfl((int)(j == 2 ? c0 : c1), src);
        const uint32_t cx = j == 0 ? c0 : (j == 3 ? c1 : got);
#pragma unroll
        for (int g = 0; g < G; ++g)
            acc[g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                cat8(wv[i][g][0], wv[i][g][1]), bq, acc[g], 0, 0, 0, (int)wcode(g, i), 0,
                (int)cx);
        // the refill goes out right behind this step's MFMAs (left alone,
        // the scheduler sinks it next to its use and exposes its latency).
        // Partial token tiles issue the weight refill at raised wave
        // priority, ahead of the other wavefronts' quantization work:
        // measured on MI355X, M = 4 9.80 against 9.93 us (M = 1 unchanged).
        // Whole tiles, which raising it cost 0.25 us at M = 16, instead run
        // at priority 1 and drop to 0 for the activation load (see the
        // first loads).
        if constexpr (FULL) __builtin_amdgcn_s_setprio(0);
        if constexpr (XA < SPW && i + XA < SPW) xload(i + XA);
        if constexpr (kXD) __builtin_amdgcn_sched_barrier(0);
        if constexpr (FULL) __builtin_amdgcn_s_setprio(1);
        if constexpr (i + WIN < SPW) {
            if constexpr (!FULL) __builtin_amdgcn_s_setprio(3);
            wload(i + WIN);
            if constexpr (!FULL) __builtin_amdgcn_s_setprio(0);
        }
        if constexpr (i + 1 < SPW) {
#pragma unroll
            for (int c = 0; c < 4; ++c) f[c] = fn[c];
        }
        __builtin_amdgcn_sched_barrier(0);
    });

    // ---- 5. wavefront-order reduction; wavefront g finishes tile g ----
#pragma unroll
    for (int g = 0; g < G; ++g) red[wave][g][lane] = acc[g];
    __syncthreads();
    const int64_t row = 16 * (int64_t)mb + r;
    if (wave >= G || row >= p.M) return;
    const int g = wave;
    v4f a = red[0][g][lane];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) a += red[w2][g][lane];
    const int64_t n0 = 16 * (int64_t)(t0 + g) + 4 * j;
    float v[4] = {a[0], a[1], a[2], a[3]};
    if (p.bias)
        for (int e = 0; e < 4; ++e) v[e] += bf16_to_f32(p.bias[n0 + e]);
    v2u o = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16), bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
    *reinterpret_cast<v2u *>(p.y + row * p.ldy + n0) = o;
}

// The even-shape GEMV on a pre-quantized row-major activation: mx_quant_act's
// e4m3 [M, ldq] with row-major codes [M, ldc], the form [rocm_native]
// apply_weights takes as a quantized activation.  The activation bytes go
// straight into LDS (buffer loads with an LDS destination, as in the T16
// kernel), but each 1 KB copy reads 8 tokens x 128 contiguous bytes (one step
// of each): copy u of step i, lane l = 8 t + q fetches token r = 8 u + t's
// 16-byte piece q ^ (r / 2) into LDS slot (t, q).  Rows of 16 tokens x 64
// bytes per copy instead, with the caller's row stride, concentrate each copy
// on few L2 channels.  Lane (r, j) then reads its pieces j and 4 + j (K 16 j
// .. and 64 + 16 j .. of the step) at slot (r % 8, p ^ (r / 2)) of copy r / 8:
// the 16 tokens' reads fall on 16 distinct 16-byte bank groups.  Its scale
// byte is token r's code of block 4 s + j, read from the row-major codes.
// Weight chunks as in the T16 kernel.  The product is the T16 path's, bit for
// bit (same bytes, codes and MFMA order).
template <int LAYOUT, int G, int SPW, int NW>
__global__ void __launch_bounds__(NW * 64) gemv_w8_rm_kernel(GemvW8Args p) {
    static_assert(2 * G * (SPW - 1) < 64, "vmcnt holds 6 bits");
    __shared__ __attribute__((aligned(1024))) uint8_t xs[NW][SPW * 2048];
    __shared__ v4f red[NW][G][64];

    const int lane = threadIdx.x % 64;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int r = lane % 16, j = lane / 16;
    const uint32_t S = (uint32_t)(p.K / 128), Q = (S + 3) / 4;
    const uint32_t mb = blockIdx.y;
    const uint32_t t0 = blockIdx.x * G;
    const uint32_t s0 = wave * SPW;
    const uint32_t lo = 16 * lane;

    // ---- 1. the first step's weight chunks ----
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w + (size_t)t0 * S * 2048, G * S * 2048);
    v4u wv[SPW][G][2];
    auto wload = [&](int i) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                wv[i][g][h] = __builtin_amdgcn_raw_buffer_load_b128(
                    wr, lo, (int)((g * S + s0 + i) * 2048 + h * 1024), kNT);
    };
    wload(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. activation bytes of the wavefront's steps -> its LDS (tokens
    // past M read zeros through the resource bounds) ----
    uint8_t *myx = xs[wave];
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xq, (uint32_t)(p.M * p.ldq));
    uint32_t xo[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tr = 8 * u + lane / 8;                 // token within the tile
        const int64_t tok = 16 * (int64_t)mb + tr;
        const uint32_t piece = (uint32_t)((lane % 8) ^ (tr / 2));
        xo[u] = tok < p.M ? (uint32_t)(tok * p.ldq) + 16 * piece : kOOB;
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (lds_void_w8 *)(myx + (2 * i + u) * 1024), 16, (int)xo[u],
                (int)(128 * (s0 + i)), 0, 0);

    // ---- 3. codes: the activation's from the row-major codes, one byte per
    // step; the weights' from their dwords (byte u is step 4 q + u) ----
    const __amdgpu_buffer_rsrc_t xcr = make_rsrc(p.xc, (uint32_t)(p.M * p.ldc));
    const int64_t tr = 16 * (int64_t)mb + r;
    const uint32_t cxo = tr < p.M ? (uint32_t)(tr * p.ldc) + (uint32_t)j : kOOB;
    uint32_t cx[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i)
        cx[i] = __builtin_amdgcn_raw_buffer_load_b8(xcr, cxo, (int)(4 * (s0 + i)), 0);
    // the weights': one dword per quad the wavefront's steps span, each
    // step's byte picked by a wavefront-uniform select and shift
    constexpr int NQ = (SPW + 6) / 4;
    const uint32_t qa = s0 / 4, a0 = s0 % 4;
    uint32_t cwd[G][NQ];
    if constexpr (LAYOUT == BLK32) {
        const __amdgpu_buffer_rsrc_t cr = make_rsrc(p.codes, (uint32_t)(p.N / 32) * Q * 16);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                if (G % 2 == 0 && g % 2 == 1) {
                    cwd[g][c] = cwd[g - 1][c];
                    continue;
                }
                cwd[g][c] = __builtin_amdgcn_raw_buffer_load_b32(
                    cr, 4 * j, (int)((((t0 + g) / 2) * Q + qa + c) * 16), 0);
            }
    } else {
        const __amdgpu_buffer_rsrc_t cr = make_rsrc(p.codes, (uint32_t)(p.N / 16) * Q * 256);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < NQ; ++c)
                cwd[g][c] = __builtin_amdgcn_raw_buffer_load_b32(
                    cr, 4 * lane, (int)(((t0 + g) * Q + qa + c) * 256), 0);
    }
    auto wcode = [&](int g, int i) -> uint32_t {
        const uint32_t k = a0 + (uint32_t)i;
        uint32_t d = cwd[g][0];
#pragma unroll
        for (int c = 1; c < NQ; ++c) d = k >= 4u * c ? cwd[g][c] : d;
        return (d >> (8 * (k & 3u))) & 0xFFu;
    };
    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. the remaining weight chunks ----
#pragma unroll
    for (int i = 1; i < SPW; ++i) wload(i);
    __builtin_amdgcn_sched_barrier(0);

    // Everything before the remaining weight chunks has landed once at most
    // that many loads are outstanding (in-order completion); the compiler
    // does not count the copies into LDS, hence the explicit wait.
    __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * G * (SPW - 1)));
    __builtin_amdgcn_sched_barrier(0);

    // ---- 5. one scaled MFMA per tile and step ----
    const uint8_t *rd0 = myx + (r / 8) * 1024 + (r % 8) * 128;
    const uint32_t sw = (uint32_t)(r / 2);
    const uint32_t pa = 16u * ((uint32_t)j ^ sw), pb = 16u * ((uint32_t)(4 + j) ^ sw);
    v4f acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};
    static_for<0, SPW>([&](auto iconst) {
        constexpr int i = decltype(iconst)::value;
        const uint8_t *base = rd0 + i * 2048;
        const v8i bq = cat8(*reinterpret_cast<const v4u *>(base + pa),
                            *reinterpret_cast<const v4u *>(base + pb));
#pragma unroll
        for (int g = 0; g < G; ++g)
            acc[g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                cat8(wv[i][g][0], wv[i][g][1]), bq, acc[g], 0, 0, 0, (int)wcode(g, i), 0,
                (int)cx[i]);
    });

    // ---- 6. wavefront-order reduction; wavefront g finishes tile g ----
#pragma unroll
    for (int g = 0; g < G; ++g) red[wave][g][lane] = acc[g];
    __syncthreads();
    const int64_t row = 16 * (int64_t)mb + r;
    if (wave >= G || row >= p.M) return;
    const int g = wave;
    v4f a = red[0][g][lane];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) a += red[w2][g][lane];
    const int64_t n0 = 16 * (int64_t)(t0 + g) + 4 * j;
    float v[4] = {a[0], a[1], a[2], a[3]};
    if (p.bias)
        for (int e = 0; e < 4; ++e) v[e] += bf16_to_f32(p.bias[n0 + e]);
    v2u o = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16), bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
    *reinterpret_cast<v2u *>(p.y + row * p.ldy + n0) = o;
}

// launch helpers of the even-shape kernels: SPW in {1, 2, 4, 7, 8}, G in
// {1, 2, 4} with G * SPW <= 16, eight wavefronts
template <int G, class F>
static hipError_t even_spw(int spw, F &&f) {
    switch (spw) {
    case 1: return f(std::integral_constant<int, G>{}, std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, G>{}, std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, G>{}, std::integral_constant<int, 4>{});
    case 7:
        if constexpr (G * 7 <= 16) return f(std::integral_constant<int, G>{}, std::integral_constant<int, 7>{});
        break;
    case 8:
        if constexpr (G * 8 <= 16) return f(std::integral_constant<int, G>{}, std::integral_constant<int, 8>{});
        break;
    default: break;
    }
    return hipErrorInvalidValue;
}
template <class F>
static hipError_t even_dispatch(const GemvW8Plan &pl, F &&f) {
    switch (pl.g) {
    case 1: return even_spw<1>(pl.spw, f);
    case 2: return even_spw<2>(pl.spw, f);
    case 4: return even_spw<4>(pl.spw, f);
    default: return hipErrorInvalidValue;
    }
}

template <bool FULL>
static hipError_t launch_fused(int layout, int rule, const GemvW8Args &a, const GemvW8Plan &pl,
                               hipStream_t st) {
    const dim3 grid((unsigned)(a.N / 16 / pl.g), (unsigned)((a.M + 15) / 16)), block(512);
    return even_dispatch(pl, [&](auto gc, auto sc) -> hipError_t {
        constexpr int G = decltype(gc)::value, SPW = decltype(sc)::value;
        if (layout == ROW32) {
            if (rule == RULE_OCP)
                hipLaunchKernelGGL((gemv_w8_fused_kernel<ROW32, RULE_OCP, G, SPW, 8, FULL>), grid, block, 0, st, a);
            else
                hipLaunchKernelGGL((gemv_w8_fused_kernel<ROW32, RULE_CEIL448, G, SPW, 8, FULL>), grid, block, 0, st, a);
        } else {
            if (rule == RULE_OCP)
                hipLaunchKernelGGL((gemv_w8_fused_kernel<BLK32, RULE_OCP, G, SPW, 8, FULL>), grid, block, 0, st, a);
            else
                hipLaunchKernelGGL((gemv_w8_fused_kernel<BLK32, RULE_CEIL448, G, SPW, 8, FULL>), grid, block, 0, st, a);
        }
        return hipSuccess;
    });
}

hipError_t launch_gemv_w8_fused(int layout, int rule, const GemvW8Args &a, const GemvW8Plan &pl,
                                hipStream_t st) {
    if (!gemv_w8_even(a.N, a.K, pl) || a.K % 128 != 0) return hipErrorInvalidValue;
    const hipError_t e = a.M % 16 == 0 ? launch_fused<true>(layout, rule, a, pl, st)
                                       : launch_fused<false>(layout, rule, a, pl, st);
    if (e != hipSuccess) return e;
    return hipGetLastError();
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
    if (xfrag && gemv_w8_even(a.N, a.K, pl)) {
        const dim3 grid((unsigned)(a.N / 16 / pl.g), (unsigned)((a.M + 15) / 16)), block(512);
        const hipError_t e = even_dispatch(pl, [&](auto gc, auto sc) -> hipError_t {
            constexpr int G = decltype(gc)::value, SPW = decltype(sc)::value;
            if (layout == ROW32)
                hipLaunchKernelGGL((gemv_w8_even_kernel<ROW32, G, SPW, 8>), grid, block, 0, st, a);
            else
                hipLaunchKernelGGL((gemv_w8_even_kernel<BLK32, G, SPW, 8>), grid, block, 0, st, a);
            return hipSuccess;
        });
        if (e != hipSuccess) return e;
        return hipGetLastError();
    }
    if (!xfrag && gemv_w8_even(a.N, a.K, pl)) {
        const dim3 grid((unsigned)(a.N / 16 / pl.g), (unsigned)((a.M + 15) / 16)), block(512);
        const hipError_t e = even_dispatch(pl, [&](auto gc, auto sc) -> hipError_t {
            constexpr int G = decltype(gc)::value, SPW = decltype(sc)::value;
            if (layout == ROW32)
                hipLaunchKernelGGL((gemv_w8_rm_kernel<ROW32, G, SPW, 8>), grid, block, 0, st, a);
            else
                hipLaunchKernelGGL((gemv_w8_rm_kernel<BLK32, G, SPW, 8>), grid, block, 0, st, a);
            return hipSuccess;
        });
        if (e != hipSuccess) return e;
        return hipGetLastError();
    }
    if (layout == ROW32)
        return xfrag ? launch_w8_g<ROW32, true>(a, pl, st) : launch_w8_g<ROW32, false>(a, pl, st);
    return xfrag ? launch_w8_g<BLK32, true>(a, pl, st) : launch_w8_g<BLK32, false>(a, pl, st);
}

}  // namespace mx
