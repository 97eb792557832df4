// mx_gemm.hip -- prefill MXFP8 GEMM (W8A8), y = x W^T at large M.
//
// ([rocm_native] module notes and apply_weights: fp8 e4m3 weights with E8M0
// block scales consumed directly by the CDNA4 microscaling matrix cores,
// activations quantized per token with row-major codes.)
//
// Workgroup tile: BN weight rows x 256 tokens, 4 wavefronts side by side
// along the tokens: each wavefront owns all BN rows and 64 tokens, NTW x 2
// output tiles of 32 x 32 accumulated by v_mfma_scale_f32_32x32x64_f8f6f4
// (A = weights, B = activations, both with per-lane E8M0 scales).  On
// MI355X the 32 x 32 x 64 form issues at its full rate (64 cycles for 2^17
// flop); the 16 x 16 x 128 form measured about 41 cycles for half as many.
// Per 128-K step the workgroup copies its weight chunks (W-T16, 2 KB per 16
// rows) and its activation rows (already in fragment order when they come in
// the T16 layout, else rearranged into it by the copy's addressing) straight
// from memory into one of two LDS buffers (buffer loads with an LDS
// destination) while the matrix cores work on the other; one barrier per
// step.  A 32 x 32 x 64 operand lane (row r, K group g) reads its two
// 16-byte pieces from those 16-row chunks.  Scale codes are read once per
// four steps as dwords whose byte u is step 4q + u's code, picked by the
// MFMA's byte select.  Out-of-range rows and K tails read zeros through
// buffer-resource bounds.
#include "mx_device.h"
#include "mx_kernels.h"

#include <type_traits>

namespace mx {

constexpr int kBM = 256;           // tokens per workgroup

// Per LDS buffer: the step's weight chunks (2 NTW x 2 KB, W-T16 as stored) then
// the activation tile in MFMA fragment order (16 chunks of 16 rows x 128 K:
// byte 1024 h + 16 l of chunk mt holds row 16 mt + l%16, K 64 h + 16 (l/16)).
template <int NTW>
struct GemmSmem {
    static constexpr int kWBytes = 2 * NTW * 2048;
    static constexpr int kXBytes = kBM / 16 * 2048;
    static constexpr int kBuf = kWBytes + kXBytes;
    static constexpr int kDma = kBuf / 1024;              // 1 KB DMA loads per step
};

typedef __attribute__((address_space(3))) void lds_void;

template <int LAYOUT, int NTW>
__global__ void __launch_bounds__(256, 1) gemm_w8a8_kernel(GemmArgs p) {
    using SM = GemmSmem<NTW>;
    // two distinct buffers: the compiler can then tell the DMA into one from
    // the operand reads of the other and waits only where it must
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[SM::kBuf];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[SM::kBuf];
    constexpr int BN = NTW * 32;
    static_assert(BN <= 256, "one bias value per thread");
    __shared__ __attribute__((aligned(16))) uint16_t bias_lds[BN];
    const int tid = threadIdx.x, lane = tid % 64;
    // bounded so the compiler can tell the two LDS buffers' accesses apart
    // (otherwise it waits for the next step's copies before reading this one)
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64) & 3;
    const int r = lane % 16, j = lane / 16;
    const int64_t Kp = (p.K + 127) / 128 * 128, S = Kp / 128, T = p.N / 16, Q = (S + 3) / 4;
    const int64_t KB = p.K / 32;

    // tile order: consecutive workgroups go to different XCDs; give each XCD
    // a band of N tiles so the weight panels it streams stay in its L2
    const int64_t tiles_n = (p.N + BN - 1) / BN;
    int64_t bid = blockIdx.x, tn, tm;
    if (tiles_n % 8 == 0) {
        const int64_t xcd = bid % 8, local = bid / 8, per = tiles_n / 8;
        tn = xcd * per + local % per;
        tm = local / per;
    } else {
        tn = bid % tiles_n;
        tm = bid / tiles_n;
    }
    const int64_t n0 = tn * BN, m0 = tm * kBM;
    const int64_t t0 = n0 / 16;                           // first weight tile

    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w, (uint32_t)(T * S * 2048));
    const int64_t MB = (p.M + 15) / 16;
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(p.xq, p.xt16 ? (uint32_t)(MB * S * 2048) : (uint32_t)(p.M * p.ldq));
    const __amdgpu_buffer_rsrc_t xcr = make_rsrc(p.xct, (uint32_t)act_codes_t16_bytes(p.M, p.K));
    const __amdgpu_buffer_rsrc_t cr =
        make_rsrc(p.codes, LAYOUT == ROW32 ? (uint32_t)(T * Q * 256)
                                           : (uint32_t)((p.N / 32) * Q * 16));

    // ---- DMA assignment: wave w issues weight chunk-halves w, w + 4, ... and
    // activation chunk-halves w, w + 4, ...; chunk-half i lands at i KB.
    // Offsets of out-of-range loads get bit 31 set (every resource is below
    // 2 GiB, so those lanes read zeros); no branches in the loop body.
    constexpr int kWq = NTW;                              // 4 NTW weight loads / 4 waves
    constexpr int kXq = 8;                                // 32 activation loads / 4 waves
    uint32_t wbase[kWq], xbase[kXq], xkmax[kXq];
#pragma unroll
    for (int q = 0; q < kWq; ++q) {
        const int i = wave + 4 * q, c = i / 2, h = i % 2;
        const int64_t t = t0 + c;
        wbase[q] = t < T ? (uint32_t)(t * S * 2048 + 1024 * h + 16 * lane) : kOOB;
    }
#pragma unroll
    for (int q = 0; q < kXq; ++q) {
        // wavefront w copies its own 64 tokens: chunks 4 w .. 4 w + 3, both
        // halves (chunk-half 8 w + q), so it may read them without a barrier
        const int i = 8 * wave + q, mc = i / 2, h = i % 2;
        const int64_t row = m0 + 16 * mc + r, k = 64 * h + 16 * j;
        if (p.xt16) {
            // T16: the 1 KB block (16-token tile, step, half) is already in
            // fragment order; padding bytes are zeros
            const int64_t mb = (m0 + 16 * mc) / 16;
            xbase[q] = mb < MB ? (uint32_t)(mb * S * 2048 + h * 1024 + 16 * lane) : kOOB;
            xkmax[q] = (uint32_t)S;
        } else {
            xbase[q] = row < p.M ? (uint32_t)(row * p.ldq + k) : kOOB;
            xkmax[q] = (uint32_t)((p.K - k + 127) / 128);     // steps with 128 s + k < K
        }
    }
    const uint32_t xstep = p.xt16 ? 2048u : 128u;         // bytes per 128-K step
    // copy i of step s into buf: i < kWq weight chunk-halves, then activation ones
    constexpr int kCopies = kWq + kXq;
    auto dma_one = [&](uint8_t *buf, int64_t s, int i) {
        const uint32_t su = (uint32_t)s;
        if (i < kWq) {
            const uint32_t past = su >= (uint32_t)S ? kOOB : 0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (lds_void *)(buf + (wave + 4 * i) * 1024), 16,
                (int)((wbase[i] + su * 2048u) | past), 0, 0, 0);
        } else {
            const int q = i - kWq;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (lds_void *)(buf + SM::kWBytes + (8 * wave + q) * 1024), 16,
                (int)((xbase[q] + su * xstep) | (su >= xkmax[q] ? kOOB : 0u)), 0, 0, 0);
        }
    };
    auto dma = [&](uint8_t *buf, int64_t s) {
#pragma unroll
        for (int i = 0; i < kCopies; ++i) dma_one(buf, s, i);
    };

    // ---- 32 x 32 x 64 operands: lane (g, rr) = lane / 32, lane % 32 holds
    // row rr with K 16 g .. and 32 + 16 g .. of a 64-K half-step kh; in the
    // 16-row chunks that is chunk 2 T + rr / 16, bytes 1024 kh + 256 g +
    // 16 (rr % 16) and 512 further ----
    const int rr = lane % 32, g = lane / 32;
    const int off_lane = (rr / 16) * 2048 + 256 * g + 16 * (rr % 16);

    // ---- per-lane scale dwords of one quad of four steps: byte u of each
    // dword is step 4 q + u's code, picked by the MFMA's opsel; lane (g, rr)
    // of half-step kh needs block 2 kh + g of its row ----
    struct QScales {
        uint32_t w[NTW][2], x[2][2];
    };
    uint32_t cwbase[NTW][2], cxbase[2][2];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const int jb = 2 * kh + g;                    // block of the 128-K step
            const int64_t row = n0 + 32 * nt + rr;
            if (LAYOUT == ROW32)
                cwbase[nt][kh] = row < p.N ? (uint32_t)((row / 16) * Q * 256 +
                                                        4 * (16 * jb + row % 16)) : kOOB;
            else
                cwbase[nt][kh] = row < p.N ? (uint32_t)((row / 32) * Q * 16 + 4 * jb) : kOOB;
        }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const int jb = 2 * kh + g;
            const int64_t tok = m0 + 64 * wave + 32 * mt + rr;    // T16 code layout
            cxbase[mt][kh] = tok < 16 * MB ? (uint32_t)((tok / 16) * Q * 256 +
                                                         4 * (16 * jb + tok % 16)) : kOOB;
        }
    auto load_qscales = [&](int64_t q, QScales &out) {
        const uint32_t qu = (uint32_t)q, past = qu >= (uint32_t)Q ? kOOB : 0u;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
                out.w[nt][kh] = load4(cr, (cwbase[nt][kh] + qu * (LAYOUT == ROW32 ? 256u : 16u)) | past);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
                out.x[mt][kh] = load4(xcr, (cxbase[mt][kh] + qu * 256u) | past);
    };

    typedef float v16f __attribute__((ext_vector_type(16)));
    // first written by the first step's MFMAs, which take a zero C operand
    v16f acc[NTW][2];

    // one 128-K step, step u of its quad: the MFMAs of step s from `cur` with
    // the quad's scales `sc`, interleaved with the copies of step s + 1 into
    // `nxt`.  The 2 NTW
    // MFMA groups (half-step kh, weight tile nt) each take two MFMAs; a
    // group's weight fragment is read two groups ahead, the activation
    // fragments of a half-step with the reads of its first groups.
    auto rd = [&](const uint8_t *base, int kh) -> v8i {
        const uint8_t *cp = base + off_lane + 1024 * kh;
        return cat8(*reinterpret_cast<const v4u *>(cp), *reinterpret_cast<const v4u *>(cp + 512));
    };
    // the wavefront's activation fragments of one step (both half-steps);
    // this wavefront alone copies them, so they are read as soon as its own
    // copies have landed, before the barrier
    v8i bf[2][2];
    auto read_b = [&](const uint8_t *buf) {
        const uint8_t *xb = buf + SM::kWBytes + (4 * wave) * 2048;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) bf[kh][mt] = rd(xb + 2 * mt * 2048, kh);
    };
    auto step = [&](uint8_t *cur, uint8_t *nxt, int64_t s, const QScales &sc, auto uconst,
                    auto firstconst) {
        constexpr int U = decltype(uconst)::value;
        constexpr bool kFirst = decltype(firstconst)::value;
        const uint8_t *wb = cur;
        constexpr int NG = 2 * NTW;                       // groups (kh, nt), kh major
        v8i af[3];
        auto issue = [&](int k) {                         // group k's weight fragment
            af[k % 3] = rd(wb + 2 * (k % NTW) * 2048, k / NTW);
        };
        issue(0);
        issue(1);
        // the copies of step s + 1 go out two per MFMA group from the top of
        // the step: issued all at once, the four wavefronts' 60 KB queue on
        // the CU's address path (64 B/clock) and hold back the MFMAs; spread,
        // the copies and the matrix cores overlap and the last copy still has
        // half a step to land before the barrier
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            if (2 * k < kCopies) dma_one(nxt, s + 1, 2 * k);
            if (2 * k + 1 < kCopies) dma_one(nxt, s + 1, 2 * k + 1);
            if (k + 2 < NG) issue(k + 2);
            __builtin_amdgcn_sched_barrier(0);
            const int kh = k / NTW, nt = k % NTW;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                acc[nt][mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af[k % 3], bf[kh][mt], kFirst && kh == 0 ? v16f{} : acc[nt][mt], 0, 0, U,
                    (int)sc.w[nt][kh], U, (int)sc.x[mt][kh]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // this wavefront's copies of step s + 1 have landed before any
        // wavefront reads them
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        read_b(nxt);
        __syncthreads();
    };
    using U0 = std::integral_constant<int, 0>;
    using U1 = std::integral_constant<int, 1>;
    using U2 = std::integral_constant<int, 2>;
    using U3 = std::integral_constant<int, 3>;
    using F0 = std::false_type;

    // the workgroup's BN bias values, staged in LDS under the first barrier
    // (the bias needs only 2-byte alignment: one element per thread)
    if (p.bias && tid < BN) bias_lds[tid] = n0 + tid < p.N ? p.bias[n0 + tid] : 0;

    QScales qa, qb;
    dma(lds0, 0);
    load_qscales(0, qa);
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __syncthreads();
    read_b(lds0);
    // eight steps (two quads) per iteration: each LDS buffer is a fixed object
    // and the two scale sets alternate without copies; a step at or past S
    // reads zeros and adds nothing
    for (int64_t s = 0; s < S; s += 8) {
        const int64_t q = s / 4;
        load_qscales(q + 1, qb);
        if (s == 0)
            step(lds0, lds1, s + 0, qa, U0{}, std::true_type{});
        else
            step(lds0, lds1, s + 0, qa, U0{}, F0{});
        step(lds1, lds0, s + 1, qa, U1{}, F0{});
        step(lds0, lds1, s + 2, qa, U2{}, F0{});
        step(lds1, lds0, s + 3, qa, U3{}, F0{});
        load_qscales(q + 2, qa);
        step(lds0, lds1, s + 4, qb, U0{}, F0{});
        step(lds1, lds0, s + 5, qb, U1{}, F0{});
        step(lds0, lds1, s + 6, qb, U2{}, F0{});
        step(lds1, lds0, s + 7, qb, U3{}, F0{});
    }

    // ---- epilogue, straight from registers: element i of lane (g, rr) in
    // tile (nt, mt) is weight row 32 nt + 8 (i / 4) + 4 g + i % 4 and token
    // 32 mt + rr, so for a = i / 4 a lane holds 4 consecutive outputs of its
    // token row and lane rr + 32 the next 4.  Bias is added in fp32 and each
    // pair rounded to bf16 once (v_cvt_pk_bf16_f32); then v_permlane32_swap
    // trades the a = 1 (3) quarter of lanes 0..31 for the a = 0 (2) quarter of
    // lanes 32..63, and every lane stores 8 consecutive outputs (16 bytes):
    // lanes 0..31 those of a = 0 (2), lanes 32..63 those of a = 1 (3). ----
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    auto pk = [](float lo, float hi) -> uint32_t {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
    };
    auto epilogue = [&](auto biasconst) {
        constexpr bool kBias = decltype(biasconst)::value;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            v2u bias2[4];                                 // packed bf16 pairs
            if constexpr (kBias) {
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    bias2[a] = *reinterpret_cast<const v2u *>(bias_lds + 32 * nt + 8 * a + 4 * g);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const v16f &c = acc[nt][mt];
                const int64_t m = m0 + 64 * wave + 32 * mt + rr;
#pragma unroll
                for (int a0 = 0; a0 < 4; a0 += 2) {
                    uint32_t o[2][2];                     // [a - a0][dword]
#pragma unroll
                    for (int d = 0; d < 2; ++d)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int i = 4 * (a0 + d) + 2 * h;
                            float lo = c[i], hi = c[i + 1];
                            if constexpr (kBias) {
                                const uint32_t bb = bias2[a0 + d][h];
                                lo += bf16_to_f32(bb & 0xFFFFu);
                                hi += bf16_to_f32(bb >> 16);
                            }
                            o[d][h] = pk(lo, hi);
                        }
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const auto sw = __builtin_amdgcn_permlane32_swap(o[0][h], o[1][h], false,
                                                                         false);
                        o[0][h] = sw[0];
                        o[1][h] = sw[1];
                    }
                    const int64_t n = n0 + 32 * nt + 8 * (a0 + g);
                    if (m < p.M && n < p.N)
                        *reinterpret_cast<v4u *>(p.y + m * p.ldy + n) =
                            v4u{o[0][0], o[0][1], o[1][0], o[1][1]};
                }
            }
            // one tile at a time: reading every accumulator up front would
            // take more registers than the loop leaves
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (p.bias)
        epilogue(std::true_type{});
    else
        epilogue(std::false_type{});
}

template <int LAYOUT, int NTW>
static hipError_t launch_ntw(const GemmArgs &a, hipStream_t st) {
    constexpr int BN = NTW * 32;
    const int64_t tiles = ((a.N + BN - 1) / BN) * ((a.M + kBM - 1) / kBM);
    hipLaunchKernelGGL((gemm_w8a8_kernel<LAYOUT, NTW>), dim3((unsigned)tiles), dim3(256), 0, st,
                       a);
    return hipGetLastError();
}

int gemm_tile_n(int64_t N) {
    // 224-row tiles when they divide N evenly into a multiple of 8 bands
    // (7168 = 32 x 224: 512 tiles at M = 4096, two per CU); 256 otherwise
    if (N % 224 == 0 && (N / 224) % 8 == 0) return 224;
    return 256;
}

hipError_t launch_gemm(int layout, const GemmArgs &a, hipStream_t st) {
    const int bn = gemm_tile_n(a.N);
    if (layout == ROW32)
        return bn == 224 ? launch_ntw<ROW32, 7>(a, st) : launch_ntw<ROW32, 8>(a, st);
    return bn == 224 ? launch_ntw<BLK32, 7>(a, st) : launch_ntw<BLK32, 8>(a, st);
}

}  // namespace mx
