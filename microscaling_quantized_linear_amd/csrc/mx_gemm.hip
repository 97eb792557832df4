// mx_gemm.hip -- prefill MXFP8 GEMM (W8A8), y = x W^T at large M.
//
// ([rocm_native] module notes and apply_weights: fp8 e4m3 weights with E8M0
// block scales consumed directly by the CDNA4 microscaling matrix cores,
// activations quantized per token.)
//
// Workgroup tile: BN weight rows x 256 tokens, 4 wavefronts side by side
// along the tokens: each wavefront owns all BN rows and 64 tokens, NTW x 2
// output tiles of 32 x 32 accumulated by v_mfma_scale_f32_32x32x64_f8f6f4
// (A = weights, B = activations, both with per-lane E8M0 scales).  On
// MI355X the 32 x 32 x 64 form issues at its full rate (64 cycles for 2^17
// flop); the 16 x 16 x 128 form measured about 41 cycles for half as many.
//
// Operands, per 128-K step:
//  - weights (shared by the four wavefronts): the workgroup copies the
//    step's W-T16 chunks (2 KB per 16 rows) straight from memory into one of
//    four LDS buffers (buffer loads with an LDS destination), two steps ahead
//    of the matrix cores; one barrier per step.  A 32 x 32 x 64 operand lane
//    (row r, K group g) reads its two 16-byte pieces from those chunks.
//  - activations (private to a wavefront): read from the T16 layout straight
//    into registers at the top of the step before they are needed, two
//    register sets.  Keeping them out of LDS leaves the weights as LDS's only
//    traffic (about two thirds of it before), and no wavefront waits on LDS
//    for its activations after the barrier.
// Measured on MI355X, the first reader of a K slice often misses the XCD's
// L2 (each XCD works on some 20 MB of panels at once), so loads get more
// than a step of lead.
// Scale codes are read once per four steps as dwords whose byte u is step
// 4 q + u's code, picked by the MFMA's byte select.  Out-of-range rows, tokens
// and K tails read zeros through buffer-resource bounds.
#include "mx_device.h"
#include "mx_kernels.h"

#include <type_traits>

namespace mx {

constexpr int kBM = 256;           // tokens per workgroup

typedef __attribute__((address_space(3))) void lds_void;

// TAIL: K % 128 != 0, the last step's chunks are cut to their valid prefix
// (instantiated apart so the steady-state copies of whole-step shapes carry
// no extra mask).  REM: the step count S is not a multiple of eight, so the
// last iteration of the eight-step loop stops after step S - 1.
template <int LAYOUT, int NTW, bool TAIL, bool REM>
__global__ void __launch_bounds__(256, 1) gemm_w8a8_kernel(GemmArgs p) {
    constexpr int BN = NTW * 32;
    constexpr int kWBytes = 2 * NTW * 2048;               // one step's weight chunks
    // four distinct buffers: the compiler can then tell the copies into one
    // from the operand reads of another and waits only where it must
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kWBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kWBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[kWBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[kWBytes];
    static_assert(BN <= 256, "one bias value per thread");
    __shared__ __attribute__((aligned(16))) uint16_t bias_lds[BN];
    const int tid = threadIdx.x, lane = tid % 64;
    // bounded so the compiler can tell the two LDS buffers' accesses apart
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64) & 3;
    const int S = (int)((p.K + 127) / 128), Q = (S + 3) / 4;
    const int64_t T = p.N / 16, MB = (p.M + 15) / 16;

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
    const int64_t mbw = m0 / 16 + 4 * wave;               // this wavefront's first token tile

    // a weight tile is 16 K bytes: S - 1 whole chunks, then the last step's
    // valid prefix of tailb bytes (no padding stored)
    const int64_t TILEB = 16 * p.K;
    const uint32_t tailb = (uint32_t)(TILEB - (S - 1) * 2048);
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(p.w + t0 * TILEB, (uint32_t)((T - t0) * TILEB));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xq, (uint32_t)(MB * S * 2048));
    const __amdgpu_buffer_rsrc_t xcr = make_rsrc(p.xct, (uint32_t)act_codes_t16_bytes(p.M, p.K));
    const __amdgpu_buffer_rsrc_t cr =
        make_rsrc(p.codes, LAYOUT == ROW32 ? (uint32_t)(T * Q * 256)
                                           : (uint32_t)((p.N / 32) * Q * 16));

    // ---- weight copies: wavefront w copies chunk-halves w, w + 4, ... of
    // the step (NTW of them); chunk-half i = 2 c + h lands at i KB.  Offsets
    // of out-of-range loads get bit 31 set (every resource is below 2 GiB, so
    // those lanes read zeros); no branches in the loop body.
    // (wtail: the piece lies past the valid prefix of the last step's chunk)
    uint32_t wofs[NTW], wtail[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int idx = wave + 4 * i, c = idx / 2, h = idx % 2;
        const uint32_t o = (uint32_t)(1024 * h + 16 * lane);
        wofs[i] = t0 + c < T ? (uint32_t)(c * TILEB) + o : kOOB;
        wtail[i] = o >= tailb ? kOOB : 0u;
    }
    auto dma_one = [&](uint8_t *buf, int s, int i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (lds_void *)(buf + (wave + 4 * i) * 1024), 16,
            (int)((wofs[i] + (uint32_t)s * 2048u) | (s >= S ? kOOB : 0u) |
                  (TAIL && s == S - 1 ? wtail[i] : 0u)),
            0, 0, 0);
    };

    // ---- 32 x 32 x 64 operands: lane (g, rr) = lane / 32, lane % 32 holds
    // row (or token) rr with K 16 g .. and 32 + 16 g .. of a 64-K half-step
    // kh; in a 16-row chunk that is chunk rr / 16, bytes 1024 kh + 256 g +
    // 16 (rr % 16) and 512 further ----
    const int rr = lane % 32, g = lane / 32;
    const int off_lane = (rr / 16) * 2048 + 256 * g + 16 * (rr % 16);
    auto rd = [&](const uint8_t *base, int kh) -> v8i {
        const uint8_t *cp = base + off_lane + 1024 * kh;
        return cat8(*reinterpret_cast<const v4u *>(cp), *reinterpret_cast<const v4u *>(cp + 512));
    };

    // ---- activation fragments, straight from the T16 layout: token slab mt
    // (32 tokens) of this wavefront is token tiles mbw + 2 mt and + 1 ----
    // (every out-of-range case is folded in with bit 31, without branches:
    // a branch would split the step's basic block, and with it the order the
    // scheduling barriers keep)
    const uint32_t xlane = (uint32_t)((rr / 16) * S * 2048 + 256 * g + 16 * (rr % 16));
    uint32_t xtile[2];                                    // slab mt's first tile, or kOOB
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
        xtile[mt] = mbw + 2 * mt < MB ? (uint32_t)((mbw + 2 * mt) * S * 2048) : kOOB;
    typedef v8i BFrag[2][2];                              // [kh][mt]
    auto load_b_one = [&](BFrag &b, int s, int n) {       // load n of 8: (kh, mt, piece)
        const int kh = n / 4, mt = (n / 2) % 2, pc = n % 2;   // the first groups' half first
        const uint32_t u = (xtile[mt] + (uint32_t)s * 2048u) | (s >= S ? kOOB : 0u);
        const v4u v = load16(xr, (xlane + u + 1024u * kh + 512u * pc) | (u & kOOB));
        if (pc == 0) {
            b[kh][mt][0] = (int)v[0]; b[kh][mt][1] = (int)v[1];
            b[kh][mt][2] = (int)v[2]; b[kh][mt][3] = (int)v[3];
        } else {
            b[kh][mt][4] = (int)v[0]; b[kh][mt][5] = (int)v[1];
            b[kh][mt][6] = (int)v[2]; b[kh][mt][7] = (int)v[3];
        }
    };

    // ---- per-lane scale dwords of one quad of four steps: byte u of each
    // dword is step 4 q + u's code, picked by the MFMA's opsel; lane (g, rr)
    // of half-step kh needs block 2 kh + g of its row.  In the 16-row C-T16
    // code layout (weights with ROW32, and the activations) that is dword
    // 16 (2 kh + g) + rr % 16 of tile row / 16; BLK32 keeps one dword per
    // (32-row group, block). ----
    struct QScales {
        uint32_t w[NTW][2], x[2][2];
    };
    const uint32_t clane = (uint32_t)((rr / 16) * Q * 256 + 64 * g + 4 * (rr % 16));
    uint32_t xctile[2];                                   // slab mt's first code tile, or kOOB
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
        xctile[mt] = mbw + 2 * mt < MB ? (uint32_t)((mbw + 2 * mt) * Q * 256) : kOOB;
    auto load_qscales = [&](int q, QScales &out) {
        // rows past N and tokens past the last tile fall outside the
        // resources; quads past Q get bit 31
        const uint32_t past = q >= Q ? kOOB : 0u;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                uint32_t off;
                if (LAYOUT == ROW32)
                    off = clane + (uint32_t)(((n0 / 16 + 2 * nt) * Q + q) * 256 + 128 * kh);
                else
                    off = 4u * g + (uint32_t)(((n0 / 32 + nt) * Q + q) * 16 + 8 * kh);
                out.w[nt][kh] = load4(cr, off | past);
            }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const uint32_t u = xctile[mt] + (uint32_t)q * 256u + 128u * kh;
                out.x[mt][kh] = load4(xcr, (clane + u) | (u & kOOB) | past);
            }
    };

    typedef float v16f __attribute__((ext_vector_type(16)));
    // first written by the first step's MFMAs, which take a zero C operand
    v16f acc[NTW][2];

    // One barrier per step, two MFMA groups before its end: each wavefront
    // has waited for its own copies of step s + 1 (vmcnt), so after it every
    // wavefront may read step s + 1's buffer; and every wavefront is past
    // step s - 1, whose buffer is refilled (with step s + 3) only from step s
    // + 1 on.  LDS is ordered only through the copies' completion, so a plain
    // s_barrier suffices; the empty asm statements keep the compiler from
    // moving any memory access across it.  Placed inside the step, the
    // barrier waits while the previous group's MFMAs run, and the next step
    // starts with its first weight fragments already in registers.
    auto step_barrier = [] {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // One 128-K step, step u of its quad: the MFMAs of step s from `cur` and
    // the activation fragments `bc`, with the quad's scales `sc`.  Spread over
    // its 2 NTW MFMA groups (half-step kh, weight tile nt; two MFMAs each) go
    // out, about one per group, first the eight activation loads of step s +
    // 1 into `bn`, then the weight copies of step s + 2 into `ahead`: each
    // load is 1 KB, 16 clocks of the CU's address path, so four wavefronts'
    // loads bunched together would stall the MFMAs behind them.  Weight fragments are read two groups ahead, across
    // the step boundary into `next` (step s + 1's buffer), into a ring of
    // four: PH = the ring slot of the step's group 0 (NG = 14 or 16 groups a
    // step, eight steps an iteration, so the phase repeats).
    constexpr int kMem = NTW + 8;                         // memory ops per step
    constexpr int NG = 2 * NTW;                           // groups (kh, nt), kh major
    // the group that issues memory op e: activations 0..7 in groups 0..7,
    // the copies in the last NTW groups
    auto op_group = [](int e) { return e < 8 ? e : e - 8 + (NG - NTW); };
    static_assert(NG - NTW <= 8 && NTW >= 2, "schedule fits the step");
    static_assert((8 * NG) % 4 == 0, "ring phase repeats every iteration");
    v8i af[4];
    auto issue = [&](const uint8_t *buf, int k, int slot) {   // group k's weight fragment
        af[slot] = rd(buf + 2 * (k % NTW) * 2048, k / NTW);
    };
    auto step = [&](uint8_t *cur, uint8_t *next, uint8_t *ahead, int s, const QScales &sc,
                    BFrag &bc, BFrag &bn, auto uconst, auto firstconst, auto phconst) {
        constexpr int U = decltype(uconst)::value;
        constexpr bool kFirst = decltype(firstconst)::value;
        constexpr int PH = decltype(phconst)::value;
#pragma unroll
        for (int k = 0; k < NG; ++k) {
#pragma unroll
            for (int e = 0; e < kMem; ++e) {
                if (op_group(e) != k) continue;
                if (e < 8) load_b_one(bn, s + 1, e);
                else dma_one(ahead, s + 2, e - 8);
            }
            if (k == NG - 2) {
                // this wavefront's copies of step s + 1 (issued during step
                // s - 1, before all of this step's loads) have landed; of this
                // step's loads, those of groups 0 .. NG - 2 are out: all but
                // the last copy
                static_assert(op_group(kMem - 2) <= NG - 2 && op_group(kMem - 1) == NG - 1,
                              "kMem - 1 loads before the barrier");
                __builtin_amdgcn_s_waitcnt(vmcnt_only(kMem - 1));
                step_barrier();
            }
            if (k + 2 < NG) issue(cur, k + 2, (PH + k + 2) % 4);
            else issue(next, k + 2 - NG, (PH + k + 2) % 4);
            __builtin_amdgcn_sched_barrier(0);
            const int kh = k / NTW, nt = k % NTW;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                acc[nt][mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af[(PH + k) % 4], bc[kh][mt], kFirst && kh == 0 ? v16f{} : acc[nt][mt], 0,
                    0, U, (int)sc.w[nt][kh], U, (int)sc.x[mt][kh]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using U0 = std::integral_constant<int, 0>;
    using U1 = std::integral_constant<int, 1>;
    using U2 = std::integral_constant<int, 2>;
    using U3 = std::integral_constant<int, 3>;
    using F0 = std::false_type;
    using P0 = std::integral_constant<int, 0>;
    using P2 = std::integral_constant<int, (NG % 4)>;    // the odd steps' phase

    // the workgroup's BN bias values, staged in LDS under the first barrier
    // (the bias needs only 2-byte alignment: one element per thread)
    if (p.bias && tid < BN) bias_lds[tid] = n0 + tid < p.N ? p.bias[n0 + tid] : 0;

    QScales qa, qb;
    BFrag ba, bb;
#pragma unroll
    for (int i = 0; i < NTW; ++i) dma_one(lds0, 0, i);
#pragma unroll
    for (int n = 0; n < 8; ++n) load_b_one(ba, 0, n);
    load_qscales(0, qa);
#pragma unroll
    for (int i = 0; i < NTW; ++i) dma_one(lds1, 1, i);
    // step 0's copies, activations and scales have landed; step 1's copies
    // are checked at step 0's barrier
    __builtin_amdgcn_s_waitcnt(vmcnt_only(NTW));
    __syncthreads();
    issue(lds0, 0, 0);
    issue(lds0, 1, 1);
    // eight steps (two quads) per iteration: each LDS buffer and activation
    // register set is a fixed object and the two scale sets alternate without
    // copies
    const int S8 = REM ? S / 8 * 8 : S;
    for (int s = 0; s < S8; s += 8) {
        const int q = s / 4;
        load_qscales(q + 1, qb);
        if (s == 0)
            step(lds0, lds1, lds2, s + 0, qa, ba, bb, U0{}, std::true_type{}, P0{});
        else
            step(lds0, lds1, lds2, s + 0, qa, ba, bb, U0{}, F0{}, P0{});
        step(lds1, lds2, lds3, s + 1, qa, bb, ba, U1{}, F0{}, P2{});
        step(lds2, lds3, lds0, s + 2, qa, ba, bb, U2{}, F0{}, P0{});
        step(lds3, lds0, lds1, s + 3, qa, bb, ba, U3{}, F0{}, P2{});
        load_qscales(q + 2, qa);
        step(lds0, lds1, lds2, s + 4, qb, ba, bb, U0{}, F0{}, P0{});
        step(lds1, lds2, lds3, s + 5, qb, bb, ba, U1{}, F0{}, P2{});
        step(lds2, lds3, lds0, s + 6, qb, ba, bb, U2{}, F0{}, P0{});
        step(lds3, lds0, lds1, s + 7, qb, bb, ba, U3{}, F0{}, P2{});
    }
    // REM: the last S % 8 steps, the leading steps of one more iteration in
    // nested uniform conditions (every wavefront takes the same ones, with
    // their barriers; loads issued for the steps not taken read zeros).
    // With S < 8 the loop did not run and the accumulators start at zero.
    if (REM && S8 < S) {
        const int s = S8, q = s / 4;
        if (s == 0) {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) acc[nt][mt] = v16f{};
        }
        load_qscales(q + 1, qb);
        step(lds0, lds1, lds2, s + 0, qa, ba, bb, U0{}, F0{}, P0{});
        if (s + 1 < S) {
            step(lds1, lds2, lds3, s + 1, qa, bb, ba, U1{}, F0{}, P2{});
            if (s + 2 < S) {
                step(lds2, lds3, lds0, s + 2, qa, ba, bb, U2{}, F0{}, P0{});
                if (s + 3 < S) {
                    step(lds3, lds0, lds1, s + 3, qa, bb, ba, U3{}, F0{}, P2{});
                    if (s + 4 < S) {
                        step(lds0, lds1, lds2, s + 4, qb, ba, bb, U0{}, F0{}, P0{});
                        if (s + 5 < S) {
                            step(lds1, lds2, lds3, s + 5, qb, bb, ba, U1{}, F0{}, P2{});
                            if (s + 6 < S)
                                step(lds2, lds3, lds0, s + 6, qb, ba, bb, U2{}, F0{}, P0{});
                        }
                    }
                }
            }
        }
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
    // Stores go through a buffer resource over y with 32-bit offsets worked
    // out once per lane; an output past M or N gets an out-of-range offset and
    // is dropped, so there is no branch and no 64-bit address per store (a
    // branch per store also made the compiler reload the kernel arguments
    // around each one).  The host keeps M * ldy * 2 below 2^31.
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(p.y, (uint32_t)(p.M * p.ldy * 2));
    const uint32_t ldy2 = (uint32_t)p.ldy * 2u;
    uint32_t ybase[2];                                    // token row of slab mt, or kOOB
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int64_t m = m0 + 64 * wave + 32 * mt + rr;
        ybase[mt] = m < p.M ? (uint32_t)m * ldy2 + (uint32_t)(n0 + 8 * g) * 2u : kOOB;
    }
    const int64_t nlim = p.N - n0 - 8 * g;                // columns left for this lane's pieces
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
                    // columns n0 + 32 nt + 8 (a0 + g) .. + 7 (N % 16 == 0: all in or out)
                    const uint32_t col = 32u * nt + 8u * a0;
                    const uint32_t off = (int64_t)col < nlim ? ybase[mt] + 2u * col : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b128(
                        v4u{o[0][0], o[0][1], o[1][0], o[1][1]}, yr, (int)(off | (off & kOOB)),
                        0, 0);
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
    const dim3 grid((unsigned)tiles), block(256);
    const bool tail = a.K % 128 != 0, rem = (a.K + 127) / 128 % 8 != 0;
    if (tail)
        hipLaunchKernelGGL((gemm_w8a8_kernel<LAYOUT, NTW, true, true>), grid, block, 0, st, a);
    else if (rem)
        hipLaunchKernelGGL((gemm_w8a8_kernel<LAYOUT, NTW, false, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((gemm_w8a8_kernel<LAYOUT, NTW, false, false>), grid, block, 0, st, a);
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
