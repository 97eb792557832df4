// mx_gemm.hip -- prefill MXFP8 GEMM (W8A8), y = x W^T at large M.
//
// ([rocm_native] module notes and apply_weights: fp8 e4m3 weights with E8M0
// block scales consumed directly by the CDNA4 microscaling matrix cores,
// activations quantized per token with row-major codes.)
//
// Workgroup tile: BN weight rows x 256 tokens, 4 wavefronts as 2 x 2, each
// wavefront NTW x 8 tiles of 16 x 16 accumulated by
// v_mfma_scale_f32_16x16x128_f8f6f4 (A = weights, B = activations, both
// with per-lane E8M0 scales).  Per 128-K step the workgroup copies its
// weight chunks (W-T16: each 2 KB chunk is already one operand in lane
// order) and its activation rows (already in fragment order when they come
// in the T16 layout, else rearranged into it by the copy's addressing)
// straight from memory into one of two LDS
// buffers (buffer loads with an LDS destination) while the matrix cores
// work on the other; one barrier per step.  Scale codes are read once per
// four steps as one dword per lane (byte u = step 4q + u) and the MFMA's
// byte select picks the step's code.  Out-of-range rows and K tails read
// zeros through buffer-resource bounds.
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
    constexpr int BN = 2 * NTW * 16;
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int r = lane % 16, j = lane / 16;
    const int wn = wave % 2, wm = wave / 2;
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
        const int i = wave + 4 * q, mc = i / 2, h = i % 2;
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
    auto dma = [&](uint8_t *buf, int64_t s) {
        const uint32_t su = (uint32_t)s, past = su >= (uint32_t)S ? kOOB : 0u;
#pragma unroll
        for (int q = 0; q < kWq; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (lds_void *)(buf + (wave + 4 * q) * 1024), 16,
                (int)((wbase[q] + su * 2048u) | past), 0, 0, 0);
#pragma unroll
        for (int q = 0; q < kXq; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (lds_void *)(buf + SM::kWBytes + (wave + 4 * q) * 1024), 16,
                (int)((xbase[q] + su * xstep) | (su >= xkmax[q] ? kOOB : 0u)), 0, 0, 0);
    };

    // ---- per-lane scale dwords of one quad of four steps: byte u of each
    // dword is step 4 q + u's code, picked by the MFMA's opsel ----
    struct QScales {
        uint32_t w[NTW], x[8];
    };
    uint32_t cwbase[NTW], cxbase[8];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int64_t t = t0 + wn * NTW + nt;
        if (LAYOUT == ROW32)
            cwbase[nt] = t < T ? (uint32_t)(t * Q * 256 + 4 * lane) : kOOB;
        else
            cwbase[nt] = t < T ? (uint32_t)(((16 * t) / 32) * Q * 16 + 4 * j) : kOOB;
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
        const int64_t row0 = m0 + wm * 128 + 16 * mt;     // XC-T16 tile of 16 rows
        cxbase[mt] = row0 < p.M ? (uint32_t)((row0 / 16) * Q * 256 + 4 * lane) : kOOB;
    }
    auto load_qscales = [&](int64_t q, QScales &out) {
        const uint32_t qu = (uint32_t)q, past = qu >= (uint32_t)Q ? kOOB : 0u;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
            out.w[nt] = load4(cr, (cwbase[nt] + qu * (LAYOUT == ROW32 ? 256u : 16u)) | past);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) out.x[mt] = load4(xcr, (cxbase[mt] + qu * 256u) | past);
    };

    v4f acc[NTW][8];
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    // one 128-K step, step u of its quad: DMA of step s + 1 into `nxt`, then
    // the MFMAs of step s from `cur` with the quad's scales `sc`
    auto step = [&](uint8_t *cur, uint8_t *nxt, int64_t s, const QScales &sc, auto uconst) {
        constexpr int U = decltype(uconst)::value;
        dma(nxt, s + 1);
        __builtin_amdgcn_sched_barrier(0);
        // the activation fragments and the first weight fragment are read
        // first; each later weight fragment is read one group of MFMAs ahead
        // of its use, so LDS latency overlaps the matrix cores
        v8i af[2], bf[8];
        auto read_a = [&](int nt, v8i &dst) {
            const uint8_t *cp = cur + (wn * NTW + nt) * 2048;
            dst = cat8(*reinterpret_cast<const v4u *>(cp + 16 * lane),
                       *reinterpret_cast<const v4u *>(cp + 1024 + 16 * lane));
        };
        read_a(0, af[0]);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const uint8_t *cp = cur + SM::kWBytes + (wm * 8 + mt) * 2048;
            bf[mt] = cat8(*reinterpret_cast<const v4u *>(cp + 16 * lane),
                          *reinterpret_cast<const v4u *>(cp + 1024 + 16 * lane));
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            if (nt + 1 < NTW) read_a(nt + 1, af[(nt + 1) % 2]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                acc[nt][mt] = mfma_fp8_scaled_sel<U>(af[nt % 2], bf[mt], acc[nt][mt],
                                                     (int)sc.w[nt], (int)sc.x[mt]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };
    using U0 = std::integral_constant<int, 0>;
    using U1 = std::integral_constant<int, 1>;
    using U2 = std::integral_constant<int, 2>;
    using U3 = std::integral_constant<int, 3>;

    QScales qa, qb;
    dma(lds0, 0);
    load_qscales(0, qa);
    __syncthreads();
    // eight steps (two quads) per iteration: each LDS buffer is a fixed object
    // and the two scale sets alternate without copies; a step at or past S
    // reads zeros and adds nothing
    for (int64_t s = 0; s < S; s += 8) {
        const int64_t q = s / 4;
        load_qscales(q + 1, qb);
        step(lds0, lds1, s + 0, qa, U0{});
        step(lds1, lds0, s + 1, qa, U1{});
        step(lds0, lds1, s + 2, qa, U2{});
        step(lds1, lds0, s + 3, qa, U3{});
        load_qscales(q + 2, qa);
        step(lds0, lds1, s + 4, qb, U0{});
        step(lds1, lds0, s + 5, qb, U1{});
        step(lds0, lds1, s + 6, qb, U2{});
        step(lds1, lds0, s + 7, qb, U3{});
    }

    // ---- epilogue: lane (r, j) of tile (nt, mt) holds n = 4 j .. 4 j + 3, m = r ----
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
        const int64_t n = n0 + (wn * NTW + nt) * 16 + 4 * j;
        if (n >= p.N) continue;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.bias)
            for (int i = 0; i < 4; ++i) bv[i] = bf16_to_f32(p.bias[n + i]);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const int64_t m = m0 + wm * 128 + 16 * mt + r;
            if (m >= p.M) continue;
            const v4f a = acc[nt][mt];
            v2u o = {bf16_bits(a[0] + bv[0]) | (bf16_bits(a[1] + bv[1]) << 16),
                     bf16_bits(a[2] + bv[2]) | (bf16_bits(a[3] + bv[3]) << 16)};
            *reinterpret_cast<v2u *>(p.y + m * p.ldy + n) = o;
        }
    }
}

template <int LAYOUT, int NTW>
static hipError_t launch_ntw(const GemmArgs &a, hipStream_t st) {
    constexpr int BN = 2 * NTW * 16;
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
