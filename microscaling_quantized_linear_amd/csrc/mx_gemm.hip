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
// order) and its activation rows (row-major, padded to a 144-byte pitch so
// the operand reads are bank-conflict free) into one of two LDS buffers
// while the matrix cores work on the other; one barrier per step.
// Loads of the next step are issued before the current step's MFMAs.
// Out-of-range rows and K tails read zeros through buffer-resource bounds.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

constexpr int kBM = 256;           // tokens per workgroup
constexpr int kXPitch = 144;       // LDS bytes per activation row (128 + 16)

template <int NTW>
struct GemmSmem {
    static constexpr int kWBytes = 2 * NTW * 2048;        // weight chunks per step
    static constexpr int kXBytes = kBM * kXPitch;
    static constexpr int kBuf = kWBytes + kXBytes;
    static constexpr int kTotal = 2 * kBuf;
};

template <int LAYOUT, int NTW>
__global__ void __launch_bounds__(256, 1) gemm_w8a8_kernel(GemmArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using SM = GemmSmem<NTW>;
    constexpr int BN = 2 * NTW * 16;
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int r = lane % 16, j = lane / 16;
    const int wn = wave % 2, wm = wave / 2;
    const int64_t Kp = (p.K + 127) / 128 * 128, S = Kp / 128, T = p.N / 16, Q = (S + 3) / 4;
    const int64_t KB = p.K / 32;

    // tile order: consecutive workgroups go to different XCDs; give each XCD
    // a band of N tiles so the weight panels it streams stay in its L2
    const int64_t tiles_n = (p.N + BN - 1) / BN, tiles_m = (p.M + kBM - 1) / kBM;
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
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xq, (uint32_t)(p.M * p.ldq));
    const __amdgpu_buffer_rsrc_t xcr = make_rsrc(p.xcodes, (uint32_t)(p.M * p.ldc));
    const __amdgpu_buffer_rsrc_t cr =
        make_rsrc(p.codes, LAYOUT == ROW32 ? (uint32_t)(T * Q * 256)
                                           : (uint32_t)((p.N / 32) * (Kp / 32)));

    // ---- global -> register staging for one step ----
    v4u wst[NTW], xst[8];
    auto issue_loads = [&](int64_t s) {
#pragma unroll
        for (int q = 0; q < NTW; ++q) {
            const int64_t c = 2 * q + tid / 128;           // chunk within the tile column
            const int64_t t = t0 + c;
            const uint32_t off = t < T ? (uint32_t)((t * S + s) * 2048 + 16 * (tid % 128)) : kOOB;
            wst[q] = load16<kNT>(wr, off);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int64_t row = m0 + 32 * q + tid / 8;
            const int64_t k = 128 * s + 16 * (tid % 8);
            const uint32_t off = (row < p.M && k < p.K) ? (uint32_t)(row * p.ldq + k) : kOOB;
            xst[q] = load16(xr, off);
        }
    };
    auto store_lds = [&](int buf) {
        uint8_t *wb = smem + buf * SM::kBuf;
        uint8_t *xb = wb + SM::kWBytes;
#pragma unroll
        for (int q = 0; q < NTW; ++q)
            *reinterpret_cast<v4u *>(wb + q * 4096 + 16 * tid) = wst[q];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            *reinterpret_cast<v4u *>(xb + (32 * q + tid / 8) * kXPitch + 16 * (tid % 8)) = xst[q];
    };
    // ---- per-lane scales of one step ----
    uint32_t sw[NTW], sx[8];
    auto load_scales = [&](int64_t s, uint32_t *w_out, uint32_t *x_out) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const int64_t t = t0 + wn * NTW + nt;
            if (LAYOUT == ROW32) {
                const uint32_t off = t < T ? (uint32_t)((t * Q + s / 4) * 256 + 4 * lane) : kOOB;
                w_out[nt] = byte_of(load4(cr, off), (uint32_t)(s % 4));
            } else {
                const uint32_t off = t < T ? (uint32_t)(((16 * t) / 32) * (Kp / 32) + 4 * s) : kOOB;
                w_out[nt] = byte_of(load4(cr, off), (uint32_t)j);
            }
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const int64_t row = m0 + wm * 128 + 16 * mt + r;
            const int64_t blk = 4 * s + j;
            x_out[mt] = load1(xcr, (row < p.M && blk < KB) ? (uint32_t)(row * p.ldc + blk) : kOOB);
        }
    };

    v4f acc[NTW][8];
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    issue_loads(0);
    load_scales(0, sw, sx);
    store_lds(0);
    __syncthreads();

    for (int64_t s = 0; s < S; ++s) {
        const int cur = (int)(s & 1);
        uint32_t swn[NTW], sxn[8];
        const bool more = s + 1 < S;
        if (more) {
            issue_loads(s + 1);
            load_scales(s + 1, swn, sxn);
        }
        const uint8_t *wb = smem + cur * SM::kBuf;
        const uint8_t *xb = wb + SM::kWBytes;
        v8i bf[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const uint8_t *rowp = xb + (wm * 128 + 16 * mt + r) * kXPitch;
            bf[mt] = cat8(*reinterpret_cast<const v4u *>(rowp + 16 * j),
                          *reinterpret_cast<const v4u *>(rowp + 64 + 16 * j));
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const uint8_t *cp = wb + (wn * NTW + nt) * 2048;
            const v8i af = cat8(*reinterpret_cast<const v4u *>(cp + 16 * lane),
                                *reinterpret_cast<const v4u *>(cp + 1024 + 16 * lane));
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                acc[nt][mt] = mfma_fp8_scaled(af, bf[mt], acc[nt][mt], (int)sw[nt], (int)sx[mt]);
        }
        if (more) {
            store_lds(cur ^ 1);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) sw[nt] = swn[nt];
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) sx[mt] = sxn[mt];
        }
        __syncthreads();
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
    const int smem = GemmSmem<NTW>::kTotal;
    // the LDS-size attribute is set once per device (outside any graph capture
    // that follows the first call)
    static bool attr_done[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !attr_done[dev]) {
        e = hipFuncSetAttribute((const void *)gemm_w8a8_kernel<LAYOUT, NTW>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) attr_done[dev] = true;
    }
    hipLaunchKernelGGL((gemm_w8a8_kernel<LAYOUT, NTW>), dim3((unsigned)tiles), dim3(256), smem, st,
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
