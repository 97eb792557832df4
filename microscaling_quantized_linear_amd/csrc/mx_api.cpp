// mx_api.cpp -- the C ABI of libmx (include/mx.h): host-side validation,
// the gfx950 gate, workspace sizing and dispatch to the kernels.
//
// Validation is pure host code and runs before any device call, so every
// error path can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/mx.h"
#include "mx_kernels.h"

namespace {

using mx::ACT_BF16;
using mx::ACT_MXFP8;
using mx::ACT_MXFP8_T16;
using mx::BLK32;
using mx::E2M1;
using mx::E4M3;
using mx::ROW32;

constexpr int64_t kMaxRsrc = (int64_t(1) << 31) - 1;   // 32-bit buffer offsets

// largest M served by the decode GEMV for W8A8; above it the GEMM runs
constexpr int64_t kGemvMaxM = 64;

// Batch-invariant mode: every W8A8 M runs on the decode GEMV, whose order of
// summation for an output depends on K alone, so a row's result does not
// depend on how many rows share the call (the GEMM above kGemvMaxM sums in
// another order).  Process-wide; MX_BATCH_INVARIANT=1 sets it at start-up and
// mx_set_batch_invariant changes it.
std::atomic<int> g_invariant{-1};
bool batch_invariant() {
    int v = g_invariant.load(std::memory_order_relaxed);
    if (v < 0) {
        const char *s = std::getenv("MX_BATCH_INVARIANT");
        int unset = -1;
        g_invariant.compare_exchange_strong(unset, s && s[0] && s[0] != '0' ? 1 : 0);
        v = g_invariant.load(std::memory_order_relaxed);
    }
    return v == 1;
}
// the W8A8 prefill GEMM serves this call (else a GEMV)
bool use_gemm(int act, int64_t M) {
    return act != ACT_BF16 && M > kGemvMaxM && !batch_invariant();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

// the W8A8 GEMV's launch plan (fails for more than 64 steps of K per wavefront)
int env_int(const char *name) {
    const char *s = std::getenv(name);
    return s ? std::atoi(s) : 0;
}

// MX_W8_WAVES and MX_W8_TILES override the plan (tuning sweeps only; read once)
mx::GemvW8Plan gemv_w8_plan(int64_t N, int64_t K, int64_t M) {
    static const int f_nw = env_int("MX_W8_WAVES"), f_g = env_int("MX_W8_TILES");
    return mx::plan_gemv_w8(N / 16, (K + 127) / 128, (M + 15) / 16, f_nw, f_g);
}
int64_t padded_k(int64_t K) { return (K + 127) / 128 * 128; }

// In-call quantization inside the decode GEMV (one launch, no workspace):
// W8A8 with M <= 64 whose shape the GEMV plan divides evenly and K % 128 == 0.
// MX_FUSED_QUANT=0 switches it off (then a quantization launch into the
// workspace precedes the GEMV); read once.
bool fused_quant_ok(int elem, int64_t N, int64_t K, int64_t M) {
    static const bool enabled = [] {
        const char *s = std::getenv("MX_FUSED_QUANT");
        return !(s && s[0] == '0');
    }();
    return enabled && elem == E4M3 && M <= kGemvMaxM && K % 128 == 0 &&
           mx::gemv_w8_even(N, K, gemv_w8_plan(N, K, M));
}

mx_status shape_ok(int elem, int layout, int64_t E, int64_t N, int64_t K) {
    if (elem != E4M3 && elem != E2M1) return MX_ERR_UNSUPPORTED;
    if (layout != ROW32 && layout != BLK32) return MX_ERR_UNSUPPORTED;
    if (E < 1 || N < 16 || K < 32 || K % 32 != 0 || N % 16 != 0) return MX_ERR_SHAPE;
    if (layout == BLK32 && N % 32 != 0) return MX_ERR_SHAPE;
    return MX_OK;
}

// one entry per device ordinal: 0 not yet known (the zero-initialized
// state, valid before any constructor runs), 1 not gfx950, 2 gfx950
std::atomic<int> g_arch[64];

mx_status device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MX_ERR_DEVICE;
    if (dev < 64) {
        const int v = g_arch[dev].load();
        if (v != 0) return v == 2 ? MX_OK : MX_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MX_ERR_DEVICE;
    const int ok = mx_arch_supported(prop.gcnArchName);
    if (dev < 64) g_arch[dev].store(ok ? 2 : 1);
    return ok ? MX_OK : MX_ERR_DEVICE;
}

mx_status launched(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_LAUNCH; }

// Dispatch trace: with MX_LOG=1 in the environment (read once per process)
// every launch decision of the hot path goes to stderr as one line: entry
// point, kernel and its launch plan, and the shape.  Off by default; no
// output and no cost beyond one branch otherwise.
bool log_on() {
    static const bool on = [] {
        const char *s = std::getenv("MX_LOG");
        return s && s[0] && s[0] != '0';
    }();
    return on;
}
__attribute__((format(printf, 1, 2))) void log_dispatch(const char *fmt, ...) {
    if (!log_on()) return;
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    std::fprintf(stderr, "mx: %s\n", buf);
}
const char *layout_name(int layout) { return layout == ROW32 ? "ROW32" : "BLK32"; }
const char *elem_name(int elem) { return elem == E4M3 ? "E4M3" : "E2M1"; }

int env_choice(const char *name) {
    const char *s = std::getenv(name);
    const int v = s ? std::atoi(s) : 0;
    return (v == 1 || v == 2 || v == 4 || v == 8) ? v : 0;
}

// Launch shape of the GEMV (see mx_kernels.h).  MX_GEMV_WAVES, MX_GEMV_CHUNK
// and MX_GEMV_TILES override it (tuning sweeps only; read once).
// Defaults measured on MI355X with graph-replayed launches: long K (S >= 32
// steps, e.g. 7168) 8 waves x chunks of 4 steps x 2 tiles; 16 <= S < 32 4
// waves x 4 steps x 1 tile; 8 <= S < 16 2 waves x 8 steps (every step of a
// wavefront in one chunk: M = 8, N = 4096, K = 1568 3.93 against 4.04 us
// with 4 waves x 4 steps); S < 8 2 waves x 2 steps (M = 1, N = 256, K = 512:
// 2.52 against 2.65 us with chunks of 4); grouped MoE 2 steps x 4 tiles of
// an expert, 4 waves from 16 steps (K >= 2048), else 2 (K = 1536 down
// projection: 17.7 vs 21.0 us).
mx::GemvShape gemv_shape(int64_t S, bool moe) {
    static const int f_nw = env_choice("MX_GEMV_WAVES"), f_chunk = env_choice("MX_GEMV_CHUNK"),
                     f_tiles = env_choice("MX_GEMV_TILES");
    mx::GemvShape g;
    if (moe)
        g = {S >= 16 ? 4 : S >= 2 ? 2 : 1, 2, 4};
    else if (S >= 32)
        g = {8, 4, 2};
    else if (S >= 16)
        g = {4, 4, 1};
    else if (S >= 8)
        g = {2, 8, 1};
    else
        g = {S >= 2 ? 2 : 1, 2, 1};
    if (f_nw) g.nw = f_nw;
    if (f_chunk) g.chunk = f_chunk < 2 ? 2 : f_chunk;
    if (f_tiles) g.tiles = f_tiles > 4 ? 4 : f_tiles;
    return g;
}

// The grouped MoE GEMV behind mx_moe_linear, mx_moe_gate_up and mx_moe_down:
// xslot reads activation row i for pair i (else its token's row), epi writes
// silu(row 2 i) * row 2 i + 1 as output i (width N / 2, per slot only).
mx_status moe_run(int elem, int64_t E, int64_t N, int64_t K, const void *w_packed,
                  const void *codes_packed, int64_t T, int64_t topk, const void *x, int64_t ldx,
                  bool xslot, bool epi, const int32_t *topk_ids, const float *topk_weights,
                  void *y, int64_t ldy, void *ws, size_t ws_bytes, mx_stream_t stream) {
    size_t need = 0;
    mx_status st = mx_moe_workspace(elem, E, N, K, T, topk, topk_weights ? 1 : 0, &need);
    if (st != MX_OK) return st;
    const int64_t xrows = xslot ? T * topk : T;
    if (ldx < K) return MX_ERR_SHAPE;
    if (xrows * ldx * 2 > kMaxRsrc) return MX_ERR_SHAPE;
    if (!w_packed || !codes_packed || !x || !topk_ids || !y) return MX_ERR_NULL;
    if (!aligned16(w_packed) || !aligned16(codes_packed) || !aligned16(x) || !aligned16(y) ||
        ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(topk_ids) & 3u) ||
        (topk_weights && (reinterpret_cast<uintptr_t>(topk_weights) & 3u)))
        return MX_ERR_ALIGN;
    if (need > 0 && (!ws || ws_bytes < need)) return MX_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return MX_ERR_ALIGN;
    if ((st = device_ok()) != MX_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int64_t Kp = padded_k(K);
    mx::GemvArgs a{};
    a.w = static_cast<const uint8_t *>(w_packed);
    a.codes = static_cast<const uint8_t *>(codes_packed);
    a.E = E;
    a.N = N;
    a.K = K;
    a.rows = T;
    a.topk = topk;
    a.xrows = xrows;
    a.x = x;
    a.ldx = ldx;
    a.ids = topk_ids;
    a.y = static_cast<uint16_t *>(y);
    a.ldy = ldy;
    a.xslot = xslot ? 1 : 0;
    a.epi = epi ? 1 : 0;
    float *slots = topk_weights ? static_cast<float *>(ws) : nullptr;
    a.ws = slots;
    const mx::GemvShape sh = gemv_shape(Kp / 128, true);
    log_dispatch("moe %s%s%s: gemv_kernel A16%s grouped, %d waves x %d-step chunks x %d tiles; "
                 "E=%lld N=%lld K=%lld T=%lld topk=%lld",
                 xslot ? "xslot " : "", epi ? "silu " : "", topk_weights ? "combined" : "per-slot",
                 elem == E4M3 ? "W8" : "W4", sh.nw, sh.chunk, sh.tiles, (long long)E,
                 (long long)N, (long long)K, (long long)T, (long long)topk);
    if ((st = launched(mx::launch_gemv(elem, ROW32, ACT_BF16, true, a, sh, s))) != MX_OK)
        return st;
    if (topk_weights) {
        log_dispatch("moe: moe_combine_kernel T=%lld topk=%lld N=%lld", (long long)T,
                     (long long)topk, (long long)N);
        return launched(mx::launch_moe_combine(T, topk, N, slots, topk_weights, y, s));
    }
    return MX_OK;
}

// Load-time checks end with a device flag read back: clear it, run the check,
// copy it to the host and wait for the stream.
template <class F>
mx_status flagged(void *ws, hipStream_t s, F launch) {
    int *bad = static_cast<int *>(ws);
    if (hipMemsetAsync(bad, 0, sizeof(int), s) != hipSuccess) return MX_ERR_LAUNCH;
    mx_status st = launched(launch(bad));
    if (st != MX_OK) return st;
    int h = 0;
    if (hipMemcpyAsync(&h, bad, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return MX_ERR_LAUNCH;
    return h ? MX_ERR_VALUE : MX_OK;
}
}  // namespace

extern "C" {

const char *mx_status_str(mx_status s) {
    switch (s) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "a required pointer is NULL";
    case MX_ERR_SHAPE: return "a size or leading dimension breaks the layout rules";
    case MX_ERR_ALIGN: return "a pointer or leading dimension is misaligned";
    case MX_ERR_VALUE: return "an E8M0 weight code is 255 (NaN)";
    case MX_ERR_UNSUPPORTED: return "format / layout / activation combination not built";
    case MX_ERR_DEVICE: return "the current device is not gfx950";
    case MX_ERR_WORKSPACE: return "workspace missing or too small";
    case MX_ERR_LAUNCH: return "a HIP call or kernel launch failed";
    }
    return "unknown status";
}

int mx_set_batch_invariant(int on) {
    const int prev = batch_invariant() ? 1 : 0;
    g_invariant.store(on ? 1 : 0, std::memory_order_relaxed);
    return prev;
}

int mx_arch_supported(const char *name) {
    if (!name) return 0;
    return std::strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':');
}

mx_status mx_packed_sizes(int elem, int layout, int64_t E, int64_t N, int64_t K,
                          size_t *w_bytes, size_t *code_bytes) {
    if (!w_bytes || !code_bytes) return MX_ERR_NULL;
    mx_status st = shape_ok(elem, layout, E, N, K);
    if (st != MX_OK) return st;
    const int64_t Kp = padded_k(K), S = Kp / 128, Q = (S + 3) / 4;
    *w_bytes = (size_t)(E * N * (elem == E4M3 ? K : K / 2));   // no stored padding
    *code_bytes = (size_t)(mx::packed_code_body_bytes(layout, E, N, K) + mx::kCodeTrailer);
    (void)Q;
    return MX_OK;
}

mx_status mx_pack_weights(int elem, int layout, int64_t E, int64_t N, int64_t K, const void *w,
                          const void *codes, void *w_packed, void *codes_packed, void *ws,
                          size_t ws_bytes, mx_stream_t stream) {
    size_t wb, cb;
    mx_status st = mx_packed_sizes(elem, layout, E, N, K, &wb, &cb);
    if (st != MX_OK) return st;
    if (!w || !codes || !w_packed || !codes_packed || !ws) return MX_ERR_NULL;
    if (!aligned16(w) || !aligned16(codes) || !aligned16(w_packed) || !aligned16(codes_packed) ||
        !aligned16(ws))
        return MX_ERR_ALIGN;
    if (ws_bytes < 256) return MX_ERR_WORKSPACE;
    if ((st = device_ok()) != MX_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // ws: the code-255 flag, then the code range's two counters (255, 0)
    int *bad = static_cast<int *>(ws);
    unsigned *range = reinterpret_cast<unsigned *>(static_cast<uint8_t *>(ws) + 4);
    if (hipMemsetAsync(bad, 0, 12, s) != hipSuccess ||
        hipMemsetAsync(range, 0xFF, 1, s) != hipSuccess)
        return MX_ERR_LAUNCH;
    if ((st = launched(mx::launch_pack(elem, layout, E, N, K, w, codes, w_packed, codes_packed,
                                       bad, range, s))) != MX_OK)
        return st;
    int h[3] = {0, 0, 0};
    if (hipMemcpyAsync(h, bad, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return MX_ERR_LAUNCH;
    if (h[0]) return MX_ERR_VALUE;
    // the trailer after the packed codes: smallest and largest given code
    uint8_t trailer[mx::kCodeTrailer] = {};
    trailer[0] = (uint8_t)h[1];
    trailer[1] = (uint8_t)h[2];
    uint8_t *tail = static_cast<uint8_t *>(codes_packed) + (cb - mx::kCodeTrailer);
    if (hipMemcpyAsync(tail, trailer, sizeof(trailer), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return MX_ERR_LAUNCH;
    return MX_OK;
}

mx_status mx_quant_act(int64_t M, int64_t K, const void *x, int64_t ldx, void *xq, int64_t ldq,
                       void *xcodes, int64_t ldc, int rule, mx_stream_t stream) {
    if (rule != mx::RULE_OCP && rule != mx::RULE_CEIL448) return MX_ERR_UNSUPPORTED;
    if (M < 1 || K < 32 || K % 32 != 0 || ldx < K || ldq < K || ldc < K / 32) return MX_ERR_SHAPE;
    if (!x || !xq || !xcodes) return MX_ERR_NULL;
    if (!aligned16(x) || !aligned16(xq) || ldx % 8 != 0 || ldq % 16 != 0) return MX_ERR_ALIGN;
    mx_status st = device_ok();
    if (st != MX_OK) return st;
    return launched(mx::launch_quant(M, K, x, ldx, xq, ldq, xcodes, ldc, rule,
                                     reinterpret_cast<hipStream_t>(stream)));
}

mx_status mx_act_t16_sizes(int64_t M, int64_t K, size_t *xq_bytes, size_t *xcodes_bytes) {
    if (!xq_bytes || !xcodes_bytes) return MX_ERR_NULL;
    if (M < 1 || K < 32 || K % 32 != 0) return MX_ERR_SHAPE;
    *xq_bytes = (size_t)mx::act_t16_data_bytes(M, K);
    *xcodes_bytes = (size_t)mx::act_codes_t16_bytes(M, K);
    return MX_OK;
}

mx_status mx_quant_act_t16(int64_t M, int64_t K, const void *x, int64_t ldx, void *xq,
                           void *xcodes, int rule, mx_stream_t stream) {
    if (rule != mx::RULE_OCP && rule != mx::RULE_CEIL448) return MX_ERR_UNSUPPORTED;
    if (M < 1 || K < 32 || K % 32 != 0 || ldx < K) return MX_ERR_SHAPE;
    if (!x || !xq || !xcodes) return MX_ERR_NULL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(xcodes) || ldx % 8 != 0)
        return MX_ERR_ALIGN;
    if (mx::act_t16_data_bytes(M, K) > kMaxRsrc) return MX_ERR_SHAPE;
    mx_status st = device_ok();
    if (st != MX_OK) return st;
    return launched(mx::launch_quant_t16(M, K, x, ldx, xq, xcodes, rule,
                                         reinterpret_cast<hipStream_t>(stream)));
}

mx_status mx_linear_workspace(int elem, int layout, int64_t N, int64_t K, int64_t M, int act,
                              int prequantized, size_t *bytes) {
    if (!bytes) return MX_ERR_NULL;
    mx_status st = shape_ok(elem, layout, 1, N, K);
    if (st != MX_OK) return st;
    if (M < 1) return MX_ERR_SHAPE;
    if (act != ACT_BF16 && act != ACT_MXFP8 && act != ACT_MXFP8_T16) return MX_ERR_UNSUPPORTED;
    *bytes = 0;
    const bool gemm = use_gemm(act, M);
    const bool long_k = !gemm && !gemv_w8_plan(N, K, M).ok;
    if (act == ACT_MXFP8 && !prequantized && fused_quant_ok(elem, N, K, M))
        return MX_OK;                                   // quantized inside the GEMV
    if (act == ACT_MXFP8 && !prequantized && !long_k)   // in-call quantization into T16
        *bytes = (size_t)(round256(mx::act_t16_data_bytes(M, K)) + mx::act_codes_t16_bytes(M, K));
    else if (act == ACT_MXFP8 && !prequantized)         // row-major, chunked GEMV for long K
        *bytes = (size_t)(round256(M * padded_k(K)) + round256(M * (padded_k(K) / 32)));
    else if (act == ACT_MXFP8 && gemm)                  // row-major input restaged into T16
        *bytes = (size_t)(round256(mx::act_t16_data_bytes(M, K)) + mx::act_codes_t16_bytes(M, K));
    return MX_OK;
}

mx_status mx_linear(int elem, int layout, int64_t N, int64_t K, const void *w_packed,
                    const void *codes_packed, int64_t M, int act, int rule, const void *x,
                    int64_t ldx, const void *xq, int64_t ldq, const void *xcodes, int64_t ldc,
                    const void *bias, void *y, int64_t ldy, void *ws, size_t ws_bytes,
                    mx_stream_t stream) {
    mx_status st = shape_ok(elem, layout, 1, N, K);
    if (st != MX_OK) return st;
    if (act != ACT_BF16 && act != ACT_MXFP8 && act != ACT_MXFP8_T16) return MX_ERR_UNSUPPORTED;
    if (rule != mx::RULE_OCP && rule != mx::RULE_CEIL448) return MX_ERR_UNSUPPORTED;
    if (elem == E2M1 && (layout != ROW32 || act != ACT_BF16)) return MX_ERR_UNSUPPORTED;
    if (M < 1 || ldy < N) return MX_ERR_SHAPE;
    if (!w_packed || !codes_packed || !y) return MX_ERR_NULL;
    if (!aligned16(w_packed) || !aligned16(codes_packed) || !aligned16(y) || ldy % 8 != 0)
        return MX_ERR_ALIGN;
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 1u)) return MX_ERR_ALIGN;
    const int64_t Kp = padded_k(K);
    const bool t16 = act == ACT_MXFP8_T16;
    const bool preq = act == ACT_MXFP8 && xq && xcodes;
    const bool incall = act == ACT_MXFP8 && !preq;
    if (act == ACT_BF16 || incall) {
        if (!x) return MX_ERR_NULL;
        if (ldx < K) return MX_ERR_SHAPE;
        if (!aligned16(x) || ldx % 8 != 0) return MX_ERR_ALIGN;
        if (M * ldx * 2 > kMaxRsrc) return MX_ERR_SHAPE;
    }
    if (preq) {
        if (ldq < K || ldc < K / 32) return MX_ERR_SHAPE;
        if (!aligned16(xq) || ldq % 16 != 0) return MX_ERR_ALIGN;
        if (M * ldq > kMaxRsrc || M * ldc > kMaxRsrc) return MX_ERR_SHAPE;
    }
    if (t16) {
        if (!xq || !xcodes) return MX_ERR_NULL;
        if (!aligned16(xq) || !aligned16(xcodes)) return MX_ERR_ALIGN;
    }
    if ((incall || t16) && mx::act_t16_data_bytes(M, K) > kMaxRsrc) return MX_ERR_SHAPE;
    size_t need = 0;
    mx_linear_workspace(elem, layout, N, K, M, act, incall ? 0 : 1, &need);
    if (need > 0 && (!ws || ws_bytes < need)) return MX_ERR_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return MX_ERR_ALIGN;
    const bool gemm = use_gemm(act, M);
    if (gemm && (N * Kp > kMaxRsrc || M * ldy * 2 > kMaxRsrc)) return MX_ERR_SHAPE;
    if ((st = device_ok()) != MX_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t *wsp = static_cast<uint8_t *>(ws);

    // the MXFP8 activation: T16 (given, or quantized here into ws) or row-major
    const uint8_t *aq = static_cast<const uint8_t *>(xq);
    const uint8_t *ac = static_cast<const uint8_t *>(xcodes);
    int64_t lq = ldq, lc = ldc;
    bool a16 = t16;
    const mx::GemvW8Plan w8 = gemv_w8_plan(N, K, M);
    if (incall && !gemm && fused_quant_ok(elem, N, K, M)) {
        mx::GemvW8Args g{};
        g.w = static_cast<const uint8_t *>(w_packed);
        g.codes = static_cast<const uint8_t *>(codes_packed);
        g.N = N;
        g.K = K;
        g.M = M;
        g.xb = static_cast<const uint16_t *>(x);
        g.ldx = ldx;
        g.bias = static_cast<const uint16_t *>(bias);
        g.y = static_cast<uint16_t *>(y);
        g.ldy = ldy;
        log_dispatch("linear: gemv_w8_fused_kernel %s, quantization inside (rule %d), "
                     "%d waves x %d steps x %d tiles; M=%lld N=%lld K=%lld",
                     layout_name(layout), rule, w8.nw, w8.spw, w8.g, (long long)M, (long long)N,
                     (long long)K);
        return launched(mx::launch_gemv_w8_fused(layout, rule, g, w8, s));
    }
    if (incall && !gemm && !w8.ok) {
        // K beyond the T16 GEMV's registers: row-major quantization into ws
        // for the chunked GEMV
        uint8_t *q = wsp, *c = wsp + round256(M * Kp);
        lq = Kp;
        lc = Kp / 32;
        log_dispatch("linear: quant_act_kernel (row-major, rule %d) M=%lld K=%lld", rule,
                     (long long)M, (long long)K);
        if ((st = launched(mx::launch_quant(M, K, x, ldx, q, lq, c, lc, rule, s))) != MX_OK)
            return st;
        aq = q;
        ac = c;
    } else if (incall) {
        uint8_t *q = wsp, *c = wsp + round256(mx::act_t16_data_bytes(M, K));
        log_dispatch("linear: quant_act_t16_kernel (rule %d) M=%lld K=%lld", rule, (long long)M,
                     (long long)K);
        if ((st = launched(mx::launch_quant_t16(M, K, x, ldx, q, c, rule, s))) != MX_OK) return st;
        aq = q;
        ac = c;
        a16 = true;
    }
    if (gemm) {
        mx::GemmArgs g{};
        g.w = static_cast<const uint8_t *>(w_packed);
        g.codes = static_cast<const uint8_t *>(codes_packed);
        g.N = N;
        g.K = K;
        g.M = M;
        g.xq = aq;
        g.xct = ac;
        if (!a16) {
            // restage the row-major bytes and codes into the T16 layout
            uint8_t *q = wsp, *c = wsp + round256(mx::act_t16_data_bytes(M, K));
            if ((st = launched(mx::launch_act_data_t16(M, K, aq, lq, q, s))) != MX_OK) return st;
            if ((st = launched(mx::launch_act_codes_t16(M, K, ac, lc, c, s))) != MX_OK) return st;
            g.xq = q;
            g.xct = c;
        }
        g.bias = static_cast<const uint16_t *>(bias);
        g.y = static_cast<uint16_t *>(y);
        g.ldy = ldy;
        log_dispatch("linear: gemm_w8a8_kernel %s, %d x 256 tiles; M=%lld N=%lld K=%lld",
                     layout_name(layout), mx::gemm_tile_n(N), (long long)M, (long long)N,
                     (long long)K);
        return launched(mx::launch_gemm(layout, g, s));
    }
    if (act != ACT_BF16 && w8.ok) {
        mx::GemvW8Args g{};
        g.w = static_cast<const uint8_t *>(w_packed);
        g.codes = static_cast<const uint8_t *>(codes_packed);
        g.N = N;
        g.K = K;
        g.M = M;
        g.bias = static_cast<const uint16_t *>(bias);
        g.y = static_cast<uint16_t *>(y);
        g.ldy = ldy;
        if (a16) {
            g.xf = aq;
            g.xct = ac;
        } else {
            g.xq = aq;
            g.ldq = lq;
            g.xc = ac;
            g.ldc = lc;
        }
        log_dispatch("linear: %s %s, %s activations, %d waves x %d steps x %d tiles; "
                     "M=%lld N=%lld K=%lld",
                     mx::gemv_w8_even(N, K, w8) ? (a16 ? "gemv_w8_even_kernel" : "gemv_w8_rm_kernel")
                                                : "gemv_w8_kernel",
                     layout_name(layout), a16 ? "T16" : "row-major", w8.nw, w8.spw, w8.g,
                     (long long)M, (long long)N, (long long)K);
        return launched(mx::launch_gemv_w8(layout, a16, g, w8, s));
    }
    if (a16) return MX_ERR_UNSUPPORTED;             // T16 input with K beyond the GEMV plan
    mx::GemvArgs a{};
    a.w = static_cast<const uint8_t *>(w_packed);
    a.codes = static_cast<const uint8_t *>(codes_packed);
    a.E = 1;
    a.N = N;
    a.K = K;
    a.rows = M;
    a.topk = 1;
    a.xrows = M;
    if (act == ACT_MXFP8) {
        a.x = aq;
        a.ldx = lq;
        a.xcodes = ac;
        a.ldc = lc;
    } else {
        a.x = x;
        a.ldx = ldx;
    }
    a.bias = static_cast<const uint16_t *>(bias);
    a.y = static_cast<uint16_t *>(y);
    a.ldy = ldy;
    const mx::GemvShape sh = gemv_shape(Kp / 128, false);
    log_dispatch("linear: gemv_kernel %s %s, %s activations, %d waves x %d-step chunks x %d "
                 "tiles; M=%lld N=%lld K=%lld",
                 elem_name(elem), layout_name(layout), act == ACT_BF16 ? "bf16" : "row-major MXFP8",
                 sh.nw, sh.chunk, sh.tiles, (long long)M, (long long)N, (long long)K);
    return launched(mx::launch_gemv(elem, layout, act, false, a, sh, s));
}

mx_status mx_moe_workspace(int elem, int64_t E, int64_t N, int64_t K, int64_t T, int64_t topk,
                           int combine, size_t *bytes) {
    if (!bytes) return MX_ERR_NULL;
    mx_status st = shape_ok(elem, ROW32, E, N, K);
    if (st != MX_OK) return st;
    if (T < 1 || topk < 1 || topk > E || T * topk > mx::kMoeMaxPairs) return MX_ERR_SHAPE;
    *bytes = combine ? (size_t)(T * topk * N * 4) : 0;
    return MX_OK;
}

mx_status mx_moe_linear(int elem, int64_t E, int64_t N, int64_t K, const void *w_packed,
                        const void *codes_packed, int64_t T, int64_t topk, const void *x,
                        int64_t ldx, const int32_t *topk_ids, const float *topk_weights, void *y,
                        void *ws, size_t ws_bytes, mx_stream_t stream) {
    return moe_run(elem, E, N, K, w_packed, codes_packed, T, topk, x, ldx, false, false,
                   topk_ids, topk_weights, y, N, ws, ws_bytes, stream);
}

mx_status mx_moe_linear_noalloc(int elem, int64_t E, int64_t N, int64_t K, const void *w_packed,
                                const void *codes_packed, int64_t T, int64_t topk, const void *x,
                                int64_t ldx, const int32_t *topk_ids, const float *topk_weights,
                                void *y, mx_stream_t stream) {
    size_t need = 0;
    mx_status st = mx_moe_workspace(elem, E, N, K, T, topk, topk_weights ? 1 : 0, &need);
    if (st != MX_OK) return st;
    if (need > (size_t)mx::kStaticScratchBytes) return MX_ERR_WORKSPACE;   // beyond the buffer
    // host-side checks first (moe_run repeats them), then the device's buffer
    if (!w_packed || !codes_packed || !x || !topk_ids || !y) return MX_ERR_NULL;
    void *ws = nullptr;
    if (need > 0) {
        if ((st = device_ok()) != MX_OK) return st;
        if (!(ws = mx::static_scratch())) return MX_ERR_DEVICE;
    }
    return moe_run(elem, E, N, K, w_packed, codes_packed, T, topk, x, ldx, false, false,
                   topk_ids, topk_weights, y, N, ws, need, stream);
}

mx_status mx_moe_copies(int elem, int64_t E, int64_t Np, int64_t inter, int64_t K, int64_t H,
                        const void *w13, const void *s13, const void *w2, const void *s2,
                        void *w13_out, void *s13_out, void *w2_out, void *s2_out, void *ws,
                        size_t ws_bytes, mx_stream_t stream) {
    if (elem != E4M3 && elem != E2M1) return MX_ERR_UNSUPPORTED;
    if (E < 1 || H < 1 || inter < 32 || inter % 32 != 0 || Np % 32 != 0 || inter > Np ||
        K < 32 || K % 32 != 0)
        return MX_ERR_SHAPE;
    if (!w13 || !s13 || !w2 || !s2 || !w13_out || !s13_out || !w2_out || !s2_out || !ws)
        return MX_ERR_NULL;
    if (!aligned16(w13) || !aligned16(w2) || !aligned16(w13_out) || !aligned16(w2_out) ||
        !aligned16(ws))
        return MX_ERR_ALIGN;
    if (ws_bytes < 256) return MX_ERR_WORKSPACE;
    mx_status st = device_ok();
    if (st != MX_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((st = flagged(ws, s, [&](int *bad) {
             return mx::launch_moe_padding_check(elem, E, Np, inter, K, H, w13, w2, bad, s);
         })) != MX_OK)
        return st;
    return launched(mx::launch_moe_copies(elem, E, Np, inter, K, H, w13, s13, w2, s2, w13_out,
                                          s13_out, w2_out, s2_out, s));
}

mx_status mx_fold_row_codes(int64_t N, int64_t K, const void *codes_row, int64_t ldc,
                            void *codes_blk, void *ws, size_t ws_bytes, mx_stream_t stream) {
    if (N < 32 || N % 32 != 0 || K < 32 || K % 32 != 0 || ldc < K / 32) return MX_ERR_SHAPE;
    if (N * ldc > kMaxRsrc) return MX_ERR_SHAPE;
    if (!codes_row || !codes_blk || !ws) return MX_ERR_NULL;
    if (!aligned16(ws)) return MX_ERR_ALIGN;
    if (ws_bytes < 256) return MX_ERR_WORKSPACE;
    mx_status st = device_ok();
    if (st != MX_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return flagged(ws, s, [&](int *bad) {
        return mx::launch_fold_codes(N, K / 32, ldc, codes_row, codes_blk, bad, s);
    });
}

mx_status mx_fused_layout_permute(int kind, int layout, int64_t N, int64_t K, int64_t heads,
                                  const void *w, const void *codes, void *w_out,
                                  void *codes_out, mx_stream_t stream) {
    if (kind != 0 && kind != 1) return MX_ERR_UNSUPPORTED;
    if (layout != ROW32 && layout != BLK32) return MX_ERR_UNSUPPORTED;
    if (kind == 0 && layout != ROW32) return MX_ERR_UNSUPPORTED;
    if (N < 1 || K < 32 || K % 32 != 0 || heads < 1) return MX_ERR_SHAPE;
    if (kind == 0 && (N % heads != 0 || (N / heads) % 16 != 0)) return MX_ERR_SHAPE;
    if (kind == 1 && (K % heads != 0 || (K / heads) % 32 != 0)) return MX_ERR_SHAPE;
    if (layout == BLK32 && N % 32 != 0) return MX_ERR_SHAPE;
    if (!w || !codes || !w_out || !codes_out) return MX_ERR_NULL;
    if (!aligned16(w) || !aligned16(w_out)) return MX_ERR_ALIGN;
    mx_status st = device_ok();
    if (st != MX_OK) return st;
    const int64_t crows = layout == BLK32 ? N / 32 : N;
    return launched(mx::launch_fused_layout(kind, N, K, heads, crows, w, codes, w_out, codes_out,
                                            reinterpret_cast<hipStream_t>(stream)));
}

mx_status mx_e4m3_from_dequant(int layout, int64_t N, int64_t K, const void *w_bf16,
                               int64_t ldw, const void *codes, void *w_out, void *ws,
                               size_t ws_bytes, mx_stream_t stream) {
    if (layout != ROW32 && layout != BLK32) return MX_ERR_UNSUPPORTED;
    if (N < 1 || K < 32 || K % 32 != 0 || ldw < K || (layout == BLK32 && N % 32 != 0))
        return MX_ERR_SHAPE;
    if (!w_bf16 || !codes || !w_out || !ws) return MX_ERR_NULL;
    if (!aligned16(w_bf16) || ldw % 8 != 0 || !aligned16(w_out) || !aligned16(ws))
        return MX_ERR_ALIGN;
    if (ws_bytes < 256) return MX_ERR_WORKSPACE;
    mx_status st = device_ok();
    if (st != MX_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return flagged(ws, s, [&](int *bad) {
        return mx::launch_e4m3_from_bf16(layout, N, K, w_bf16, ldw, codes, w_out, bad, s);
    });
}

mx_status mx_moe_gate_up(int elem, int64_t E, int64_t inter, int64_t K, const void *w13_packed,
                         const void *codes_packed, int64_t T, int64_t topk, const void *x,
                         int64_t ldx, const int32_t *topk_ids, void *h, int64_t ldh,
                         mx_stream_t stream) {
    if (inter < 8 || inter % 8 != 0) return MX_ERR_SHAPE;
    if (ldh < inter) return MX_ERR_SHAPE;
    if (ldh % 8 != 0) return MX_ERR_ALIGN;
    return moe_run(elem, E, 2 * inter, K, w13_packed, codes_packed, T, topk, x, ldx, false, true,
                   topk_ids, nullptr, h, ldh, nullptr, 0, stream);
}

mx_status mx_moe_down(int elem, int64_t E, int64_t H, int64_t inter, const void *w2_packed,
                      const void *codes_packed, int64_t T, int64_t topk, const void *h,
                      int64_t ldh, const int32_t *topk_ids, const float *topk_weights, void *y,
                      void *ws, size_t ws_bytes, mx_stream_t stream) {
    return moe_run(elem, E, H, inter, w2_packed, codes_packed, T, topk, h, ldh, true, false,
                   topk_ids, topk_weights, y, H, ws, ws_bytes, stream);
}

}  // extern "C"
