// mx_plan.cpp -- host-only launch plans of the W8A8 decode GEMV (kept out of
// the kernel sources so the host logic builds alone, e.g. with sanitizers).
#include "mx_kernels.h"

namespace mx {

// (K % 128 == 0: the even kernels step through whole 2 KB chunks, S per tile)
bool gemv_w8_even(int64_t N, int64_t K, const GemvW8Plan &pl) {
    const int64_t S = K / 128, T = N / 16;
    return K % 128 == 0 && pl.ok && pl.nw == 8 && S == 8 * (int64_t)pl.spw && T % pl.g == 0 &&
           pl.g * pl.spw <= 16;
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
