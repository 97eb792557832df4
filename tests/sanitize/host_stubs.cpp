// host_stubs.cpp -- test infrastructure: stand-ins for the HIP runtime calls
// and the kernel launchers of libmx, so that the library's host code
// (mx_api.cpp, mx_plan.cpp) builds and runs on a CPU under AddressSanitizer
// and UndefinedBehaviorSanitizer.  A fake gfx950 device 0 is current; no
// launcher touches memory; device-to-host copies of the load-time flags
// read zeros (nothing refused).  Every launch is counted.
#include <hip/hip_runtime.h>

#include <cstring>

#include "../../microscaling_quantized_linear_amd/csrc/mx_kernels.h"

extern "C" {

long mx_stub_launches = 0;

hipError_t hipGetDevice(int *dev) {
    *dev = 0;
    return hipSuccess;
}

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *prop, int dev) {
    if (dev != 0) return hipErrorInvalidDevice;
    std::memset(prop, 0, sizeof(*prop));
    std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
    return hipSuccess;
}

hipError_t hipMemsetAsync(void *, int, size_t, hipStream_t) { return hipSuccess; }

hipError_t hipMemcpyAsync(void *dst, const void *, size_t n, hipMemcpyKind kind, hipStream_t) {
    if (kind == hipMemcpyDeviceToHost) std::memset(dst, 0, n);
    return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

}  // extern "C"

namespace mx {

static hipError_t counted() {
    ++mx_stub_launches;
    return hipSuccess;
}

hipError_t launch_act_codes_t16(int64_t, int64_t, const void *, int64_t, void *, hipStream_t) {
    return counted();
}
hipError_t launch_act_data_t16(int64_t, int64_t, const void *, int64_t, void *, hipStream_t) {
    return counted();
}
hipError_t launch_pack(int, int, int64_t, int64_t, int64_t, const void *, const void *, void *,
                       void *, int *, unsigned *, hipStream_t) {
    return counted();
}
void *static_scratch() { return reinterpret_cast<void *>(uintptr_t(1) << 40); }
hipError_t launch_moe_padding_check(int, int64_t, int64_t, int64_t, int64_t, int64_t,
                                    const void *, const void *, int *, hipStream_t) {
    return counted();
}
hipError_t launch_moe_copies(int, int64_t, int64_t, int64_t, int64_t, int64_t, const void *,
                             const void *, const void *, const void *, void *, void *, void *,
                             void *, hipStream_t) {
    return counted();
}
hipError_t launch_fused_layout(int, int64_t, int64_t, int64_t, int64_t, const void *,
                               const void *, void *, void *, hipStream_t) {
    return counted();
}
hipError_t launch_fold_codes(int64_t, int64_t, int64_t, const void *, void *, int *, hipStream_t) {
    return counted();
}
hipError_t launch_e4m3_from_bf16(int, int64_t, int64_t, const void *, int64_t, const void *,
                                 void *, int *, hipStream_t) {
    return counted();
}
hipError_t launch_quant(int64_t, int64_t, const void *, int64_t, void *, int64_t, void *, int64_t,
                        int, hipStream_t) {
    return counted();
}
hipError_t launch_gemv(int, int, int, bool, const GemvArgs &, const GemvShape &, hipStream_t) {
    return counted();
}
hipError_t launch_moe_combine(int64_t, int64_t, int64_t, const float *, const float *, void *,
                              hipStream_t) {
    return counted();
}
hipError_t launch_gemm(int, const GemmArgs &, hipStream_t) { return counted(); }
int gemm_tile_n(int64_t N) { return N % 224 == 0 && (N / 224) % 8 == 0 ? 224 : 256; }
hipError_t launch_gemv_w8(int, bool, const GemvW8Args &, const GemvW8Plan &, hipStream_t) {
    return counted();
}
hipError_t launch_gemv_w8_fused(int, int, const GemvW8Args &, const GemvW8Plan &, hipStream_t) {
    return counted();
}
hipError_t launch_quant_t16(int64_t, int64_t, const void *, int64_t, void *, void *, int,
                            hipStream_t) {
    return counted();
}

}  // namespace mx
