// abi_stubs.cpp -- host stand-ins for the kernel launchers and the one HIP
// runtime call of fa_api.cpp, so that the C ABI's argument checking and
// dispatch can be built with g++ and run under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  Each launcher
// records the arguments it received; nothing is launched.
#include <hip/hip_runtime_api.h>

#include "abi_stubs.h"
#include "fa_internal.h"

namespace stub {
Record last;
}

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

namespace fa {

static hipError_t record(const char *kernel, const FwdArgs &a) {
    stub::last = stub::Record();
    stub::last.kernel = kernel;
    stub::last.fwd = a;
    stub::last.calls += 1;
    return hipSuccess;
}

hipError_t launch_fwd_rowwise(const FwdArgs &a) { return record("fwd_rowwise", a); }
hipError_t launch_fwd_mfma16(const FwdArgs &a) { return record("fwd_mfma16", a); }
hipError_t launch_fwd_mfma_wide(const FwdArgs &a) { return record("fwd_mfma_wide", a); }
hipError_t launch_fwd_mfma_generic(const FwdArgs &a) { return record("fwd_mfma_generic", a); }

// The same support rules as the device code's, restated for the stand-in.
bool fwd_mfma_supported(int dtype, int64_t d, int64_t dv, float scale) {
    return dtype != kF32 && (d == 64 || d == 128) && (dv == 64 || dv == 128) && scale > 0.f;
}
bool fwd_wide_preferred(int64_t d, int64_t dv, int64_t Nk) {
    return (d == 128 && dv == 128) || (d == 64 && dv == 64 && Nk <= 3072) || (d == 64 && dv == 128);
}

hipError_t launch_decode_splitkv(const DecodeArgs &a) {
    (void)record("decode", a.a);
    stub::last.dec = a;
    return hipSuccess;
}

int64_t decode_workgroups_per_split(int dtype, int64_t d, int64_t dv, int64_t B, int64_t Hkv,
                                    int64_t rows) {
    const int64_t r = (dtype != kF32 && d == dv && d <= 128 && rows >= 2) ? 16
                      : rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : 8;
    return B * Hkv * ((rows + r - 1) / r);
}

// A fake, 256-byte aligned address standing in for the static scratch.
hipError_t decode_scratch(void **ptr) {
    *ptr = reinterpret_cast<void *>(uintptr_t(0x800000));
    stub::last.scratch_lookups += 1;
    return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs &b) {
    (void)record("bwd", b.a);
    stub::last.bwd = b;
    return hipSuccess;
}

}  // namespace fa
