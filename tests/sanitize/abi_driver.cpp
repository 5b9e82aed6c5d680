// abi_driver.cpp -- drives every entry point of the C ABI (fa_api.cpp) over
// valid and invalid arguments with the stand-in launchers of abi_stubs.cpp,
// built with -fsanitize=address,undefined: every argument check, size
// product and pointer derivation of the host code runs under the
// sanitizers.  Exits non-zero on the first unexpected status or recorded
// argument (a sanitizer report aborts the run by itself).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <string_view>

#include "abi_stubs.h"
#include "fa.h"

namespace {

int failures = 0;

#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__,      \
                         __LINE__, #cond);                                   \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

// Fake, 16-byte aligned device addresses: the stand-ins never touch them.
void *const P = reinterpret_cast<void *>(uintptr_t(0x10000));
float *const L = reinterpret_cast<float *>(uintptr_t(0x20000));
void *const W = reinterpret_cast<void *>(uintptr_t(0x40000));

fa_status_t fwd(int64_t B, int64_t H, int64_t N, int64_t Nk, int64_t d, int64_t dv,
                float scale = 0.125f, fa_dtype_t t = FA_DTYPE_BF16, const void *q = P,
                void *o = P, float *lse = L) {
    return fa_fwd(q, P, P, o, lse, B, H, N, Nk, d, dv, 1, scale, t, nullptr);
}

void test_fwd() {
    const int before = stub::last.calls;
    // invalid arguments: no launcher is reached
    CHECK(fwd(1, 1, 4, 4, 64, 64, 0.1f, FA_DTYPE_BF16, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(fwd(1, 1, 4, 4, 64, 64, 0.1f, FA_DTYPE_BF16, P, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(fwd(1, 1, 4, 4, 64, 64, 0.1f, FA_DTYPE_BF16, P, P, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(fwd(0, 1, 4, 4, 64, 64) == FA_ERR_INVALID_ARG);
    CHECK(fwd(1, -1, 4, 4, 64, 64) == FA_ERR_INVALID_ARG);
    CHECK(fwd(1, 1, 0, 4, 64, 64) == FA_ERR_INVALID_ARG);
    CHECK(fwd(1, 1, 4, 0, 64, 64) == FA_ERR_INVALID_ARG);
    CHECK(fwd(1, 1, 4, 4, 64, 64, NAN) == FA_ERR_INVALID_ARG);
    CHECK(fwd(1, 1, 4, 4, 64, 64, INFINITY) == FA_ERR_INVALID_ARG);
    CHECK(fwd(1, 1, 4, 4, 64, 64, 0.1f, static_cast<fa_dtype_t>(7)) == FA_ERR_INVALID_ARG);
    CHECK(fwd(1, 1, 4, 4, 64, 64, 0.1f, FA_DTYPE_BF16, reinterpret_cast<void *>(0x10008)) ==
          FA_ERR_INVALID_ARG);
    CHECK(fwd(1, 1, 4, 4, 64, 64, 0.1f, FA_DTYPE_BF16, P, P, reinterpret_cast<float *>(0x20002)) ==
          FA_ERR_INVALID_ARG);
    const int64_t big = std::numeric_limits<int64_t>::max();
    CHECK(fwd(big, big, 4, 4, 64, 64) == FA_ERR_INVALID_ARG);          // B*H overflows
    CHECK(fwd(1, 1, big / 2, 4, 64, 64) == FA_ERR_INVALID_ARG);        // N*d overflows
    CHECK(fwd(1, 1, 4, big, 64, 64) == FA_ERR_INVALID_ARG);
    CHECK(fwd(int64_t(1) << 20, int64_t(1) << 12, 1, 4, 64, 64) == FA_ERR_INVALID_ARG);
    CHECK(fwd(1, 1, 4, 4, 48, 64) == FA_ERR_UNSUPPORTED);
    CHECK(fwd(1, 1, 4, 4, 64, 512) == FA_ERR_UNSUPPORTED);
    CHECK(fwd(1, 1, 4, int64_t(1) << 23, 128, 128) == FA_ERR_UNSUPPORTED);   // 2 GiB per head
    CHECK(stub::last.calls == before);

    // valid calls reach the expected launcher with the arguments unchanged
    CHECK(fwd(64, 16, 1024, 1024, 64, 64) == FA_OK);
    CHECK(std::string_view(stub::last.kernel) == "fwd_mfma_wide");
    CHECK(stub::last.fwd.B == 64 && stub::last.fwd.H == 16 && stub::last.fwd.N == 1024 &&
          stub::last.fwd.causal == 1 && stub::last.fwd.scale == 0.125f);
    CHECK(fwd(2, 32, 8192, 8192, 128, 128) == FA_OK);
    CHECK(std::string_view(stub::last.kernel) == "fwd_mfma_wide");
    CHECK(fwd(1, 1, 5000, 5000, 64, 64) == FA_OK);
    CHECK(std::string_view(stub::last.kernel) == "fwd_mfma16");
    CHECK(fwd(1, 1, 50, 50, 32, 256) == FA_OK);
    CHECK(std::string_view(stub::last.kernel) == "fwd_mfma_generic");
    CHECK(fwd(1, 1, 50, 50, 64, 64, 0.f) == FA_OK);
    CHECK(std::string_view(stub::last.kernel) == "fwd_mfma_generic");
    CHECK(fwd(1, 1, 50, 50, 64, 64, 0.1f, FA_DTYPE_F32) == FA_OK);
    CHECK(std::string_view(stub::last.kernel) == "fwd_rowwise");
    // the largest accepted per-head slice: just under 2 GiB
    CHECK(fwd(1, 1, 1, (int64_t(1) << 23) - 1, 128, 128) == FA_OK);
}

void test_decode() {
    const size_t ws = fa_decode_splitkv_workspace_size(8, 32, 1, 128, 64);
    CHECK(ws == 8454144u);
    CHECK(fa_decode_splitkv_workspace_size(std::numeric_limits<int64_t>::max(), 2, 1, 128, 64) == 0);
    CHECK(fa_decode_splitkv_workspace_size(1, 1, 1, std::numeric_limits<int64_t>::max(), 1) == 0);
    const int before = stub::last.calls;
    CHECK(fa_decode_splitkv(P, P, P, P, L, 8, 32, 1, 32768, 128, 128, 0, 0.1f, FA_DTYPE_BF16, -1,
                            W, ws, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(fa_decode_splitkv(P, P, P, P, L, 8, 32, 1, 32768, 128, 128, 0, 0.1f, FA_DTYPE_BF16, 64,
                            nullptr, ws, nullptr) == FA_ERR_WORKSPACE);
    CHECK(fa_decode_splitkv(P, P, P, P, L, 8, 32, 1, 32768, 128, 128, 0, 0.1f, FA_DTYPE_BF16, 64,
                            W, ws - 1, nullptr) == FA_ERR_WORKSPACE);
    CHECK(fa_decode_splitkv(P, P, P, P, L, 8, 32, 1, 32768, 128, 128, 0, 0.1f, FA_DTYPE_BF16, 64,
                            reinterpret_cast<void *>(0x40004), ws, nullptr) == FA_ERR_WORKSPACE);
    CHECK(fa_decode_splitkv(P, P, P, P, L, 8, 32, 1, 32768, 128, 128, 0, 0.1f, FA_DTYPE_BF16,
                            65537, W, size_t(1) << 40, nullptr) == FA_ERR_UNSUPPORTED);
    CHECK(fa_decode_splitkv_gqa(P, P, P, P, L, 8, 32, 6, 1, 32768, 128, 128, 0, 0.1f,
                                FA_DTYPE_BF16, 64, W, ws, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(fa_decode_splitkv_gqa(P, P, P, P, L, 8, 32, 0, 1, 32768, 128, 128, 0, 0.1f,
                                FA_DTYPE_BF16, 64, W, ws, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(stub::last.calls == before);

    CHECK(fa_decode_splitkv(P, P, P, P, L, 8, 32, 1, 32768, 128, 128, 0, 0.1f, FA_DTYPE_BF16, 64,
                            W, ws, nullptr) == FA_OK);
    const fa::DecodeArgs &d = stub::last.dec;
    CHECK(d.num_splits == 64 && d.seg_len == 512 && d.Hkv == 32);
    CHECK(d.ws_o == static_cast<float *>(W));
    CHECK(d.ws_lse == static_cast<float *>(W) + int64_t(8) * 32 * 64 * 1 * 128);
    // segments are 64-key aligned: 1000 keys over 3 splits -> 384 keys each
    CHECK(fa_decode_splitkv(P, P, P, P, L, 1, 1, 1, 1000, 64, 64, 0, 0.1f, FA_DTYPE_F32, 3, W,
                            fa_decode_splitkv_workspace_size(1, 1, 1, 64, 3), nullptr) == FA_OK);
    CHECK(stub::last.dec.seg_len == 384);
    // num_splits = 0 runs the automatic count
    const int S = fa_decode_splitkv_auto_splits(8, 32, 8, 1, 32768, 128, 128, FA_DTYPE_BF16);
    CHECK(S >= 1 && S <= 256);
    CHECK(fa_decode_splitkv_gqa(P, P, P, P, L, 8, 32, 8, 1, 32768, 128, 128, 0, 0.1f,
                                FA_DTYPE_BF16, 0, W, fa_decode_splitkv_workspace_size(8, 32, 1, 128, S),
                                nullptr) == FA_OK);
    CHECK(stub::last.dec.num_splits == S && stub::last.dec.Hkv == 8);
    CHECK(fa_decode_splitkv_auto_splits(1, 6, 4, 1, 100, 64, 64, FA_DTYPE_BF16) == 0);
    CHECK(fa_decode_splitkv_auto_splits(std::numeric_limits<int64_t>::max(), 2, 1, 1, 100, 64, 64,
                                        FA_DTYPE_BF16) == 0);
}

void test_decode_noalloc() {
    const int before = stub::last.calls;
    // partials of 8 x 64 heads x 128 splits x 129 floats: 33.8 MB > 16 MiB
    CHECK(fa_decode_splitkv_noalloc(P, P, P, P, L, 8, 64, 1, 32768, 128, 128, 0, 0.1f,
                                    FA_DTYPE_BF16, 128, nullptr) == FA_ERR_WORKSPACE);
    CHECK(fa_decode_splitkv_noalloc(nullptr, P, P, P, L, 8, 32, 1, 32768, 128, 128, 0, 0.1f,
                                    FA_DTYPE_BF16, 64, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(stub::last.calls == before);
    CHECK(fa_decode_splitkv_noalloc(P, P, P, P, L, 8, 32, 1, 32768, 128, 128, 0, 0.1f,
                                    FA_DTYPE_BF16, 64, nullptr) == FA_OK);
    const fa::DecodeArgs &d = stub::last.dec;
    float *const s = reinterpret_cast<float *>(uintptr_t(0x800000));
    CHECK(d.ws_o == s && d.ws_lse == s + int64_t(8) * 32 * 64 * 128 && d.num_splits == 64);
    CHECK(fa_decode_splitkv_workspace_size(8, 32, 1, 128, 64) <= FA_DECODE_NOALLOC_MAX_WORKSPACE);
}

void test_bwd() {
    const size_t ws = fa_bwd_workspace_size(4, 8, 300);
    CHECK(ws == size_t(4) * 8 * 300 * 8);
    CHECK(fa_bwd_workspace_size(std::numeric_limits<int64_t>::max(), 2, 2) == 0);
    const int before = stub::last.calls;
    CHECK(fa_bwd(P, P, P, P, L, nullptr, P, P, P, 4, 8, 300, 200, 64, 64, 1, 0.1f, FA_DTYPE_BF16,
                 W, ws, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(fa_bwd(P, P, P, P, L, P, P, reinterpret_cast<void *>(0x10002), P, 4, 8, 300, 200, 64, 64,
                 1, 0.1f, FA_DTYPE_BF16, W, ws, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(fa_bwd(P, P, P, P, L, P, P, P, P, 4, 8, 300, 200, 64, 64, 1, 0.1f, FA_DTYPE_BF16, W,
                 ws - 4, nullptr) == FA_ERR_WORKSPACE);
    CHECK(stub::last.calls == before);
    CHECK(fa_bwd(P, P, P, P, L, P, P, P, P, 4, 8, 300, 200, 64, 32, 1, 0.1f, FA_DTYPE_F16, W, ws,
                 nullptr) == FA_OK);
    CHECK(std::string_view(stub::last.kernel) == "bwd");
    CHECK(stub::last.bwd.Dsum == static_cast<float *>(W) && stub::last.bwd.a.dv == 32);
}

void test_status_strings() {
    for (int s = -2; s < 8; ++s) CHECK(fa_status_string(static_cast<fa_status_t>(s)) != nullptr);
}

}  // namespace

int main() {
    test_fwd();
    test_decode();
    test_decode_noalloc();
    test_bwd();
    test_status_strings();
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::puts("abi_driver: all checks passed");
    return 0;
}
