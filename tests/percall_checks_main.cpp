// The per-call path of the library's host code reads no environment
// variable and makes no device-property query after the first call on a
// device (tests/test_host_sanitizers.py::test_per_call_path_is_quiet).
//
// The host code (csrc/nt_api.cpp) is linked into this program with:
//  - getenv defined here, counting its calls (it scans environ itself);
//  - the HIP calls the host code can make defined here as counting fakes
//    (device 0 current, 256 compute units, no stream capture), so nothing
//    touches a GPU;
//  - kernel launchers that count and succeed without launching anything.
// The pointers passed are host addresses that are never dereferenced.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attention.hpp"
#include "launch.hpp"
#include "nt.h"

extern "C" char **environ;

static std::atomic<long> g_getenv{0}, g_attr{0}, g_getdev{0}, g_capt{0}, g_launch{0}, g_symbol{0};

extern "C" char *getenv(const char *name) {
    g_getenv.fetch_add(1);
    const size_t n = std::strlen(name);
    for (char **e = environ; e && *e; ++e)
        if (std::strncmp(*e, name, n) == 0 && (*e)[n] == '=') return *e + n + 1;
    return nullptr;
}

hipError_t hipGetDevice(int *dev) {
    g_getdev.fetch_add(1);
    *dev = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t attr, int dev) {
    g_attr.fetch_add(1);
    *v = (attr == hipDeviceAttributeMultiprocessorCount && dev == 0) ? 256 : 0;
    return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t *dev) {
    *dev = 0;
    return hipSuccess;
}
hipError_t hipGetSymbolAddress(void **p, const void *) {
    g_symbol.fetch_add(1);
    *p = reinterpret_cast<void *>((uintptr_t)1 << 46);      // a device address stand-in, never dereferenced
    return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus *st) {
    g_capt.fetch_add(1);
    *st = hipStreamCaptureStatusNone;
    return hipSuccess;
}

namespace ntk {
#define NT_LAUNCH            \
    {                        \
        g_launch.fetch_add(1); \
        return hipSuccess;   \
    }
hipError_t launch_resident_f32(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_LAUNCH
hipError_t launch_resident_f16(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_LAUNCH
hipError_t launch_resident_bf16(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_LAUNCH
hipError_t launch_looped_f32(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_LAUNCH
hipError_t launch_looped_f16(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_LAUNCH
hipError_t launch_looped_bf16(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_LAUNCH
hipError_t launch_persistent_f32(int, int, int, const RowArgs &, hipStream_t, int64_t, int) NT_LAUNCH
hipError_t launch_persistent_f16(int, int, int, const RowArgs &, hipStream_t, int64_t, int) NT_LAUNCH
hipError_t launch_persistent_bf16(int, int, int, const RowArgs &, hipStream_t, int64_t, int) NT_LAUNCH
hipError_t launch_split_f32(int, int, bool, int, const RowArgs &, hipStream_t) NT_LAUNCH
hipError_t launch_split_f16(int, int, bool, int, const RowArgs &, hipStream_t) NT_LAUNCH
hipError_t launch_split_bf16(int, int, bool, int, const RowArgs &, hipStream_t) NT_LAUNCH
hipError_t launch_norm_split_f32(int, int, int, bool, bool, const RowArgs &, hipStream_t) NT_LAUNCH
hipError_t launch_norm_split_f16(int, int, int, bool, bool, const RowArgs &, hipStream_t) NT_LAUNCH
hipError_t launch_norm_split_bf16(int, int, int, bool, bool, const RowArgs &, hipStream_t) NT_LAUNCH
hipError_t launch_attention(int, int, const AttnArgs &, hipStream_t) NT_LAUNCH
#undef NT_LAUNCH
}  // namespace ntk

static int failures = 0;

static void expect_ok(nt_status s, const char *what) {
    if (s != NT_OK) {
        std::fprintf(stderr, "%s: %s\n", what, nt_status_string(s));
        ++failures;
    }
}

// One call of every entry point on shapes that take each path: single pass
// (one row and persistent workgroups), split softmax (workspace), looped
// and split norms, fused add + norm, causal softmax, plans and sizes.
static void every_entry_point(char *base) {
    // distinct, 256-byte-aligned addresses that are never dereferenced: the
    // row matrices 1 TiB apart, so no overlap check trips
    const size_t big = (size_t)1 << 40;
    char *x = base + ((size_t)1 << 44), *y = x + big, *r = y + big, *h = r + big, *ws = h + big;
    char *w = base, *b = base + (1 << 12);
    float *mean = reinterpret_cast<float *>(base + (2 << 12)), *rstd = reinterpret_cast<float *>(base + (3 << 12));
    expect_ok(nt_softmax_rows(1024, 781, NT_F32, x, y, nullptr, 0, nullptr), "softmax single pass");
    expect_ok(nt_softmax_rows(64, 262144, NT_F32, x, y, ws, 1 << 20, nullptr), "softmax split, one pass");
    expect_ok(nt_softmax_rows(64, 262144, NT_F32, x, x, ws, 1 << 20, nullptr), "softmax split, two kernels");
    expect_ok(nt_softmax_rows_noalloc(64, 262144, NT_F32, x, y, nullptr), "softmax split without a workspace");
    expect_ok(nt_softmax_causal_rows(131072, 4096, NT_BF16, 1.0f, 4096, 0, x, y, nullptr, 0, nullptr), "causal");
    expect_ok(nt_layernorm_rows(4096, 4096, NT_F16, 1e-5f, x, w, b, y, mean, rstd, nullptr), "layernorm persistent");
    expect_ok(nt_layernorm_rows(4096, 4095, NT_F16, 1e-5f, x, w, b, y, mean, rstd, nullptr), "layernorm one row");
    expect_ok(nt_rmsnorm_rows(16384, 8192, NT_BF16, 1e-6f, x, w, y, nullptr), "rmsnorm persistent");
    expect_ok(nt_rmsnorm_rows(16, 1 << 20, NT_BF16, 1e-6f, x, w, y, nullptr), "rmsnorm looped");
    expect_ok(nt_rmsnorm_rows_ws(16, 1 << 20, NT_BF16, 1e-6f, x, w, y, ws, 1 << 20, nullptr), "rmsnorm split");
    expect_ok(nt_layernorm_rows_ws(8, 1 << 20, NT_F32, 1e-5f, x, w, b, y, mean, rstd, ws, 1 << 20, nullptr),
              "layernorm split");
    expect_ok(nt_add_rmsnorm_rows(16384, 8192, NT_BF16, 1e-6f, x, r, w, h, y, nullptr), "add + rmsnorm");
    expect_ok(nt_add_layernorm_rows(4096, 4096, NT_F16, 1e-5f, x, r, w, b, h, y, mean, rstd, nullptr),
              "add + layernorm");
    expect_ok(nt_attention_fwd(32, 4096, 4096, 128, NT_BF16, 0.088f, 1, 0, x, r, h, y, nullptr), "attention");
    nt_plan p;
    expect_ok(nt_plan_launch(NT_OP_RMSNORM_WS, 16, 1 << 20, NT_BF16, 1, &p), "plan");
    (void)nt_softmax_workspace_bytes(64, 262144, NT_F32);
    (void)nt_norm_workspace_bytes(NT_OP_RMSNORM, 16, 1 << 20, NT_BF16);
}

int main() {
    static char arena[1 << 15];
    char *base = reinterpret_cast<char *>(((uintptr_t)arena + 255) & ~(uintptr_t)255);
    // the first calls may fill the per-device cache (one attribute query)
    every_entry_point(base);
    const long attr_first = g_attr.load(), symbol_first = g_symbol.load();
    const long getenv0 = g_getenv.load(), attr0 = g_attr.load(), launch0 = g_launch.load();
    for (int i = 0; i < 100; ++i) {
        every_entry_point(base);
        if (i == 50) expect_ok(nt_set_override("NT_COOP", "0"), "override");   // later calls: two kernels
    }
    expect_ok(nt_set_override("NT_COOP", nullptr), "override reset");
    const long getenv_calls = g_getenv.load() - getenv0, attr_calls = g_attr.load() - attr0;
    const long launches = g_launch.load() - launch0;
    std::printf("getenv %ld, device attribute queries %ld (first round %ld), symbol lookups %ld (first round %ld), "
                "launches %ld, capture queries %ld\n",
                getenv_calls, attr_calls, attr_first, g_symbol.load() - symbol_first, symbol_first, launches,
                g_capt.load());
    if (getenv_calls != 0) ++failures;
    if (attr_calls != 0 || attr_first > 1) ++failures;
    if (g_symbol.load() != 1) ++failures;
    if (launches < 100 * 14) ++failures;
    std::printf("%s, %d failures\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
