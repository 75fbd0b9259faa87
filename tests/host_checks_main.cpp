// Host-side checks of the library's planning and argument validation, built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
// (tests/test_host_sanitizers.py).  The kernel launchers are replaced by
// stubs that abort: every call made here must be answered by the host code
// alone (a plan, a size or an error status), so reaching a launcher is a
// failure, and so is any overflow, division by zero or out-of-bounds access
// the sanitizers see.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "attention.hpp"
#include "launch.hpp"
#include "nt.h"

namespace ntk {
#define NT_STUB                                              \
    {                                                        \
        std::fprintf(stderr, "a kernel launcher was reached\n"); \
        std::abort();                                        \
    }
hipError_t launch_resident_f32(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_STUB
hipError_t launch_resident_f16(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_STUB
hipError_t launch_resident_bf16(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_STUB
hipError_t launch_looped_f32(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_STUB
hipError_t launch_looped_f16(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_STUB
hipError_t launch_looped_bf16(int, int, int, bool, const RowArgs &, int64_t, hipStream_t) NT_STUB
hipError_t launch_persistent_f32(int, int, int, const RowArgs &, hipStream_t, int64_t, int) NT_STUB
hipError_t launch_persistent_f16(int, int, int, const RowArgs &, hipStream_t, int64_t, int) NT_STUB
hipError_t launch_persistent_bf16(int, int, int, const RowArgs &, hipStream_t, int64_t, int) NT_STUB
hipError_t launch_split_f32(int, int, bool, int, const RowArgs &, hipStream_t) NT_STUB
hipError_t launch_split_f16(int, int, bool, int, const RowArgs &, hipStream_t) NT_STUB
hipError_t launch_split_bf16(int, int, bool, int, const RowArgs &, hipStream_t) NT_STUB
hipError_t launch_norm_split_f32(int, int, int, bool, bool, const RowArgs &, hipStream_t) NT_STUB
hipError_t launch_norm_split_f16(int, int, int, bool, bool, const RowArgs &, hipStream_t) NT_STUB
hipError_t launch_norm_split_bf16(int, int, int, bool, bool, const RowArgs &, hipStream_t) NT_STUB
hipError_t launch_attention(int, int, const AttnArgs &, hipStream_t) NT_STUB
#undef NT_STUB
}  // namespace ntk

static int failures = 0;

static void expect_error(nt_status s, const char *what) {
    if (s == NT_OK) {
        std::fprintf(stderr, "expected an error: %s\n", what);
        ++failures;
    }
}

int main() {
    // plans and workspace sizes over every op, type and extreme sizes
    const int64_t Ms[] = {0, 1, 2, 255, 256, 2047, 2048, 4096, 1 << 20, (1LL << 31) - 1, 1LL << 31, 1LL << 40,
                          INT64_MAX};
    const int64_t Ns[] = {-1, 0, 1, 7, 781, 8192, 16385, 32769, 1 << 20, (1LL << 31) - 1, 1LL << 31, INT64_MAX};
    long plans = 0;
    for (int op = -1; op <= 8; ++op)
        for (int64_t M : Ms)
            for (int64_t N : Ns)
                for (int dt = -1; dt <= 3; ++dt) {
                    for (int al = 0; al <= 1; ++al) {
                        nt_plan p;
                        if (nt_plan_launch((nt_op)op, M, N, (nt_dtype)dt, al, &p) == NT_OK) ++plans;
                    }
                    (void)nt_softmax_workspace_bytes(M, N, (nt_dtype)dt);
                    (void)nt_norm_workspace_bytes(op, M, N, (nt_dtype)dt);
                }
    expect_error(nt_plan_launch(NT_OP_SOFTMAX, 4, 8, NT_F32, 1, nullptr), "plan into NULL");

    // argument errors are answered before anything is launched
    char buf[256];
    void *P = buf + 64;  // a 16-byte aligned address never dereferenced on the host
    void *odd = buf + 65;
    const int64_t wide = 1 << 20;
    expect_error(nt_softmax_rows(4, 8, (nt_dtype)7, P, P, nullptr, 0, nullptr), "softmax bad dtype");
    expect_error(nt_softmax_rows(-1, 8, NT_F32, P, P, nullptr, 0, nullptr), "softmax M < 0");
    expect_error(nt_softmax_rows(4, 0, NT_F32, P, P, nullptr, 0, nullptr), "softmax N = 0");
    expect_error(nt_softmax_rows(1LL << 40, 1 << 30, NT_F32, P, P, nullptr, 0, nullptr), "softmax M*N too big");
    expect_error(nt_softmax_rows(4, 8, NT_F32, nullptr, P, nullptr, 0, nullptr), "softmax x NULL");
    expect_error(nt_softmax_rows(4, 8, NT_F16, P, odd, nullptr, 0, nullptr), "softmax y misaligned");
    expect_error(nt_softmax_rows(4, wide, NT_F32, P, P, nullptr, wide, nullptr), "softmax workspace NULL");
    expect_error(nt_softmax_rows(4, wide, NT_F32, P, P, P, 8, nullptr), "softmax workspace small");
    expect_error(nt_softmax_causal_rows(4, 8, NT_F32, 0.0f, 4, 0, P, P, nullptr, 0, nullptr), "causal scale 0");
    expect_error(nt_softmax_causal_rows(4, 8, NT_F32, 1.0f, 0, 0, P, P, nullptr, 0, nullptr), "causal queries 0");
    expect_error(nt_softmax_causal_rows(4, 8, NT_F32, 1.0f, 4, -1, P, P, nullptr, 0, nullptr), "causal offset < 0");
    expect_error(nt_layernorm_rows(4, 8, NT_F32, -1.0f, P, nullptr, nullptr, P, nullptr, nullptr, nullptr),
                 "layernorm eps < 0");
    expect_error(nt_layernorm_rows(4, 8, NT_F16, 1e-5f, P, odd, nullptr, P, nullptr, nullptr, nullptr),
                 "layernorm gamma misaligned");
    expect_error(nt_rmsnorm_rows(4, 8, NT_BF16, 1e-6f, nullptr, nullptr, P, nullptr), "rmsnorm x NULL");
    expect_error(nt_rmsnorm_rows(4, 1LL << 31, NT_BF16, 1e-6f, P, nullptr, P, nullptr), "rmsnorm N too big");
    expect_error(nt_layernorm_rows_ws(4, wide, NT_F32, 1e-5f, P, nullptr, nullptr, P, nullptr, nullptr, P, 64,
                                      nullptr),
                 "layernorm_ws workspace small");
    expect_error(nt_rmsnorm_rows_ws(4, wide, NT_BF16, 1e-6f, P, nullptr, P, odd, wide, nullptr),
                 "rmsnorm_ws workspace misaligned");
    expect_error(nt_add_rmsnorm_rows(4, 8, NT_BF16, 1e-6f, P, nullptr, nullptr, P, P, nullptr),
                 "add_rmsnorm residual NULL");
    expect_error(nt_add_rmsnorm_rows(4, 8, NT_BF16, 1e-6f, P, buf + 96, nullptr, buf + 128, buf + 128, nullptr),
                 "add_rmsnorm h == y");
    expect_error(nt_add_layernorm_rows(4, 8, NT_F32, 1e-5f, P, buf + 100, nullptr, nullptr, buf + 128, buf + 160,
                                       nullptr, nullptr, nullptr),
                 "add_layernorm residual out of x's phase");
    // attention: every argument error before a launch
    const int64_t big3 = INT64_MAX / 4;
    expect_error(nt_attention_fwd(2, 8, 8, 64, NT_F32, 0.1f, 0, 0, P, P, P, buf + 128, nullptr), "attn fp32");
    expect_error(nt_attention_fwd(2, 8, 8, 96, NT_BF16, 0.1f, 0, 0, P, P, P, buf + 128, nullptr), "attn D");
    expect_error(nt_attention_fwd(2, 8, 0, 64, NT_BF16, 0.1f, 0, 0, P, P, P, buf + 128, nullptr), "attn Lk 0");
    expect_error(nt_attention_fwd(-1, 8, 8, 64, NT_BF16, 0.1f, 0, 0, P, P, P, buf + 128, nullptr), "attn BH < 0");
    expect_error(nt_attention_fwd(2, 8, 8, 64, NT_BF16, 0.1f, 1, -1, P, P, P, buf + 128, nullptr), "attn offset");
    expect_error(nt_attention_fwd(2, 8, 8, 64, NT_BF16, 0.1f, 3, 0, P, P, P, buf + 128, nullptr), "attn causal");
    expect_error(nt_attention_fwd(2, big3, 8, 64, NT_BF16, 0.1f, 0, 0, P, P, P, buf + 128, nullptr), "attn size");
    expect_error(nt_attention_fwd(1 << 20, 1 << 20, 8, 64, NT_BF16, 0.1f, 0, 0, P, P, P, buf + 128, nullptr),
                 "attn grid");
    expect_error(nt_attention_fwd(2, 8, 8, 64, NT_BF16, -0.1f, 0, 0, P, P, P, buf + 128, nullptr), "attn scale");
    expect_error(nt_attention_fwd(2, 8, 8, 64, NT_BF16, 0.1f, 0, 0, nullptr, P, P, buf + 128, nullptr), "attn q NULL");
    expect_error(nt_attention_fwd(2, 8, 8, 64, NT_BF16, 0.1f, 0, 0, buf + 66, P, P, buf + 128, nullptr),
                 "attn misaligned");
    expect_error(nt_attention_fwd(2, 8, 8, 64, NT_BF16, 0.1f, 0, 0, P, P, P, P, nullptr), "attn o over q");
    for (int s = -1; s <= 12; ++s) (void)nt_status_string((nt_status)s);
    // tuning overrides: unknown names and malformed values change nothing
    expect_error(nt_set_override(nullptr, "1"), "override NULL name");
    expect_error(nt_set_override("NT_NOPE", "1"), "override unknown name");
    expect_error(nt_set_override("NT_FORCE_SHAPE", "4,x"), "override malformed shape");
    expect_error(nt_set_override("NT_FORCE_SHAPE", "4,2,1"), "override shape with a tail");
    expect_error(nt_set_override("NT_COOP_SPIN", "65537"), "override spin out of range");
    expect_error(nt_set_override("NT_PERSIST_GRID", "0"), "override grid 0");
    expect_error(nt_set_override("NT_PERSISTENT", "sometimes"), "override persistent mode");
    expect_error(nt_set_override("NT_FORCE_PATH", "both"), "override path");
    if (nt_set_override("NT_FORCE_SHAPE", "4,4") != NT_OK || nt_set_override("NT_FORCE_SHAPE", nullptr) != NT_OK) {
        std::fprintf(stderr, "override set/reset failed\n");
        ++failures;
    }

    std::printf("ok %ld plans, %d failures\n", plans, failures);
    return failures ? 1 : 0;
}
