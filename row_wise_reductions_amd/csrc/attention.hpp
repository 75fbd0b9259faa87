// Launcher of the attention forward kernel (attention.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ntk {

// q [BH, Lq, D], k and v [BH, Lk, D], o [BH, Lq, D]: row-major 16-bit
// arrays, 16-byte aligned.  Query i of head b sees keys j < Lk, and when
// `causal` only j <= i + offset.  s2 = scale * log2(e), rounded to fp32.
struct AttnArgs {
    const char *q;
    const char *k;
    const char *v;
    char *o;
    int64_t BH, Lq, Lk;
    int64_t offset;
    int64_t nqb;        // query blocks of 128 per head
    float s2;
    int32_t causal;
};

// dt: DT_F16 or DT_BF16; D: 64 or 128.  Returns the launch's status, or
// hipErrorInvalidValue for a (dt, D) that is not built.
hipError_t launch_attention(int dt, int D, const AttnArgs &a, hipStream_t s);

}  // namespace ntk
