// Reference streams, used only to measure what this GPU's memory system
// delivers: the attainable bandwidth the row kernels are compared with, and
// the bytes the memory counters (FETCH_SIZE, WRITE_SIZE) report for a copy
// of known size.  Every 256-thread workgroup moves one contiguous tile of K
// 16-byte chunks per lane (chunk c of the tile belongs to lane c mod 256, as
// in the row kernels), with all K loads in flight before the first store.
//   copy   read `bytes`, write `bytes`
//   read   read `bytes` (folded into a value that is stored only if it
//          equals a number the host passes and never occurs): a read-only
//          stream
//   fill   write `bytes` of a constant: a write-only stream
// Loads are non-temporal; stores are non-temporal (policy 0) or the
// device-scope streaming stores of the row kernels (policy 1, nt sc1).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "row_kernels.hpp"

namespace {
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte store of lane t's k-th chunk of the tile at `tile`: device-scope
// streaming (the row kernels' st16_nt_at, wave-uniform tile base) or plain
// non-temporal.
template <int SC1>
__device__ __forceinline__ void store16(u32x4 *tile, int k, int t, u32x4 v) {
    if constexpr (SC1)
        ntk::st16_nt_at(reinterpret_cast<const char *>(tile), (uint32_t)(k * 256 * 16), (uint32_t)(t * 16),
                        make_uint4(v.x, v.y, v.z, v.w));
    else
        __builtin_nontemporal_store(v, tile + k * 256 + t);
}

template <int K, int SC1>
__global__ void __launch_bounds__(256) ntcal_copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                         int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * 256 * K + threadIdx.x;
    u32x4 v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t i = base + (int64_t)k * 256;
        v[k] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
    }
    u32x4 *tile = dst + (int64_t)blockIdx.x * 256 * K;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t i = base + (int64_t)k * 256;
        if (i < n16) store16<SC1>(tile, k, threadIdx.x, v[k]);
    }
}

template <int K>
__global__ void __launch_bounds__(256) ntcal_read_kernel(const u32x4 *__restrict__ src, uint32_t *__restrict__ out,
                                                         int64_t n16, uint32_t never) {
    const int64_t base = (int64_t)blockIdx.x * 256 * K + threadIdx.x;
    u32x4 v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t i = base + (int64_t)k * 256;
        v[k] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) acc += v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    if (acc == never) out[0] = acc;
}

template <int K, int SC1>
__global__ void __launch_bounds__(256) ntcal_fill_kernel(u32x4 *__restrict__ dst, int64_t n16, uint32_t val) {
    const int64_t base = (int64_t)blockIdx.x * 256 * K + threadIdx.x;
    const u32x4 v = {val, val, val, val};
    u32x4 *tile = dst + (int64_t)blockIdx.x * 256 * K;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t i = base + (int64_t)k * 256;
        if (i < n16) store16<SC1>(tile, k, threadIdx.x, v);
    }
}

template <int K>
hipError_t launch(int kind, int sc1, void *dst, const void *src, int64_t n16, uint32_t arg, hipStream_t s) {
    const int64_t grid = (n16 + 256 * K - 1) / (256 * K);
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    const dim3 g((uint32_t)grid), b(256);
    const u32x4 *in = static_cast<const u32x4 *>(src);
    u32x4 *out = static_cast<u32x4 *>(dst);
    void *a3[] = {&in, &out, &n16};
    uint32_t *out32 = static_cast<uint32_t *>(dst);
    void *ar[] = {&in, &out32, &n16, &arg};
    void *af[] = {&out, &n16, &arg};
    if (kind == 0)
        return hipLaunchKernel(sc1 ? reinterpret_cast<const void *>(ntcal_copy_kernel<K, 1>)
                                   : reinterpret_cast<const void *>(ntcal_copy_kernel<K, 0>),
                               g, b, a3, 0, s);
    if (kind == 1) return hipLaunchKernel(reinterpret_cast<const void *>(ntcal_read_kernel<K>), g, b, ar, 0, s);
    return hipLaunchKernel(sc1 ? reinterpret_cast<const void *>(ntcal_fill_kernel<K, 1>)
                               : reinterpret_cast<const void *>(ntcal_fill_kernel<K, 0>),
                           g, b, af, 0, s);
}
}  // namespace

// One reference stream over `bytes` (a multiple of 16; pointers 16-byte
// aligned): kind 0 copy src -> dst, 1 read src (dst: 4 writable bytes, written
// only if the folded value equals `arg`), 2 fill dst with `arg`.  K: 16-byte
// chunks per lane (1, 2, 4 or 8); sc1 != 0: device-scope streaming stores.
// Returns 0, -1 for invalid arguments, or the HIP error of the launch.
extern "C" int ntcal_stream(int kind, int K, int sc1, void *dst, const void *src, int64_t bytes, uint32_t arg,
                            void *stream) {
    if (kind < 0 || kind > 2 || bytes < 0 || bytes % 16 || !dst || (kind < 2 && !src) ||
        ((uintptr_t)dst | (uintptr_t)src) % 16)
        return -1;
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (K) {
    case 1: return (int)launch<1>(kind, sc1, dst, src, n16, arg, s);
    case 2: return (int)launch<2>(kind, sc1, dst, src, n16, arg, s);
    case 4: return (int)launch<4>(kind, sc1, dst, src, n16, arg, s);
    case 8: return (int)launch<8>(kind, sc1, dst, src, n16, arg, s);
    }
    return -1;
}

// The plain copy (one chunk per lane) with non-temporal stores (sc1 == 0) or
// device-scope streaming stores (sc1 != 0).
extern "C" int ntcal_copy_policy(void *dst, const void *src, int64_t bytes, int sc1, void *stream) {
    if (!src) return -1;
    return ntcal_stream(0, 1, sc1, dst, src, bytes, 0, stream);
}

extern "C" int ntcal_copy(void *dst, const void *src, int64_t bytes, void *stream) {
    return ntcal_copy_policy(dst, src, bytes, 0, stream);
}
