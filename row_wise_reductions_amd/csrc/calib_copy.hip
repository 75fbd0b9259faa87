// Plain device-to-device copy, used only as a reference: the bandwidth a
// simple streaming kernel reaches on this GPU, and the bytes the memory
// counters (FETCH_SIZE, WRITE_SIZE) report for a copy of known size.  Every
// 256-thread workgroup copies one contiguous 4 KiB tile with non-temporal
// 16-byte loads and stores.  A second kernel stores with the device-scope
// streaming policy (nt sc1) that the row kernels use: the ceiling they meet.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) ntcal_copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                         int64_t n16) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ void __launch_bounds__(256) ntcal_copy_sc1_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                             int64_t n16) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        // s_nop 1: no VALU may overwrite the data registers within 2 wait states.
        asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" : : "v"(dst + i), "v"(v) : "memory");
    }
}
}  // namespace

// Copies `bytes` (a multiple of 16, both pointers 16-byte aligned) on
// `stream`; `sc1` != 0 selects the device-scope streaming stores.  Returns 0,
// or -1 for invalid arguments, or the HIP error code.
extern "C" int ntcal_copy_policy(void *dst, const void *src, int64_t bytes, int sc1, void *stream) {
    if (!dst || !src || bytes < 0 || bytes % 16 || ((uintptr_t)dst | (uintptr_t)src) % 16) return -1;
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    const int64_t grid = (n16 + 255) / 256;
    if (grid > INT32_MAX) return -1;
    hipLaunchKernelGGL(sc1 ? ntcal_copy_sc1_kernel : ntcal_copy_kernel, dim3((uint32_t)grid), dim3(256), 0,
                       (hipStream_t)stream, (const u32x4 *)src, (u32x4 *)dst, n16);
    return (int)hipGetLastError();
}

// ntcal_copy_policy with non-temporal stores.
extern "C" int ntcal_copy(void *dst, const void *src, int64_t bytes, void *stream) {
    return ntcal_copy_policy(dst, src, bytes, 0, stream);
}
