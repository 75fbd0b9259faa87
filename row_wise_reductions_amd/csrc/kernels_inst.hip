// Instantiation of the row kernels for one element type, selected at build
// time with -DNTK_DT=0 (fp32), 1 (fp16) or 2 (bf16).
#include <atomic>

#include "launch.hpp"

#ifndef NTK_DT
#error "NTK_DT must be defined"
#endif

namespace ntk {
namespace {

constexpr int DT = NTK_DT;
// fp32 holds 4 values per chunk, 16-bit types 8.
constexpr bool kWide = dt_info<DT>::VEC == 4;

// Launch a row kernel; the status is the one the launch call returns (the
// thread's last-error state is neither read nor cleared).
hipError_t launch_k(void (*k)(RowArgs), int64_t grid, int threads, hipStream_t s, RowArgs a) {
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), dim3((uint32_t)grid), dim3((uint32_t)threads), args, 0,
                           s);
}

template <int OP, int W, int K, bool PR, bool RES>
hipError_t go_pr(bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    constexpr int T = GroupShape<W>::THREADS;
    return al ? launch_k(row_resident<OP, DT, W, K, true, PR, RES>, grid, T, s, a)
              : launch_k(row_resident<OP, DT, W, K, false, PR, RES>, grid, T, s, a);
}

// Values a lane holds for one row: LayerNorm keeps at most 16 (its fp64
// arithmetic needs twice the registers) except 32 at 5 to 8 waves (rows of up
// to 16384 elements in one pass; 320- to 512-thread workgroups leave a wave
// 256 registers; the persistent fp32 form would spill and is not built), RMSNorm
// and softmax 64, and a fused residual add (which also
// holds the residual's words) 32.  Wider shapes would spill registers and are
// not built.
template <int OP, int K, bool RES = false, int W = 0>
constexpr bool shape_built() {
    constexpr int V = K * dt_info<DT>::VEC;
    // LayerNorm is never planned with more than 12 waves per row
    return OP == OP_LAYERNORM ? ((V <= 16 || (W >= 5 && W <= 8 && V == 32)) && W <= 12) : V <= (RES ? 32 : 64);
}

// Norms with every parameter vector present take the specialised PR kernel;
// a residual input (a.r) selects the fused add + norm kernel.
template <int OP, int W, int K>
hipError_t go(bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    if constexpr (OP == OP_SOFTMAX || OP == OP_SOFTMAX_CAUSAL) {
        return go_pr<OP, W, K, false, false>(al, a, grid, s);
    } else {
        const bool pr = a.p0 != nullptr && (OP == OP_RMSNORM || a.p1 != nullptr);
        if (a.r) {
            if constexpr (shape_built<OP, K, true, W>())
                return pr ? go_pr<OP, W, K, true, true>(al, a, grid, s) : go_pr<OP, W, K, false, true>(al, a, grid, s);
            return hipErrorInvalidValue;
        }
        return pr ? go_pr<OP, W, K, true, false>(al, a, grid, s) : go_pr<OP, W, K, false, false>(al, a, grid, s);
    }
}

template <int OP>
hipError_t resident(int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    // A 1024-thread workgroup caps a wave at 128 registers: W = 16 is built
    // only with one or two chunks per lane.
#define NTK_CASE(w, k)                                          \
    if (W == w && K == k) {                                     \
        if constexpr (shape_built<OP, k, false, w>()) return go<OP, w, k>(al, a, grid, s); \
        return hipErrorInvalidValue;                            \
    }
    NTK_CASE(1, 1) NTK_CASE(1, 2) NTK_CASE(1, 4) NTK_CASE(1, 8) NTK_CASE(1, 16)
    NTK_CASE(2, 2) NTK_CASE(2, 4) NTK_CASE(2, 8) NTK_CASE(4, 1) NTK_CASE(4, 2) NTK_CASE(4, 4) NTK_CASE(4, 8)
    NTK_CASE(8, 1) NTK_CASE(8, 2) NTK_CASE(8, 4) NTK_CASE(8, 8) NTK_CASE(8, 16)
    NTK_CASE(16, 1) NTK_CASE(16, 2)
    // LayerNorm's shapes between powers of two: 16-bit 7 x 2 and 5..7 x 4,
    // fp32 12 x 4 (768 threads: a wave keeps up to 170 registers)
    if constexpr (OP == OP_LAYERNORM && !kWide) {
        NTK_CASE(7, 2) NTK_CASE(5, 4) NTK_CASE(6, 4) NTK_CASE(7, 4)
    }
    if constexpr (OP == OP_LAYERNORM && kWide) {
        NTK_CASE(12, 4)
    }
#undef NTK_CASE
    return hipErrorInvalidValue;
}

// Persistent norm kernel on `grid` workgroups (the plan's k per compute
// unit, never more than there are rows), at most as many as fit on the
// device at once when `cap_cus` > 0 (occupancy x `cap_cus` compute units, the
// occupancy cached per instantiation).  The grid stays a multiple of the CU
// count: uneven grids leave some CUs a row more than others (7-10% slower).
template <int OP, int W, int K, bool RES>
hipError_t persist_go(const RowArgs &a, hipStream_t s, int64_t grid, int cap_cus) {
    if (cap_cus > 0) {
        static std::atomic<int> per_cu{0};
        int pc = per_cu.load(std::memory_order_relaxed);
        if (pc == 0) {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, row_norm_persistent<OP, DT, W, K, RES>, 64 * W, 0) !=
                    hipSuccess || n <= 0)
                n = 1;
            per_cu.store(n, std::memory_order_relaxed);
            pc = n;
        }
        if (grid > (int64_t)pc * cap_cus) grid = (int64_t)pc * cap_cus;
    }
    if (grid > a.M) grid = a.M;
    if (grid < 1) grid = 1;
    return launch_k(row_norm_persistent<OP, DT, W, K, RES>, grid, 64 * W, s, a);
}

// The persistent kernel is planned for LayerNorm (plain, and fused with the
// residual add), plain 16-bit RMSNorm and fp32 RMSNorm at 8 waves x 8
// chunks; other norms stream faster one row per workgroup, and their
// persistent forms are not built.
template <int OP, int W, int K>
hipError_t persist_pick(const RowArgs &a, hipStream_t s, int64_t grid, int cap) {
    if (a.r) {
        if constexpr (OP == OP_LAYERNORM) return persist_go<OP, W, K, true>(a, s, grid, cap);
        return hipErrorInvalidValue;
    }
    if constexpr (OP == OP_LAYERNORM || !kWide || (W == 8 && K == 8)) return persist_go<OP, W, K, false>(a, s, grid, cap);
    return hipErrorInvalidValue;
}

template <int OP>
hipError_t persistent(int W, int K, const RowArgs &a, hipStream_t s, int64_t grid, int cap) {
#define NTK_CASE(w, k)                                                   \
    if (W == w && K == k) {                                              \
        if constexpr (shape_built<OP, k, false, w>() && k * dt_info<DT>::VEC <= 32 &&                       \
                      !(OP == OP_LAYERNORM && kWide && k * dt_info<DT>::VEC > 16))                        \
            return persist_pick<OP, w, k>(a, s, grid, cap);                                               \
        return hipErrorInvalidValue;                                     \
    }
    NTK_CASE(2, 2) NTK_CASE(2, 4) NTK_CASE(2, 8) NTK_CASE(4, 1) NTK_CASE(4, 2) NTK_CASE(4, 4) NTK_CASE(4, 8)
    NTK_CASE(8, 1) NTK_CASE(8, 2) NTK_CASE(8, 4) NTK_CASE(8, 8) NTK_CASE(8, 16)
    if constexpr (OP == OP_LAYERNORM && !kWide) {
        NTK_CASE(7, 2) NTK_CASE(5, 4) NTK_CASE(6, 4) NTK_CASE(7, 4)
    }
#undef NTK_CASE
    return hipErrorInvalidValue;
}

hipError_t persistent_any(int op, int W, int K, const RowArgs &a, hipStream_t s, int64_t grid, int cap) {
    switch (op) {
    case OP_LAYERNORM: return persistent<OP_LAYERNORM>(W, K, a, s, grid, cap);
    case OP_RMSNORM: return persistent<OP_RMSNORM>(W, K, a, s, grid, cap);
    }
    return hipErrorInvalidValue;
}

template <int OP>
hipError_t looped(int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    if (W == 8 && K == 4) {
        if (a.r)
            return al ? launch_k(row_looped<OP, DT, 8, 4, true, true>, grid, 512, s, a)
                      : launch_k(row_looped<OP, DT, 8, 4, false, true>, grid, 512, s, a);
        return al ? launch_k(row_looped<OP, DT, 8, 4, true, false>, grid, 512, s, a)
                  : launch_k(row_looped<OP, DT, 8, 4, false, false>, grid, 512, s, a);
    }
    return hipErrorInvalidValue;
}

// coop: 0 the two kernels, 1 the cooperative kernel, 2 the cooperative
// kernel with two rows per workgroup
template <int W, int K, bool AL, bool CAUSAL>
hipError_t split_al(int coop, const RowArgs &a, hipStream_t s) {
    const int64_t grid = a.M * a.P;
    if (coop == 2) return launch_k(softmax_coop2<DT, W, K, AL, CAUSAL>, (a.M + 1) / 2 * a.P, 64 * W, s, a);
    if (coop) return launch_k(softmax_coop<DT, W, K, AL, CAUSAL>, grid, 64 * W, s, a);
    const hipError_t e = launch_k(softmax_split_partial<DT, W, K, AL, CAUSAL>, grid, 64 * W, s, a);
    if (e != hipSuccess) return e;
    return launch_k(softmax_split_finalize<DT, W, K, AL, CAUSAL>, grid, 64 * W, s, a);
}

// The causal split kernels are built for the planner's split shapes only:
// the cooperative ones (fp32 8 x 8, 16-bit 4 x 8) and the wide (4, 4).
template <int W, int K>
constexpr bool causal_split_built() {
    return (kWide ? (W == 8 && K == 8) : (W == 4 && K == 8)) || (W == 4 && K == 4);
}

template <int W, int K>
hipError_t split_go(bool al, int coop, const RowArgs &a, hipStream_t s) {
    if (a.queries > 0) {
        if constexpr (causal_split_built<W, K>())
            return al ? split_al<W, K, true, true>(coop, a, s) : split_al<W, K, false, true>(coop, a, s);
        return hipErrorInvalidValue;
    }
    return al ? split_al<W, K, true, false>(coop, a, s) : split_al<W, K, false, false>(coop, a, s);
}

hipError_t split(int W, int K, bool al, int coop, const RowArgs &a, hipStream_t s) {
#define NTK_CASE(w, k) \
    if (W == w && K == k) return split_go<w, k>(al, coop, a, s);
    NTK_CASE(4, 1) NTK_CASE(4, 2) NTK_CASE(4, 4) NTK_CASE(4, 8) NTK_CASE(8, 1) NTK_CASE(8, 2) NTK_CASE(8, 4)
    NTK_CASE(8, 8)
    if constexpr (kWide) {
        NTK_CASE(4, 16) NTK_CASE(8, 16)
    }
#undef NTK_CASE
    return hipErrorInvalidValue;
}

template <int OP, int W, int K, bool AL>
hipError_t norm_split_go(bool coop, const RowArgs &a, hipStream_t s) {
    const int64_t grid = a.M * a.P;
    if (coop) {
        // the one-pass form is planned for 8 x 4 chunks, not for 16-bit
        // LayerNorm, and in fp32 also 8 x 8
        if constexpr ((W == 8 && K == 4 && !(OP == OP_LAYERNORM && DT != DT_F32)) ||
                      (DT == DT_F32 && W == 8 && K == 8))
            return launch_k(norm_coop<OP, DT, W, K, AL>, grid, 64 * W, s, a);
        return hipErrorInvalidValue;
    }
    const hipError_t e = launch_k(norm_split_partial<OP, DT, W, K, AL>, grid, 64 * W, s, a);
    if (e != hipSuccess) return e;
    return launch_k(norm_split_finalize<OP, DT, W, K, AL>, grid, 64 * W, s, a);
}

// The split norm's chunk shapes: 8 waves x 4 chunks (32 KiB), 8 x 1, 4 x 1 (two kernels); 8 x 4 in one pass,
// and fp32 8 x 8 (64 KiB) in one pass or, in place or under capture, in two kernels.
template <int OP>
hipError_t norm_split(int W, int K, bool al, bool coop, const RowArgs &a, hipStream_t s) {
#define NTK_CASE(w, k) \
    if (W == w && K == k) \
        return al ? norm_split_go<OP, w, k, true>(coop, a, s) : norm_split_go<OP, w, k, false>(coop, a, s);
    NTK_CASE(8, 4) NTK_CASE(8, 1) NTK_CASE(4, 1)
    if constexpr (DT == DT_F32) {
        NTK_CASE(8, 8)     // the one-pass plan's chunks, in two kernels in place or under capture
    }
#undef NTK_CASE
    return hipErrorInvalidValue;
}

hipError_t norm_split_any(int op, int W, int K, bool al, bool coop, const RowArgs &a, hipStream_t s) {
    switch (op) {
    case OP_LAYERNORM: return norm_split<OP_LAYERNORM>(W, K, al, coop, a, s);
    case OP_RMSNORM: return norm_split<OP_RMSNORM>(W, K, al, coop, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t looped_any(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    switch (op) {
    case OP_LAYERNORM: return looped<OP_LAYERNORM>(W, K, al, a, grid, s);
    case OP_RMSNORM: return looped<OP_RMSNORM>(W, K, al, a, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t resident_any(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    switch (op) {
    case OP_SOFTMAX: return resident<OP_SOFTMAX>(W, K, al, a, grid, s);
    case OP_LAYERNORM: return resident<OP_LAYERNORM>(W, K, al, a, grid, s);
    case OP_RMSNORM: return resident<OP_RMSNORM>(W, K, al, a, grid, s);
    case OP_SOFTMAX_CAUSAL: return resident<OP_SOFTMAX_CAUSAL>(W, K, al, a, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

#if NTK_DT == 0
hipError_t launch_resident_f32(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    return resident_any(op, W, K, al, a, grid, s);
}
hipError_t launch_split_f32(int W, int K, bool al, int coop, const RowArgs &a, hipStream_t s) {
    return split(W, K, al, coop, a, s);
}
hipError_t launch_looped_f32(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    return looped_any(op, W, K, al, a, grid, s);
}
hipError_t launch_persistent_f32(int op, int W, int K, const RowArgs &a, hipStream_t s, int64_t grid,
                                 int cap_cus) {
    return persistent_any(op, W, K, a, s, grid, cap_cus);
}
hipError_t launch_norm_split_f32(int op, int W, int K, bool al, bool coop, const RowArgs &a, hipStream_t s) {
    return norm_split_any(op, W, K, al, coop, a, s);
}
#elif NTK_DT == 1
hipError_t launch_resident_f16(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    return resident_any(op, W, K, al, a, grid, s);
}
hipError_t launch_split_f16(int W, int K, bool al, int coop, const RowArgs &a, hipStream_t s) {
    return split(W, K, al, coop, a, s);
}
hipError_t launch_looped_f16(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    return looped_any(op, W, K, al, a, grid, s);
}
hipError_t launch_persistent_f16(int op, int W, int K, const RowArgs &a, hipStream_t s, int64_t grid,
                                 int cap_cus) {
    return persistent_any(op, W, K, a, s, grid, cap_cus);
}
hipError_t launch_norm_split_f16(int op, int W, int K, bool al, bool coop, const RowArgs &a, hipStream_t s) {
    return norm_split_any(op, W, K, al, coop, a, s);
}
#else
hipError_t launch_resident_bf16(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    return resident_any(op, W, K, al, a, grid, s);
}
hipError_t launch_split_bf16(int W, int K, bool al, int coop, const RowArgs &a, hipStream_t s) {
    return split(W, K, al, coop, a, s);
}
hipError_t launch_looped_bf16(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s) {
    return looped_any(op, W, K, al, a, grid, s);
}
hipError_t launch_persistent_bf16(int op, int W, int K, const RowArgs &a, hipStream_t s, int64_t grid,
                                 int cap_cus) {
    return persistent_any(op, W, K, a, s, grid, cap_cus);
}
hipError_t launch_norm_split_bf16(int op, int W, int K, bool al, bool coop, const RowArgs &a, hipStream_t s) {
    return norm_split_any(op, W, K, al, coop, a, s);
}
#endif

}  // namespace ntk
