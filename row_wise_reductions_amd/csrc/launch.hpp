// Host-side launchers of the row kernels (defined in kernels_inst.hip, one
// translation unit per element type so they compile in parallel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "row_kernels.hpp"

namespace ntk {

// Launch the single-pass kernel for (op, dt) with W waves per row and K
// 16-byte chunks per lane.  Returns hipErrorInvalidValue for a (W, K) pair
// that is not instantiated.
hipError_t launch_resident_f32(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_resident_f16(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_resident_bf16(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s);

// Launch the looped one-workgroup-per-row kernel (LayerNorm / RMSNorm rows
// wider than the single-pass shapes).
hipError_t launch_looped_f32(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_looped_f16(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_looped_bf16(int op, int W, int K, bool al, const RowArgs &a, int64_t grid, hipStream_t s);

// Launch the persistent norm kernel (aligned rows, every parameter vector
// present) on `grid` workgroups, capped at what fits on the device at once
// on `cap_cus` compute units when that is > 0.
hipError_t launch_persistent_f32(int op, int W, int K, const RowArgs &a, hipStream_t s, int64_t grid, int cap_cus);
hipError_t launch_persistent_f16(int op, int W, int K, const RowArgs &a, hipStream_t s, int64_t grid, int cap_cus);
hipError_t launch_persistent_bf16(int op, int W, int K, const RowArgs &a, hipStream_t s, int64_t grid, int cap_cus);

// Launch the split softmax: with `coop` 1, the one cooperative kernel
// (a.P <= COOP_PMAX, x not aliasing y, a.tag unique to the call); with 2,
// the cooperative kernel with two rows per workgroup; with 0, the two
// kernels (partials, then merge + write).
hipError_t launch_split_f32(int W, int K, bool al, int coop, const RowArgs &a, hipStream_t s);
hipError_t launch_split_f16(int W, int K, bool al, int coop, const RowArgs &a, hipStream_t s);
hipError_t launch_split_bf16(int W, int K, bool al, int coop, const RowArgs &a, hipStream_t s);

// Launch the split norm (rows too wide for one pass, cut into a.P chunks of
// 64*W*K 16-byte pieces, one workgroup per (row, chunk)): with `coop` the
// one-pass kernel (a.wsd holds four tagged 64-bit words per (row, chunk);
// a.tag, a.spin set), else the partial kernel, then the finalize kernel
// (a.wsd holds 2 doubles per (row, chunk), then a pivot per row).
hipError_t launch_norm_split_f32(int op, int W, int K, bool al, bool coop, const RowArgs &a, hipStream_t s);
hipError_t launch_norm_split_f16(int op, int W, int K, bool al, bool coop, const RowArgs &a, hipStream_t s);
hipError_t launch_norm_split_bf16(int op, int W, int K, bool al, bool coop, const RowArgs &a, hipStream_t s);

}  // namespace ntk
