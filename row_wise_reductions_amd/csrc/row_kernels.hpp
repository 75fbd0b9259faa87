// Fused row-reduction kernels for gfx950 (MI355X, CDNA4, wave64).
//
// One row (or, on the split path, one chunk of a row) is owned by a group of
// W waves.  The row is read from HBM once with 16-byte vector loads, held in
// VGPRs, reduced (lane-serial, then a 64-lane DPP butterfly, then an LDS
// combine across the group's waves), transformed and written back once with
// 16-byte stores.  The data layout is the group-cyclic one described in
// "Rebuilding Triton and Helion from Scratch in 4,000 Lines of Python",
// section "The register layout": the row is cut into 16-byte chunks and chunk
// c belongs to lane c mod (64*W), so a wave-wide load covers 1 KiB of
// consecutive bytes.  The three-level reduction shape (registers, wave,
// cross-wave through LDS with a broadcast back) is the one of section
// "Reductions and broadcasting", rebuilt for 64-lane waves and DPP.
//
// Masked tails use the identities of "Portable Triton Kernels" ("Hard
// Constraints", "Safe Softmax Pattern"): -inf for the max, so exp() of a
// padding lane is exactly 0, and 0 for sums.
//
// Two variants of most kernels exist:
//   AL = true   every row start, x, y and the parameter vectors are 16-byte
//               aligned and N*sizeof(T) is a multiple of 16: whole chunks only.
//   AL = false  rows start anywhere (element-aligned).  Chunks are cut on the
//               16-byte grid of x; the partial first and last chunk of a row
//               are gathered and scattered element by element, and the
//               parameter vectors are read per element.
//
// Kernels:
//   row_resident          one row per group of W waves (W = 1: 4 rows per
//                         workgroup): softmax, causal softmax, LayerNorm,
//                         RMSNorm, and the fused residual add + norm (RES)
//   row_norm_persistent   norms with the parameters held in registers across
//                         rows and the next row prefetched (aligned rows)
//   row_looped            norms of rows too wide for registers (two passes)
//   softmax_coop          split softmax in one pass: the workgroups of a row
//                         exchange (max, denominator) records
//   softmax_split_partial / softmax_split_finalize
//                         the same split softmax in two kernels
//   norm_coop             split LayerNorm / RMSNorm in one pass: the
//                         workgroups of a row exchange fp64 sum records
//   norm_split_partial / norm_split_finalize
//                         the same split norm in two kernels
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ntk {

enum { OP_SOFTMAX = 0, OP_LAYERNORM = 1, OP_RMSNORM = 2, OP_SOFTMAX_CAUSAL = 3 };
enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT> struct dt_info;
template <> struct dt_info<DT_F32> {
    static constexpr int E = 4, VEC = 4;
    static constexpr uint32_t NEG_INF_WORD = 0xFF800000u;
};
template <> struct dt_info<DT_F16> {
    static constexpr int E = 2, VEC = 8;
    static constexpr uint32_t NEG_INF_WORD = 0xFC00FC00u;
};
template <> struct dt_info<DT_BF16> {
    static constexpr int E = 2, VEC = 8;
    static constexpr uint32_t NEG_INF_WORD = 0xFF80FF80u;
};

// Arguments of every row kernel (passed by value as the kernarg segment).
struct RowArgs {
    const char *x;
    char *y;
    const char *r;       // fused add + norm: residual input (null otherwise)
    char *h;             // fused add + norm: h = x + r output
    const char *p0;      // gamma (LayerNorm) or weight (RMSNorm); may be null
    const char *p1;      // beta (LayerNorm); may be null
    float *mean;         // LayerNorm statistics outputs; may be null
    float *rstd;
    float2 *ws;          // split softmax: (max, denominator) per (row, chunk)
    double *wsd;         // split norm: (sum(x - p), sum((x - p)^2)) per (row, chunk)
    double inv_nd;       // 1/N in fp64
    int64_t M;
    int32_t N;
    int32_t P;           // split softmax: chunks per row
    float eps;
    float inv_n;         // 1/N in fp32
    uint32_t tag;        // cooperative split kernels: this call's record tag
    int32_t spin;        // cooperative split softmax: polls before recomputing
    int64_t queries;     // causal softmax: row r is query r mod queries (0: not causal)
    int64_t offset;      // causal softmax: query q sees keys k <= q + offset
    float s2;            // causal softmax: scale * log2(e), rounded to fp32
    const uint32_t *tagp; // cooperative split kernels: when set, the record tag is read
                          // from this device word (calls captured into a graph)
};

// The record tag of a cooperative split launch: the host's per-call value,
// or, for a call captured into a graph, the device word that a one-thread
// kernel ahead of it in the stream increments, so that each replay tags its
// records afresh.  Every workgroup reads the same value.
__device__ __forceinline__ uint32_t call_tag(const struct RowArgs &a) {
    if (a.tagp) return __hip_atomic_load(a.tagp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return a.tag;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// 16-byte chunk <-> fp32 values
// ---------------------------------------------------------------------------

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Build-time memory-policy switches (see ld16_nt, st16_nt and xcd_band).
// Measured on MI355X: streaming loads and stores together add 6-35% on the
// row kernels; XCD banding helps some shapes and costs others up to 8%, so
// it is off.
#ifndef NTK_NT_LOADS
#define NTK_NT_LOADS 1
#endif
#ifndef NTK_NT_STORES
#define NTK_NT_STORES 1
#endif
// Streaming stores at device scope (nt sc1): measured on MI355X, a 1 GiB copy
// runs 3% faster than with plain non-temporal stores.
#ifndef NTK_STORE_SC1
#define NTK_STORE_SC1 1
#endif
#ifndef NTK_XCD_BAND
#define NTK_XCD_BAND 0
#endif

__device__ __forceinline__ uint4 ld16(const char *p) {
    return *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ void st16(char *p, uint4 v) {
    *reinterpret_cast<uint4 *>(p) = v;
}
// Streaming (non-temporal) 16-byte load and store for row data that is
// touched once: they keep single-use lines from displacing reused ones
// (the parameter vectors) and measurably raise read+write HBM throughput.
__device__ __forceinline__ uint4 ld16_nt(const char *p) {
#if NTK_NT_LOADS
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
#else
    return ld16(p);
#endif
}
// Wait until this wave's own stores have completed: s_waitcnt vmcnt(0)
// (gfx9 encoding: vmcnt 0, expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_own_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Cache-policy operand of the buffer store for "nt sc1": bit 1 streaming
// (non-temporal), bit 4 device scope (the store writes through the XCD's L2).
constexpr int CPOL_NT_SC1 = (1 << 1) | (1 << 4);

// Streaming store of one 16-byte chunk to base + soff + voff.  `base` is the
// same for every lane of the wave (a row's or a chunk's start), `soff` a
// wave-uniform byte offset and `voff` the lane's own one; soff + voff must
// stay below 2^32 - 16.  With device-scope streaming stores this is a raw
// buffer store, which the compiler sees (it keeps the store's hazards and
// wait counts itself): the buffer resource is built from `base` in scalar
// registers (readfirstlane, which folds away when the compiler already
// knows the value is uniform), `soff` goes to the scalar offset and only
// `voff` is per lane, so the address costs no vector instruction per store.
// The range check is effectively off (2^32 - 1 bytes).
__device__ __forceinline__ void st16_nt_at(const char *base, uint32_t soff, uint32_t voff, uint4 v) {
    const u32x4 t = {v.x, v.y, v.z, v.w};
#if NTK_NT_STORES && NTK_STORE_SC1
    const uint64_t pa = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)pa);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(pa >> 32));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>((((uint64_t)hi) << 32) | lo), 0, (int)0xFFFFFFFFu, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(t, rs, (int)voff, (int)soff, CPOL_NT_SC1);
#elif NTK_NT_STORES
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(const_cast<char *>(base) + soff + voff));
#else
    st16(const_cast<char *>(base) + soff + voff, v);
#endif
}

// Streaming store of one 16-byte chunk at base + voff that writes nothing
// when voff + 16 > bytes: the buffer resource's range is [base, base +
// bytes) and the buffer unit discards out-of-range stores, so lanes past
// the row need no branch around their store.  Every lane then issues the
// same stores on every path, and the compiler can wait for an earlier load
// (the next row's, in the persistent kernel) without waiting for these
// stores to complete.  `base` is wave-uniform, `bytes` a multiple of 16.
__device__ __forceinline__ void st16_nt_bounded(const char *base, uint32_t bytes, uint32_t voff, uint4 v) {
#if NTK_NT_STORES && NTK_STORE_SC1
    const u32x4 t = {v.x, v.y, v.z, v.w};
    const uint64_t pa = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)pa);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(pa >> 32));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>((((uint64_t)hi) << 32) | lo), 0, (int)bytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(t, rs, (int)voff, 0, CPOL_NT_SC1);
#else
    if (voff + 16 <= bytes) st16_nt_at(base, 0, voff, v);
#endif
}

// One fp32 value at p + voff, written only where voff + 4 <= bytes (a
// buffer store with that range; bytes = 0 writes nothing, p may then be
// null).  A plain (cached) store: the per-row statistics.
__device__ __forceinline__ void st4_bounded(const float *p, uint32_t bytes, uint32_t voff, float v) {
    const uint64_t pa = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)pa);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(pa >> 32));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>((((uint64_t)hi) << 32) | lo), 0, (int)bytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, (int)voff, 0, 0);
}

// Workgroups are dealt round-robin to the 8 XCDs (workgroup b runs on XCD
// b mod 8).  Renumbering so that XCD x receives a contiguous band of row
// blocks gives each XCD's L2 and memory queues a sequential stream.
__device__ __forceinline__ int64_t xcd_band(int64_t b, int64_t G) {
#if NTK_XCD_BAND
    return (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
#else
    (void)G;
    return b;
#endif
}

template <int DT>
__device__ __forceinline__ void unpack(uint4 r, float (&f)[dt_info<DT>::VEC]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __builtin_bit_cast(float, w[i]);
    } else if constexpr (DT == DT_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2 p = __builtin_convertvector(__builtin_bit_cast(f16x2, w[i]), f32x2);
            f[2 * i] = p.x;
            f[2 * i + 1] = p.y;
        }
    } else {
        // bf16 is the top half of a binary32: the widening is a shift, but
        // written as a conversion the compiler knows the result is a
        // canonical float and needs no quieting before v_max.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2 p = __builtin_convertvector(__builtin_bit_cast(bf16x2, w[i]), f32x2);
            f[2 * i] = p.x;
            f[2 * i + 1] = p.y;
        }
    }
}

// fp32 -> storage type, round to nearest even (v_cvt_f16_f32 and
// v_cvt_pk_bf16_f32 both round to nearest even in the default mode).
template <int DT>
__device__ __forceinline__ uint4 pack(const float (&f)[dt_info<DT>::VEC]) {
    uint32_t w[4];
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __builtin_bit_cast(uint32_t, f[i]);
    } else if constexpr (DT == DT_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2 p = {f[2 * i], f[2 * i + 1]};
            w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, f16x2));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2 p = {f[2 * i], f[2 * i + 1]};
            w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Element-granular gather of the chunk whose first column is col0 (may be
// negative or run past N); columns outside [0, N) take the fill pattern.
template <int DT>
__device__ __forceinline__ uint4 gather(const char *row, int64_t col0, int32_t N, uint32_t fill) {
    uint32_t w[4];
    if constexpr (dt_info<DT>::E == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t c = col0 + i;
            w[i] = (c >= 0 && c < N) ? reinterpret_cast<const uint32_t *>(row)[c] : fill;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t c = col0 + 2 * i;
            const uint32_t lo = (c >= 0 && c < N) ? reinterpret_cast<const uint16_t *>(row)[c] : (fill & 0xFFFFu);
            const uint32_t hi = (c + 1 >= 0 && c + 1 < N) ? reinterpret_cast<const uint16_t *>(row)[c + 1] : (fill >> 16);
            w[i] = lo | (hi << 16);
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Element-granular store of the in-row columns of a chunk.
template <int DT>
__device__ __forceinline__ void scatter(char *row, int64_t col0, int32_t N, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (dt_info<DT>::E == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t c = col0 + i;
            if (c >= 0 && c < N) reinterpret_cast<uint32_t *>(row)[c] = w[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t c = col0 + i;
            if (c >= 0 && c < N)
                reinterpret_cast<uint16_t *>(row)[c] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
        }
    }
}

// ---------------------------------------------------------------------------
// Wave64 all-reduce: DPP butterfly inside each 16-lane row (xor 1, xor 2,
// half-row mirror, row mirror), then the four row totals are read into
// scalars and combined in a fixed order.  Every lane returns the same bits.
// ---------------------------------------------------------------------------

// Every permutation used below reads a valid lane for every lane, so the
// "old" operand is never observed.  For fp32 the zero-old form lets the
// compiler fold the DPP into the consuming v_add/v_max; the fp64 halves use
// bound_ctrl moves, which need no initialized destination.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = dpp_mov<CTRL>((int)(uint32_t)u);
    const int hi = dpp_mov<CTRL>((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
template <int CTRL>
__device__ __forceinline__ double2 dpp(double2 v) {
    return double2{dpp<CTRL>(v.x), dpp<CTRL>(v.y)};
}
__device__ __forceinline__ float readlane(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ double readlane(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane(double v, int l);
__device__ __forceinline__ double2 readlane(double2 v, int l) {
    return double2{readlane(v.x, l), readlane(v.y, l)};
}

struct SumOp {
    template <class V> __device__ __forceinline__ V operator()(V a, V b) const { return a + b; }
    __device__ __forceinline__ double2 operator()(double2 a, double2 b) const {
        return double2{a.x + b.x, a.y + b.y};
    }
};
struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return __builtin_fmaxf(a, b); }
};

template <class V, class Op>
__device__ __forceinline__ V wave_allreduce(V v, Op op) {
    v = op(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]: lane ^ 1
    v = op(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]: lane ^ 2
    v = op(v, dpp<0x141>(v));   // row_half_mirror: other quad of the 8-lane half
    v = op(v, dpp<0x140>(v));   // row_mirror: other half of the 16-lane row
    const V r0 = readlane(v, 0), r1 = readlane(v, 16), r2 = readlane(v, 32), r3 = readlane(v, 48);
    return op(op(r0, r1), op(r2, r3));
}

// All-reduce over the W waves of a row group.  `slot` points at W entries
// of LDS owned by this reduction; the caller guarantees that no other wave
// can still be reading them (distinct slots per reduction and per parity of
// the row-loop iteration).
template <int W, class V, class Op>
__device__ __forceinline__ V group_allreduce(V v, Op op, V *slot, int wv, int lane) {
    v = wave_allreduce(v, op);
    if constexpr (W == 1) {
        return v;
    } else {
        if (lane == 0) slot[wv] = v;
        __syncthreads();
        V r = slot[0];
#pragma unroll
        for (int i = 1; i < W; ++i) r = op(r, slot[i]);
        return r;
    }
}

// ---------------------------------------------------------------------------
// Row geometry: which 16-byte chunks of the row a lane owns.
// ---------------------------------------------------------------------------

template <int DT, bool AL>
struct RowGeom {
    const char *xb;    // 16-byte aligned address of chunk 0
    int64_t nch;       // chunks touched by the row
    int32_t head;      // elements of chunk 0 that precede the row (AL: 0)

    __device__ __forceinline__ RowGeom(const char *xr, int32_t N) {
        constexpr int E = dt_info<DT>::E, VEC = dt_info<DT>::VEC;
        if constexpr (AL) {
            head = 0;
            nch = ((int64_t)N * E) >> 4;
        } else {
            head = (int32_t)(((uintptr_t)xr & 15) / E);
            nch = ((int64_t)head + N + VEC - 1) / VEC;
        }
        xb = xr - (int64_t)head * E;
    }
    __device__ __forceinline__ int64_t col0(int64_t c) const {
        return c * dt_info<DT>::VEC - head;
    }
    __device__ __forceinline__ bool full(int64_t c, int32_t N) const {
        if constexpr (AL) return c < nch;
        const int64_t c0 = col0(c);
        return c0 >= 0 && c0 + dt_info<DT>::VEC <= N;
    }
};

// Load the chunk c of a row (identity `fill` outside the row).
template <int DT, bool AL>
__device__ __forceinline__ uint4 load_chunk(const RowGeom<DT, AL> &g, const char *xr, int64_t c,
                                            int32_t N, uint32_t fill) {
    if (c < g.nch) {
        if constexpr (AL) {
            return ld16(g.xb + c * 16);
        } else {
            if (g.full(c, N)) return ld16(g.xb + c * 16);
            return gather<DT>(xr, g.col0(c), N, fill);
        }
    }
    return make_uint4(fill, fill, fill, fill);
}

// Load the parameter-vector chunk that lines up with row chunk c.
template <int DT, bool AL>
__device__ __forceinline__ uint4 load_param(const RowGeom<DT, AL> &g, const char *p, int64_t c,
                                            int32_t N) {
    if constexpr (AL) {
        if (c < g.nch) return ld16(p + c * 16);
        return make_uint4(0, 0, 0, 0);
    } else {
        if (c < g.nch) return gather<DT>(p, g.col0(c), N, 0u);
        return make_uint4(0, 0, 0, 0);
    }
}

// Store chunk c = cbase + k*TPR + t of a row (the k-th slice of lane t,
// from chunk cbase on).  `yvec` tells whether y shares x's 16-byte phase
// (then whole chunks are stored as vectors).
template <int DT, bool AL, int TPR>
__device__ __forceinline__ void store_chunk(const RowGeom<DT, AL> &g, char *yr, int64_t cbase, int k, int t,
                                            int32_t N, bool yvec, uint4 v) {
    const int64_t c = cbase + (int64_t)k * TPR + t;
    if (c < g.nch) {
        if constexpr (AL) {
            st16_nt_at(yr + cbase * 16, (uint32_t)(k * TPR * 16), (uint32_t)(t * 16), v);
        } else {
            if (yvec && g.full(c, N))
                st16_nt_at(yr - (int64_t)g.head * dt_info<DT>::E + cbase * 16, (uint32_t)(k * TPR * 16),
                           (uint32_t)(t * 16), v);
            else
                scatter<DT>(yr, g.col0(c), N, v);
        }
    }
}

// Elements i of a chunk outside [lo, hi) set to the fill pattern (0 <= lo,
// hi <= VEC): the out-of-row elements of a misaligned row's first and last
// chunk.
template <int DT>
__device__ __forceinline__ uint4 mask_range(uint4 r, int lo, int hi, uint32_t fill) {
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
    if constexpr (dt_info<DT>::E == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i < lo || i >= hi) w[i] = fill;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < lo || i >= hi)
                w[i >> 1] = (i & 1) ? ((w[i >> 1] & 0xFFFFu) | (fill & 0xFFFF0000u))
                                    : ((w[i >> 1] & 0xFFFF0000u) | (fill & 0xFFFFu));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// First step of a row load: the K chunks a lane owns, every vector load in
// flight at once.  Each lane issues each of its K loads unconditionally,
// with the chunk index clamped into the row's chunks (a slot past the row
// re-reads a chunk that is already in cache); finish_row() later replaces
// out-of-row slots and elements with the fill pattern.  A misaligned row's
// partial first and last chunks are loaded whole as well: a 16-byte-aligned
// chunk that holds an element of the row lies in the memory page holding
// that element, so the load cannot fault, and its bytes outside the row are
// masked in registers -- one memory round trip for the whole row.
template <int DT, bool AL, int K, int TPR, bool NT = true>
__device__ __forceinline__ void load_row(uint4 (&raw)[K], const RowGeom<DT, AL> &g, int t, int32_t N,
                                         int64_t cbase = 0) {
    (void)N;
    const int64_t last = g.nch - 1;            // the row touches chunks 0 .. nch - 1 (nch >= 1)
#pragma unroll
    for (int k = 0; k < K; ++k) {
        int64_t c = cbase + (int64_t)k * TPR + t;
        // (c >= 0 always; finish_row() repeats this exact test, which lets the
        // compiler keep one predicate per slot instead of the 64-bit indices:
        // the 8 x 8 fp32 cooperative softmax holds 56 instead of 66 VGPRs)
        c = c < 0 ? 0 : (c > last ? last : c);
        raw[k] = NT ? ld16_nt(g.xb + c * 16) : ld16(g.xb + c * 16);
    }
}

// Second step of a row load, after every other load meant to be in flight
// with the row (the parameter vectors) has been issued: slots past the row
// get the fill pattern, the elements of a misaligned row's partial chunks
// that lie outside the row too, and an empty asm statement pins the packed
// values, so their widening is not moved into these branches and widened
// values are known to be canonical floats (no quieting before v_max).
template <int DT, bool AL, int K, int TPR>
__device__ __forceinline__ void finish_row(uint4 (&raw)[K], const RowGeom<DT, AL> &g, const char *xr, int t,
                                           int32_t N, uint32_t fill, int64_t cbase = 0) {
    (void)xr;
    constexpr int VEC = dt_info<DT>::VEC;
    const int64_t last = g.nch - 1;        // the tests of load_row's clamp
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t c = cbase + (int64_t)k * TPR + t;
        if (AL && cbase + ((int64_t)k + 1) * TPR <= g.nch) continue;   // whole slice: uniform
        if (c < 0 || c > last) {
            raw[k] = make_uint4(fill, fill, fill, fill);
        } else if constexpr (!AL) {
            const int64_t c0 = g.col0(c);                               // column of the chunk's element 0
            if (c0 < 0 || c0 + VEC > N) {
                const int lo = c0 < 0 ? (int)-c0 : 0;
                const int hi = (int64_t)N - c0 < VEC ? (int)((int64_t)N - c0) : VEC;
                raw[k] = mask_range<DT>(raw[k], lo, hi, fill);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k)
        asm volatile("" : "+v"(raw[k].x), "+v"(raw[k].y), "+v"(raw[k].z), "+v"(raw[k].w));
}

// Load the parameter-vector chunks that line up with the row's chunks (the
// same clamped, branch-free scheme; misaligned rows read per element).
template <int DT, bool AL, int K, int TPR>
__device__ __forceinline__ void load_params(uint4 (&out)[K], const RowGeom<DT, AL> &g, const char *p, int t,
                                            int32_t N, int64_t cbase = 0) {
    if constexpr (AL) {
        const int64_t last = g.nch - 1;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            int64_t c = cbase + (int64_t)k * TPR + t;
            c = c > last ? last : c;
            out[k] = ld16(p + c * 16);
        }
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k) out[k] = load_param<DT, AL>(g, p, cbase + (int64_t)k * TPR + t, N);
    }
}

template <int DT, bool AL, int TPR>
__device__ __forceinline__ void store_slice(const RowGeom<DT, AL> &g, char *yr, int k, int t, int32_t N, bool yvec,
                                            uint4 v, int64_t cbase = 0) {
    if (AL && cbase + ((int64_t)k + 1) * TPR <= g.nch)
        st16_nt_at(yr + cbase * 16, (uint32_t)(k * TPR * 16), (uint32_t)(t * 16), v);   // whole slice
    else
        store_chunk<DT, AL, TPR>(g, yr, cbase, k, t, N, yvec, v);
}

// Is element i of chunk c a column of the row?
template <int DT, bool AL>
__device__ __forceinline__ bool in_row(const RowGeom<DT, AL> &g, int64_t c, int i, int32_t N) {
    if constexpr (AL) {
        return c < g.nch;
    } else {
        const int64_t col = g.col0(c) + i;
        return c < g.nch && col >= 0 && col < N;
    }
}

// The value of the first element packed in a storage word, widened to fp32.
template <int DT>
__device__ __forceinline__ float elem_of_word(uint32_t w) {
    if constexpr (DT == DT_F32) return __builtin_bit_cast(float, w);
    else if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(f16x2, w).x;
    else return __builtin_bit_cast(float, w << 16);
}

// The word a LayerNorm row is padded with: its first element (the pivot of
// the shifted sums), repeated in both halves for 16-bit types.
template <int DT>
__device__ __forceinline__ uint32_t pivot_word(const char *xr) {
    if constexpr (dt_info<DT>::E == 4) {
        return *reinterpret_cast<const uint32_t *>(xr);
    } else {
        const uint32_t e = *reinterpret_cast<const uint16_t *>(xr);
        return e | (e << 16);
    }
}

// ---------------------------------------------------------------------------
// Fused residual add (the step before a norm): h = x + r, summed in fp32 and
// rounded once to the element type.  For two fp32, fp16 or bf16 values the
// rounded fp32 sum rounds to the element type exactly as the exact sum does,
// so h is the stored sum of an add kernel run on its own.
// ---------------------------------------------------------------------------

// Pivot word of the fused row: the first element of h.
template <int DT>
__device__ __forceinline__ uint32_t pivot_word_sum(const char *xr, const char *rr) {
    constexpr int VEC = dt_info<DT>::VEC;
    const float s = elem_of_word<DT>(pivot_word<DT>(xr)) + elem_of_word<DT>(pivot_word<DT>(rr));
    float f[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) f[i] = s;
    return pack<DT>(f).x;
}

// raw holds the row's x words, rr its residual words (same chunk geometry:
// x, r and h share their 16-byte phase).  On return raw holds the words of h,
// which are also stored to the h row.  Padding slots hold pad + 0 = pad.
template <int DT, bool AL, int K, int TPR>
__device__ __forceinline__ void add_residual(uint4 (&raw)[K], const uint4 (&rr)[K], const RowGeom<DT, AL> &g,
                                             char *hrow, int t, int32_t N, int64_t cbase = 0) {
    constexpr int VEC = dt_info<DT>::VEC;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float xv[VEC], rv[VEC];
        unpack<DT>(raw[k], xv);
        unpack<DT>(rr[k], rv);
#pragma unroll
        for (int i = 0; i < VEC; ++i) xv[i] += rv[i];
        raw[k] = pack<DT>(xv);
        store_slice<DT, AL, TPR>(g, hrow, k, t, N, true, raw[k], cbase);
    }
}

// ---------------------------------------------------------------------------
// Causal softmax rows: query q = row mod queries sees keys 0 .. q + offset.
// A row is loaded as if it were only its visible prefix of L columns (the
// general, element-gathering geometry, so a partial last chunk is read
// element by element and nothing past column L is fetched: clamped loads
// past the prefix re-read its last whole chunk, a cache hit), and padded
// with -inf, which turns into exact zeros in the output; the store covers
// the whole row.  Both geometries give chunk c the same columns.
// ---------------------------------------------------------------------------

// The host clamps `queries` to M, so a 32-bit remainder serves whenever the
// row index fits in 32 bits (a 64-bit one is a long instruction sequence).
__device__ __forceinline__ int32_t visible_len(const RowArgs &a, int64_t row) {
    const int64_t q = (a.M <= 0xFFFFFFFFll) ? (int64_t)((uint32_t)row % (uint32_t)a.queries) : row % a.queries;
    const int64_t v = q + a.offset + 1;
    return v < (int64_t)a.N ? (int32_t)v : a.N;
}

// Elements i >= rem of a chunk set to -inf (rem in 1 .. VEC-1).
template <int DT>
__device__ __forceinline__ uint4 mask_tail(uint4 r, int rem) {
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
    if constexpr (dt_info<DT>::E == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i >= rem) w[i] = dt_info<DT>::NEG_INF_WORD;
    } else {
        const uint32_t ninf = dt_info<DT>::NEG_INF_WORD & 0xFFFFu;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i >= rem) w[i >> 1] = (i & 1) ? ((w[i >> 1] & 0xFFFFu) | (ninf << 16)) : ((w[i >> 1] & 0xFFFF0000u) | ninf);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Issue the loads of a softmax row slice.  Causal rows read their visible
// prefix only: on 16-byte-aligned rows the chunk holding the last visible
// column is loaded whole (it lies inside the row) and masked in registers;
// misaligned rows use the element-gathering geometry on the prefix.
template <int DT, bool AL, int K, int TPR, bool CAUSAL, bool NT = true>
__device__ __forceinline__ void softmax_issue(uint4 (&raw)[K], const RowGeom<DT, AL> &geo, const char *xr, int t,
                                              int32_t N, int32_t L, int64_t cbase = 0) {
    constexpr int VEC = dt_info<DT>::VEC;
    if constexpr (CAUSAL && AL) {
        const int64_t f1 = (L + VEC - 1) / VEC - 1;      // chunk holding column L - 1
#pragma unroll
        for (int k = 0; k < K; ++k) {
            int64_t c = cbase + (int64_t)k * TPR + t;
            c = c > f1 ? f1 : c;
            raw[k] = NT ? ld16_nt(xr + c * 16) : ld16(xr + c * 16);
        }
    } else if constexpr (CAUSAL) {
        load_row<DT, false, K, TPR, NT>(raw, RowGeom<DT, false>(xr, L), t, L, cbase);
    } else {
        load_row<DT, AL, K, TPR, NT>(raw, geo, t, N, cbase);
    }
}

// Complete it: -inf outside the row (causal: outside the visible prefix).
template <int DT, bool AL, int K, int TPR, bool CAUSAL>
__device__ __forceinline__ void softmax_finish(uint4 (&raw)[K], const RowGeom<DT, AL> &geo, const char *xr, int t,
                                               int32_t N, int32_t L, int64_t cbase = 0) {
    constexpr int VEC = dt_info<DT>::VEC;
    constexpr uint32_t NI = dt_info<DT>::NEG_INF_WORD;
    if constexpr (CAUSAL && AL) {
        const int64_t f1 = (L + VEC - 1) / VEC - 1;
        const int rem = L - (int)(f1 * VEC);                // visible elements of chunk f1: 1 .. VEC
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t c = cbase + (int64_t)k * TPR + t;
            if (c > f1)
                raw[k] = make_uint4(NI, NI, NI, NI);
            else if (c == f1 && rem < VEC)
                raw[k] = mask_tail<DT>(raw[k], rem);
        }
#pragma unroll
        for (int k = 0; k < K; ++k)
            asm volatile("" : "+v"(raw[k].x), "+v"(raw[k].y), "+v"(raw[k].z), "+v"(raw[k].w));
    } else if constexpr (CAUSAL) {
        finish_row<DT, false, K, TPR>(raw, RowGeom<DT, false>(xr, L), xr, t, L, NI, cbase);
    } else {
        finish_row<DT, AL, K, TPR>(raw, geo, xr, t, N, NI, cbase);
    }
}

// ---------------------------------------------------------------------------
// Per-row scalar helpers
// ---------------------------------------------------------------------------

// Exponent offset of every softmax kernel.  Each term is taken as
// 2^(x*s2 - c) with c = m*s2 - EXP_SHIFT rounded once (m the row's or the
// chunk's max, s2 = log2(e) or scale*log2(e)), so the largest term is about
// 2^EXP_SHIFT.  v_exp_f32 flushes results below 2^-126 to zero; with the
// offset, every term down to 2^-150 of the largest (the smallest that can
// still round to a non-zero fp32 output, the sum being >= the largest term)
// is a normal float, and the output multiply by 1/sum rounds it once into
// the subnormal range.  Shift invariance makes any c exact in real
// arithmetic; the sum stays far from overflow (at most 2^24 * N).
constexpr float EXP_SHIFT = 24.0f;
__device__ __forceinline__ float exp_offset(float m, float s2) { return __builtin_fmaf(m, s2, -EXP_SHIFT); }

// 1/x and 1/sqrt(x) in fp32 from the hardware approximations (v_rcp_f32,
// v_rsq_f32: about 1 ulp), used once per row.
__device__ __forceinline__ float rcp_approx(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float rsq_approx(float x) { return __builtin_amdgcn_rsqf(x); }

// 1/sqrt(v) in fp64: hardware estimate refined by two Newton steps
// r <- r * (3 - v r^2) / 2, each roughly doubling the correct bits.
__device__ __forceinline__ double rsqrt_f64(double v) {
    if (v == 0.0) return __builtin_inf();      // eps = 0 and a constant row
    double r = __builtin_amdgcn_rsq(v);
#pragma unroll
    for (int i = 0; i < 2; ++i) r = r * __builtin_fma(-0.5 * v, r * r, 1.5);
    return r;
}

// Per-lane max over K*VEC widened values (padding holds -inf).
template <int K, int VEC>
__device__ __forceinline__ float lane_max(const float (&v)[K][VEC]) {
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int i = 0; i < VEC; i += 2) m = __builtin_fmaxf(m, __builtin_fmaxf(v[k][i], v[k][i + 1]));
    return m;
}

// ---------------------------------------------------------------------------
// Single-pass kernel: one row per group of W waves, row held in VGPRs.
// W == 1: four independent rows per 256-thread workgroup, no LDS or barrier.
// W >= 2: one row per workgroup of 64*W threads.
// Each element is widened to fp32 once; every pass then works on the
// widened registers.
// ---------------------------------------------------------------------------

template <int W>
struct GroupShape {
    static constexpr int G = (W == 1) ? 4 : 1;           // rows per workgroup
    static constexpr int THREADS = 64 * W * G;
};

// PR (norms only): the parameter vectors are all present (gamma and beta for
// LayerNorm, the weight for RMSNorm); otherwise absent ones act as identity.
template <int OP, int DT, int W, int K, bool AL, bool PR, bool RES = false>
__global__ void __launch_bounds__(GroupShape<W>::THREADS)
row_resident(RowArgs a) {
    constexpr bool SM = OP == OP_SOFTMAX || OP == OP_SOFTMAX_CAUSAL;
    constexpr bool CAUSAL = OP == OP_SOFTMAX_CAUSAL;
    static_assert(!RES || !SM, "the residual add precedes a norm");
    using I = dt_info<DT>;
    constexpr int VEC = I::VEC, TPR = 64 * W, G = GroupShape<W>::G;
    // LayerNorm keeps an fp64 copy of its values when they are few per lane
    constexpr bool CACHE_D = (OP == OP_LAYERNORM) && (K * VEC <= 16);
    const int tid = threadIdx.x;
    const int g = (W == 1) ? (tid >> 6) : 0;
    const int t = (W == 1) ? (tid & 63) : tid;
    const int wv = t >> 6, lane = t & 63;
    const int32_t N = a.N;
    const int64_t rowbytes = (int64_t)N * I::E;
    const uint32_t fill = SM ? I::NEG_INF_WORD : 0u;
    const bool has_p0 = PR || a.p0 != nullptr, has_p1 = PR || a.p1 != nullptr;

    __shared__ float red_f[2][2][W];
    __shared__ double2 red_d2[2][W];

    const int64_t nrb = (a.M + G - 1) / G;
    int par = 0;
    for (int64_t rb = xcd_band(blockIdx.x, gridDim.x); rb < nrb; rb += gridDim.x, par ^= 1) {
        int64_t row = rb * G + g;
        // Causal rows (one per workgroup): workgroups alternate between rows
        // from the two ends of the matrix, so a short and a long visible
        // prefix stream side by side (in the square layout each pair reads
        // N + 1 elements) instead of runs of read-light then read-heavy rows:
        // 5-6% faster on 131072 x 4096 and 32768 x 8192 bf16 scores.
        if constexpr (CAUSAL && G == 1) row = (rb & 1) ? a.M - 1 - (rb >> 1) : (rb >> 1);
        if (row >= a.M) break;   // only possible when W == 1 (no barriers there)
        const char *xr = a.x + row * rowbytes;
        char *yr = a.y + row * rowbytes;
        const RowGeom<DT, AL> geo(xr, N);
        bool yvec = true;
        if constexpr (!AL) yvec = (((uintptr_t)yr ^ (uintptr_t)xr) & 15) == 0;

        // ---- issue every load of the row (and of the parameter vectors,
        // which are L2 hits after the first rows) before using any of them
        // LayerNorm pads with its pivot (the row's first element), which adds
        // exactly nothing to the shifted sums; softmax pads with -inf, RMSNorm 0
        const char *rr = RES ? a.r + row * rowbytes : nullptr;
        uint32_t padw = fill;
        if constexpr (OP == OP_LAYERNORM) padw = RES ? pivot_word_sum<DT>(xr, rr) : pivot_word<DT>(xr);
        uint4 raw[K], rraw[RES ? K : 1];
        const int32_t L = CAUSAL ? visible_len(a, row) : N;
        if constexpr (SM)
            softmax_issue<DT, AL, K, TPR, CAUSAL>(raw, geo, xr, t, N, L);
        else
            load_row<DT, AL, K, TPR>(raw, geo, t, N);
        if constexpr (RES) load_row<DT, AL, K, TPR>(rraw, RowGeom<DT, AL>(rr, N), t, N);
        constexpr int KP0 = SM ? 1 : K;
        constexpr int KP1 = (OP == OP_LAYERNORM) ? K : 1;
        uint4 p0[KP0], p1[KP1];
        if constexpr (!SM) {
            if (has_p0) load_params<DT, AL, K, TPR>(p0, geo, a.p0, t, N);
        }
        if constexpr (OP == OP_LAYERNORM) {
            if (has_p1) load_params<DT, AL, K, TPR>(p1, geo, a.p1, t, N);
        }
        if constexpr (SM)
            softmax_finish<DT, AL, K, TPR, CAUSAL>(raw, geo, xr, t, N, L);
        else
            finish_row<DT, AL, K, TPR>(raw, geo, xr, t, N, padw);
        if constexpr (RES) {
            // x padded with the pivot of h, r with 0: h's padding is the pivot
            finish_row<DT, AL, K, TPR>(rraw, RowGeom<DT, AL>(rr, N), rr, t, N, 0u);
            add_residual<DT, AL, K, TPR>(raw, rraw, geo, a.h + row * rowbytes, t, N);
        }
        float v[K][VEC];
#pragma unroll
        for (int k = 0; k < K; ++k) unpack<DT>(raw[k], v[k]);

        if constexpr (SM) {
            // ---- softmax.  With c = exp_offset(m), every element is
            // 2^(x*log2(e) - c): one fma (exact product, one rounding) and
            // one v_exp_f32; shift invariance makes the offset exact.  The
            // causal softmax of scale*x uses s2 = scale*log2(e) in place of
            // log2(e) (scale > 0, so the max of x gives the max of scale*x).
            const float s2 = CAUSAL ? a.s2 : LOG2E;
            const float mx = group_allreduce<W>(lane_max(v), MaxOp(), red_f[par][0], wv, lane);
            const float c = exp_offset(mx, s2);
            // fp32 rows of 4 or 8 chunks per lane recompute each exponential
            // for the output instead of keeping them all (the same arguments,
            // so the same bits): their stores then leave one chunk at a time,
            // 1-3% faster; with fewer values per lane, with 16-bit types and
            // on causal rows keeping them is as fast or faster.
            constexpr bool RECOMP = DT == DT_F32 && (K == 4 || K == 8) && !CAUSAL;
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(v[k][i], s2, -c));
                    if constexpr (!RECOMP) v[k][i] = e;
                    s += e;
                }
            s = group_allreduce<W>(s, SumOp(), red_f[par][1], wv, lane);
            const float inv = rcp_approx(s);
#pragma unroll
            for (int k = 0; k < K; ++k) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    if constexpr (RECOMP) {
                        float x = v[k][i];
                        asm volatile("" : "+v"(x));      // recompute: no reuse of the first pass
                        v[k][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, s2, -c)) * inv;
                    } else {
                        v[k][i] *= inv;
                    }
                }
                store_slice<DT, AL, TPR>(geo, yr, k, t, N, yvec, pack<DT>(v[k]));
            }
        } else if constexpr (OP == OP_RMSNORM) {
            // ---- RMSNorm: sum of squares in fp32, y = (x * inv) * w
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int i = 0; i < VEC; ++i) ss = __builtin_fmaf(v[k][i], v[k][i], ss);
            ss = group_allreduce<W>(ss, SumOp(), red_f[par][0], wv, lane);
            const float inv = rsq_approx(ss * a.inv_n + a.eps);
            if (PR) {
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    float w[VEC];
                    unpack<DT>(p0[k], w);
#pragma unroll
                    for (int i = 0; i < VEC; ++i) v[k][i] = (v[k][i] * inv) * w[i];
                    store_slice<DT, AL, TPR>(geo, yr, k, t, N, yvec, pack<DT>(v[k]));
                }
            } else {
#pragma unroll
                for (int k = 0; k < K; ++k) {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) v[k][i] *= inv;
                    store_slice<DT, AL, TPR>(geo, yr, k, t, N, yvec, pack<DT>(v[k]));
                }
            }
        } else {
            // ---- LayerNorm.  Statistics in one pass around the pivot p (the
            // row's first element): S1 = sum(x - p), S2 = sum((x - p)^2) in
            // fp64, so mean = p + S1/N and var = S2/N - (S1/N)^2.  For fp16 or
            // bf16 input every x - p and S1 are exact in fp64; the cancellation
            // in var costs about log2((p - mean)^2 / var) of fp64's 53 bits.
            // The affine step is fp64 too: fp32 cannot keep y within one ulp
            // of a 16-bit output where beta cancels (x - mean) * rstd * gamma.
            const double pv = (double)elem_of_word<DT>(padw);
            double dp[CACHE_D ? K : 1][CACHE_D ? VEC : 1];
            double s1 = 0.0, s2 = 0.0;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const double d = (double)v[k][i] - pv;    // padding gives 0
                    if constexpr (CACHE_D) dp[k][i] = d;
                    s1 += d;
                    s2 = __builtin_fma(d, d, s2);
                }
            const double2 st = group_allreduce<W>(double2{s1, s2}, SumOp(), red_d2[par], wv, lane);
            const double m1 = st.x * a.inv_nd;                  // mean - p
            const double var = __builtin_fmax(st.y * a.inv_nd - m1 * m1, 0.0);
            const double mean = pv + m1;
            const double rstd = rsqrt_f64(var + (double)a.eps);
            // (x - mean) * rstd = fma(x - p, rstd, -m1 * rstd): the same
            // expression in every LayerNorm kernel, so they agree bitwise
            const double nm = -m1 * rstd;
            if constexpr (PR) {
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    float gm[VEC], bt[VEC];
                    unpack<DT>(p0[k], gm);
                    unpack<DT>(p1[k], bt);
#pragma unroll
                    for (int i = 0; i < VEC; ++i) {
                        double d;
                        if constexpr (CACHE_D) {
                            d = dp[CACHE_D ? k : 0][CACHE_D ? i : 0];
                        } else {
                            float x = v[k][i];
                            asm volatile("" : "+v"(x));  // recompute, no fp64 copy of the row kept
                            d = (double)x - pv;
                        }
                        v[k][i] = (float)__builtin_fma(__builtin_fma(d, rstd, nm), (double)gm[i], (double)bt[i]);
                    }
                    store_slice<DT, AL, TPR>(geo, yr, k, t, N, yvec, pack<DT>(v[k]));
                }
            } else {
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    float gm[VEC], bt[VEC];
                    if (has_p0) unpack<DT>(p0[k], gm);
                    if (has_p1) unpack<DT>(p1[k], bt);
#pragma unroll
                    for (int i = 0; i < VEC; ++i) {
                        double d;
                        if constexpr (CACHE_D) {
                            d = dp[CACHE_D ? k : 0][CACHE_D ? i : 0];
                        } else {
                            float x = v[k][i];
                            asm volatile("" : "+v"(x));
                            d = (double)x - pv;
                        }
                        const double g = has_p0 ? (double)gm[i] : 1.0;
                        const double b = has_p1 ? (double)bt[i] : 0.0;
                        v[k][i] = (float)__builtin_fma(__builtin_fma(d, rstd, nm), g, b);
                    }
                    store_slice<DT, AL, TPR>(geo, yr, k, t, N, yvec, pack<DT>(v[k]));
                }
            }
            if (t == 0) {
                if (a.mean) a.mean[row] = (float)mean;
                if (a.rstd) a.rstd[row] = (float)rstd;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Persistent kernel for LayerNorm / RMSNorm with every parameter vector
// present and 16-byte-aligned rows: each lane always owns the same columns,
// so a workgroup widens its gamma/beta (fp64, LayerNorm) or weight (fp32,
// RMSNorm) once, then strides over rows with the next row's loads in flight
// while the current row is reduced and written.  One row per workgroup of
// 64*W threads (W >= 2).
// ---------------------------------------------------------------------------

template <int OP, int DT, int W, int K, bool RES = false>
__global__ void __launch_bounds__(64 * W)
row_norm_persistent(RowArgs a) {
    static_assert(OP == OP_LAYERNORM || OP == OP_RMSNORM, "persistent kernel is for the norms");
    static_assert(W >= 2, "one row per workgroup");
    using I = dt_info<DT>;
    constexpr int VEC = I::VEC, TPR = 64 * W;
    constexpr bool LN = OP == OP_LAYERNORM;
    const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
    const int32_t N = a.N;
    const int64_t rowbytes = (int64_t)N * I::E;
    __shared__ double2 red_d2[2][W];
    __shared__ float red_f[2][W];

    int64_t row = blockIdx.x;
    if (row >= a.M) return;
    const RowGeom<DT, true> geo(a.x, N);     // every row has the same chunk geometry

    // ---- parameters, widened once per workgroup.  LayerNorm with 32 values
    // per lane keeps gamma, beta as fp32 (widened to fp64 at use: exact) and
    // recomputes x - p in the epilogue, so the row, its successor and the
    // parameters fit a 512-thread workgroup's registers; the values are the
    // same either way.  16-bit LayerNorm at 5 to 8 waves does the same with
    // 16 values per lane: 125 instead of 139 registers fit two workgroups per
    // CU instead of one (4224- to 8192-wide rows 4-7.5% faster); with fewer
    // waves, or fp32, the fp64 caches measured as fast or faster.
    constexpr bool LN_WIDE = LN && (K * VEC > 16 || (VEC == 8 && W >= 5));
    constexpr bool LN_D = LN && !LN_WIDE;
    double g64[LN_D ? K : 1][LN_D ? VEC : 1], b64[LN_D ? K : 1][LN_D ? VEC : 1];
    float w32[LN_D ? 1 : K][LN_D ? 1 : VEC], b32[LN_WIDE ? K : 1][LN_WIDE ? VEC : 1];
    {
        uint4 p0[K], p1[LN ? K : 1];
        load_params<DT, true, K, TPR>(p0, geo, a.p0, t, N);
        if constexpr (LN) load_params<DT, true, K, TPR>(p1, geo, a.p1, t, N);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float g[VEC], b[VEC];
            unpack<DT>(p0[k], g);
            if constexpr (LN_D) {
                unpack<DT>(p1[k], b);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    g64[k][i] = (double)g[i];
                    b64[k][i] = (double)b[i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < VEC; ++i) w32[k][i] = g[i];
                if constexpr (LN_WIDE) {
                    unpack<DT>(p1[k], b);
#pragma unroll
                    for (int i = 0; i < VEC; ++i) b32[k][i] = b[i];
                }
            }
        }
    }

    // ---- prime the pipeline with the first row (and its residual)
    uint4 raw[K], rraw[RES ? K : 1];
    uint32_t padw = 0;
    {
        const char *xr = a.x + row * rowbytes;
        load_row<DT, true, K, TPR>(raw, RowGeom<DT, true>(xr, N), t, N);
        if constexpr (RES) load_row<DT, true, K, TPR>(rraw, RowGeom<DT, true>(a.r + row * rowbytes, N), t, N);
        if constexpr (LN) padw = RES ? pivot_word_sum<DT>(xr, a.r + row * rowbytes) : pivot_word<DT>(xr);
    }
    int par = 0;
    for (; row < a.M; row += gridDim.x, par ^= 1) {
        const char *xr = a.x + row * rowbytes;
        char *yr = a.y + row * rowbytes;
        const RowGeom<DT, true> g(xr, N);
        finish_row<DT, true, K, TPR>(raw, g, xr, t, N, padw);
        if constexpr (RES) {
            const char *rr = a.r + row * rowbytes;
            finish_row<DT, true, K, TPR>(rraw, RowGeom<DT, true>(rr, N), rr, t, N, 0u);
            add_residual<DT, true, K, TPR>(raw, rraw, g, a.h + row * rowbytes, t, N);
        }
        float v[K][VEC];
#pragma unroll
        for (int k = 0; k < K; ++k) unpack<DT>(raw[k], v[k]);
        const uint32_t pw = padw;

        // issue the next row's loads (clamped to the last row, so no branch)
        {
            const int64_t nr = row + gridDim.x < a.M ? row + gridDim.x : a.M - 1;
            const char *xn = a.x + nr * rowbytes;
            load_row<DT, true, K, TPR>(raw, RowGeom<DT, true>(xn, N), t, N);
            if constexpr (RES) load_row<DT, true, K, TPR>(rraw, RowGeom<DT, true>(a.r + nr * rowbytes, N), t, N);
            if constexpr (LN) padw = RES ? pivot_word_sum<DT>(xn, a.r + nr * rowbytes) : pivot_word<DT>(xn);
        }

        if constexpr (LN) {
            const double pv = (double)elem_of_word<DT>(pw);
            double s1 = 0.0, s2 = 0.0;
            double dp[LN_D ? K : 1][LN_D ? VEC : 1];
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const double d = (double)v[k][i] - pv;  // padding holds p: 0
                    if constexpr (LN_D) dp[LN_D ? k : 0][LN_D ? i : 0] = d;
                    s1 += d;
                    s2 = __builtin_fma(d, d, s2);
                }
            const double2 st = group_allreduce<W>(double2{s1, s2}, SumOp(), red_d2[par], wv, lane);
            const double m1 = st.x * a.inv_nd;
            const double var = __builtin_fmax(st.y * a.inv_nd - m1 * m1, 0.0);
            const double rstd = rsqrt_f64(var + (double)a.eps);
            const double nm = -m1 * rstd;                     // (dp - m1) * rstd = fma(dp, rstd, nm)
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float o[VEC];
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    if constexpr (LN_D) {
                        o[i] = (float)__builtin_fma(__builtin_fma(dp[k][i], rstd, nm), g64[k][i], b64[k][i]);
                    } else {
                        float x = v[k][i];
                        asm volatile("" : "+v"(x));      // recompute x - p, no copy of the first pass's
                        const double d = (double)x - pv;
                        o[i] = (float)__builtin_fma(__builtin_fma(d, rstd, nm), (double)w32[k][i],
                                                    (double)b32[LN_WIDE ? k : 0][LN_WIDE ? i : 0]);
                    }
                }
                st16_nt_bounded(yr, (uint32_t)rowbytes, (uint32_t)((k * TPR + t) * 16), pack<DT>(o));
            }
            // lane 0 writes the statistics (the other lanes' offsets are out of range)
            st4_bounded(a.mean ? a.mean + row : nullptr, a.mean ? 4u : 0u, (uint32_t)t * 4u, (float)(pv + m1));
            st4_bounded(a.rstd ? a.rstd + row : nullptr, a.rstd ? 4u : 0u, (uint32_t)t * 4u, (float)rstd);
        } else {
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int i = 0; i < VEC; ++i) ss = __builtin_fmaf(v[k][i], v[k][i], ss);
            ss = group_allreduce<W>(ss, SumOp(), red_f[par], wv, lane);
            const float inv = rsq_approx(ss * a.inv_n + a.eps);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float o[VEC];
#pragma unroll
                for (int i = 0; i < VEC; ++i) o[i] = (v[k][i] * inv) * w32[k][i];
                st16_nt_bounded(yr, (uint32_t)rowbytes, (uint32_t)((k * TPR + t) * 16), pack<DT>(o));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Looped kernel for LayerNorm / RMSNorm rows wider than the single-pass
// shapes: one workgroup of 64*W threads per row streams the row in tiles of
// 64*W*K chunks twice, first for the statistics, then for the output.  The
// second read of a row is usually served by L2 or the Infinity Cache.  The
// statistics accumulate in fp64 (a lane may sum thousands of values).
// ---------------------------------------------------------------------------

template <int OP, int DT, int W, int K, bool AL, bool RES = false>
__global__ void __launch_bounds__(64 * W)
row_looped(RowArgs a) {
    static_assert(OP == OP_LAYERNORM || OP == OP_RMSNORM, "looped kernel is for the norms");
    using I = dt_info<DT>;
    constexpr int VEC = I::VEC, TPR = 64 * W;
    constexpr int64_t TILE = (int64_t)TPR * K;
    const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
    const int32_t N = a.N;
    const int64_t rowbytes = (int64_t)N * I::E;
    const bool has_p0 = a.p0 != nullptr, has_p1 = a.p1 != nullptr;
    __shared__ double2 red[2][W];

    int par = 0;
    for (int64_t row = blockIdx.x; row < a.M; row += gridDim.x, par ^= 1) {
        const char *xr = a.x + row * rowbytes;
        char *yr = a.y + row * rowbytes;
        const RowGeom<DT, AL> geo(xr, N);
        bool yvec = true;
        if constexpr (!AL) yvec = (((uintptr_t)yr ^ (uintptr_t)xr) & 15) == 0;
        const char *rr = RES ? a.r + row * rowbytes : nullptr;
        char *hr = RES ? a.h + row * rowbytes : nullptr;
        uint32_t padw = 0;
        if constexpr (OP == OP_LAYERNORM) padw = RES ? pivot_word_sum<DT>(xr, rr) : pivot_word<DT>(xr);
        const double pv = (double)elem_of_word<DT>(padw);   // 0 for RMSNorm
        const int64_t ntiles = (geo.nch + TILE - 1) / TILE;

        // ---- pass 1: statistics (of h = x + r, which is stored on the way)
        double s1 = 0.0, s2 = 0.0;
        for (int64_t tl = 0; tl < ntiles; ++tl) {
            uint4 raw[K];
            load_row<DT, AL, K, TPR>(raw, geo, t, N, tl * TILE);
            if constexpr (RES) {
                uint4 rraw[K];
                const RowGeom<DT, AL> gr(rr, N);
                load_row<DT, AL, K, TPR>(rraw, gr, t, N, tl * TILE);
                finish_row<DT, AL, K, TPR>(raw, geo, xr, t, N, padw, tl * TILE);
                finish_row<DT, AL, K, TPR>(rraw, gr, rr, t, N, 0u, tl * TILE);
                add_residual<DT, AL, K, TPR>(raw, rraw, geo, hr, t, N, tl * TILE);
            } else {
                finish_row<DT, AL, K, TPR>(raw, geo, xr, t, N, padw, tl * TILE);
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float v[VEC];
                unpack<DT>(raw[k], v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const double d = (double)v[i] - pv;          // padding gives 0
                    if constexpr (OP == OP_LAYERNORM) s1 += d;
                    s2 = __builtin_fma(d, d, s2);
                }
            }
        }
        const double2 st = group_allreduce<W>(double2{s1, s2}, SumOp(), red[par], wv, lane);
        double m1 = 0.0, scale;
        if constexpr (OP == OP_LAYERNORM) {
            m1 = st.x * a.inv_nd;
            const double var = __builtin_fmax(st.y * a.inv_nd - m1 * m1, 0.0);
            scale = rsqrt_f64(var + (double)a.eps);
            if (t == 0) {
                if (a.mean) a.mean[row] = (float)(pv + m1);
                if (a.rstd) a.rstd[row] = (float)scale;
            }
        } else {
            scale = rsqrt_f64(st.y * a.inv_nd + (double)a.eps);
        }
        const float scale_f = (float)scale;
        const double nm = -m1 * scale;                  // as in the single-pass kernels

        // ---- pass 2: normalize.  With the residual add it reads back h:
        // every lane reads exactly the chunks it stored in pass 1, so a
        // workgroup-scope fence (stores complete before these loads) orders it.
        const char *src = RES ? hr : xr;
        if constexpr (RES) {
            wait_own_stores();
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
        }
        const RowGeom<DT, AL> gs(src, N);
        for (int64_t tl = 0; tl < ntiles; ++tl) {
            uint4 raw[K], g4[K], b4[(OP == OP_LAYERNORM) ? K : 1];
            load_row<DT, AL, K, TPR>(raw, gs, t, N, tl * TILE);
            if (has_p0) load_params<DT, AL, K, TPR>(g4, geo, a.p0, t, N, tl * TILE);
            if constexpr (OP == OP_LAYERNORM) {
                if (has_p1) load_params<DT, AL, K, TPR>(b4, geo, a.p1, t, N, tl * TILE);
            }
            finish_row<DT, AL, K, TPR>(raw, gs, src, t, N, padw, tl * TILE);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float v[VEC], g[VEC], b[VEC];
                unpack<DT>(raw[k], v);
                if (has_p0) unpack<DT>(g4[k], g);
                if constexpr (OP == OP_LAYERNORM) {
                    if (has_p1) unpack<DT>(b4[k], b);
                }
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const float gi = has_p0 ? g[i] : 1.0f;
                    if constexpr (OP == OP_LAYERNORM) {
                        const double d = (double)v[i] - pv;
                        v[i] = (float)__builtin_fma(__builtin_fma(d, scale, nm), (double)gi,
                                                    has_p1 ? (double)b[i] : 0.0);
                    } else {
                        v[i] = (v[i] * scale_f) * gi;
                    }
                }
                store_slice<DT, AL, TPR>(geo, yr, k, t, N, yvec, pack<DT>(v), tl * TILE);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Split norm, for a few rows too wide for one pass: workgroup b handles chunk
// j = b mod P of row r = b / P (64*W*K 16-byte pieces, as in the split
// softmax), so the row's chunks run on many CUs instead of one.  The partial
// kernel writes each chunk's (sum(x - p), sum((x - p)^2)) in fp64 around the
// row's first element p (RMSNorm: p = 0) to the workspace; the finalize
// kernel sums the row's P pairs in a fixed order (lane l takes pairs l,
// l + 64, ..., then the wave's fixed reduction), so every workgroup of the
// row derives the same statistics, and writes its chunk's outputs, reading
// the chunk again (usually from the Infinity Cache).  Workspace: M*P pairs,
// then the M pivots (the finalize kernel takes p from there: in place,
// workgroup 0 of the row overwrites the row's first element).
// ---------------------------------------------------------------------------

// (sum(x - p), sum((x - p)^2)) of chunk `qbase` of a row, in registers,
// reduced over the workgroup (`slot`: W entries of LDS, see group_allreduce).
template <int OP, int DT, int W, int K>
__device__ __forceinline__ double2 norm_chunk_sums(const uint4 (&raw)[K], double pv, double2 *slot, int wv,
                                                   int lane) {
    constexpr int VEC = dt_info<DT>::VEC;
    double s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float v[VEC];
        unpack<DT>(raw[k], v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const double d = (double)v[i] - pv;          // padding gives 0
            if constexpr (OP == OP_LAYERNORM) s1 += d;
            s2 = __builtin_fma(d, d, s2);
        }
    }
    return group_allreduce<W>(double2{s1, s2}, SumOp(), slot, wv, lane);
}

// The same sums of a chunk that is not in registers, one 16-byte slice per
// lane at a time: slice k holds exactly slot k of a whole-chunk load and the
// additions run in the same order, so the pair is bitwise norm_chunk_sums'.
template <int OP, int DT, int W, int K, bool AL>
__device__ __forceinline__ double2 norm_chunk_sums_reload(const RowGeom<DT, AL> &geo, const char *xr, int t,
                                                          int32_t N, uint32_t padw, double pv, int64_t qbase,
                                                          double2 *slot, int wv, int lane) {
    constexpr int VEC = dt_info<DT>::VEC, TPR = 64 * W;
    double s1 = 0.0, s2 = 0.0;
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
        uint4 r[1];
        load_row<DT, AL, 1, TPR>(r, geo, t, N, qbase + (int64_t)k * TPR);
        finish_row<DT, AL, 1, TPR>(r, geo, xr, t, N, padw, qbase + (int64_t)k * TPR);
        float v[VEC];
        unpack<DT>(r[0], v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const double d = (double)v[i] - pv;
            if constexpr (OP == OP_LAYERNORM) s1 += d;
            s2 = __builtin_fma(d, d, s2);
        }
    }
    return group_allreduce<W>(double2{s1, s2}, SumOp(), slot, wv, lane);
}

template <int OP, int DT, int W, int K, bool AL>
__global__ void __launch_bounds__(64 * W)
norm_split_partial(RowArgs a) {
    static_assert(OP == OP_LAYERNORM || OP == OP_RMSNORM, "split norm");
    using I = dt_info<DT>;
    constexpr int TPR = 64 * W;
    const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
    const int32_t N = a.N, P = a.P;
    const int64_t row = blockIdx.x / P;
    const int64_t j = blockIdx.x - row * P;
    const char *xr = a.x + row * (int64_t)N * I::E;
    const RowGeom<DT, AL> geo(xr, N);
    __shared__ double2 red[W];

    const int64_t cbase = j * (int64_t)(TPR * K);
    uint32_t padw = 0;
    if constexpr (OP == OP_LAYERNORM) padw = pivot_word<DT>(xr);
    const double pv = (double)elem_of_word<DT>(padw);
    uint4 raw[K];
    load_row<DT, AL, K, TPR>(raw, geo, t, N, cbase);
    finish_row<DT, AL, K, TPR>(raw, geo, xr, t, N, padw, cbase);
    const double2 st = norm_chunk_sums<OP, DT, W, K>(raw, pv, red, wv, lane);
    if (t == 0) {
        double *w = a.wsd + 2 * (row * P + j);
        w[0] = st.x;
        w[1] = st.y;
        if (j == 0) a.wsd[2 * a.M * P + row] = pv;
    }
}

template <int OP, int DT, int W, int K, bool AL>
__global__ void __launch_bounds__(64 * W)
norm_split_finalize(RowArgs a) {
    static_assert(OP == OP_LAYERNORM || OP == OP_RMSNORM, "split norm");
    using I = dt_info<DT>;
    constexpr int VEC = I::VEC, TPR = 64 * W;
    const int t = threadIdx.x, lane = t & 63;
    const int32_t N = a.N, P = a.P;
    const int64_t row = blockIdx.x / P;
    const int64_t j = blockIdx.x - row * P;
    const int64_t rowbytes = (int64_t)N * I::E;
    const char *xr = a.x + row * rowbytes;
    char *yr = a.y + row * rowbytes;
    const RowGeom<DT, AL> geo(xr, N);
    bool yvec = true;
    if constexpr (!AL) yvec = (((uintptr_t)yr ^ (uintptr_t)xr) & 15) == 0;
    const bool has_p0 = a.p0 != nullptr, has_p1 = a.p1 != nullptr;

    // the loads of this chunk first, then the row's pairs
    const int64_t cbase = j * (int64_t)(TPR * K);
    const double *w = a.wsd + 2 * row * P;
    const double pv = OP == OP_LAYERNORM ? a.wsd[2 * a.M * P + row] : 0.0;
    uint4 raw[K], g4[K], b4[(OP == OP_LAYERNORM) ? K : 1];
    load_row<DT, AL, K, TPR>(raw, geo, t, N, cbase);
    if (has_p0) load_params<DT, AL, K, TPR>(g4, geo, a.p0, t, N, cbase);
    if constexpr (OP == OP_LAYERNORM) {
        if (has_p1) load_params<DT, AL, K, TPR>(b4, geo, a.p1, t, N, cbase);
    }
    double s1 = 0.0, s2 = 0.0;
    for (int q = lane; q < P; q += 64) {
        s1 += w[2 * q];
        s2 += w[2 * q + 1];
    }
    const double2 st = wave_allreduce(double2{s1, s2}, SumOp());
    double m1 = 0.0, scale;
    if constexpr (OP == OP_LAYERNORM) {
        m1 = st.x * a.inv_nd;
        const double var = __builtin_fmax(st.y * a.inv_nd - m1 * m1, 0.0);
        scale = rsqrt_f64(var + (double)a.eps);
        if (j == 0 && t == 0) {
            if (a.mean) a.mean[row] = (float)(pv + m1);
            if (a.rstd) a.rstd[row] = (float)scale;
        }
    } else {
        scale = rsqrt_f64(st.y * a.inv_nd + (double)a.eps);
    }
    const float scale_f = (float)scale;
    const double nm = -m1 * scale;                  // as in the single-pass kernels

    finish_row<DT, AL, K, TPR>(raw, geo, xr, t, N, 0u, cbase);     // padding is not stored
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float v[VEC], g[VEC], b[VEC];
        unpack<DT>(raw[k], v);
        if (has_p0) unpack<DT>(g4[k], g);
        if constexpr (OP == OP_LAYERNORM) {
            if (has_p1) unpack<DT>(b4[k], b);
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const float gi = has_p0 ? g[i] : 1.0f;
            if constexpr (OP == OP_LAYERNORM) {
                const double d = (double)v[i] - pv;
                v[i] = (float)__builtin_fma(__builtin_fma(d, scale, nm), (double)gi, has_p1 ? (double)b[i] : 0.0);
            } else {
                v[i] = (v[i] * scale_f) * gi;
            }
        }
        store_slice<DT, AL, TPR>(geo, yr, k, t, N, yvec, pack<DT>(v), cbase);
    }
}

// ---------------------------------------------------------------------------
// Split online softmax for rows too wide for one group's registers.
// The row is cut into P chunks of 64*W*K 16-byte pieces; workgroup b handles
// chunk j = b mod P of row r = b / P.  Per chunk: (m_j, l_j) = (max of the
// chunk, sum exp(x - m_j)); per row: m = max_j m_j, l = sum_j l_j*exp(m_j - m)
// (the online normalizer merge); then y = exp(x - m) / l on every chunk.
// ---------------------------------------------------------------------------

// (max, denominator) of one chunk of a softmax row, from its loaded and
// finished words: m_j = max over the chunk, l_j = sum of 2^(x*log2e - c_j)
// with c_j = m_j*log2e rounded to fp32.  Every path that needs a chunk's
// pair (the two-kernel split, the cooperative kernel for its own chunk and
// for a chunk it recomputes) calls this, so the pair is bitwise the same
// whichever workgroup computes it.
template <int DT, int W, int K>
__device__ __forceinline__ float2 chunk_stats(const uint4 (&raw)[K], float (&red)[2][W], int wv, int lane,
                                              float s2 = LOG2E) {
    constexpr int VEC = dt_info<DT>::VEC;
    // Each pass widens one 16-byte slice at a time (the same order as a
    // whole-chunk lane_max and sum), so no widened copy of the chunk stays
    // live beside the packed words the caller keeps for its output.
    float lm = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float v[VEC];
        unpack<DT>(raw[k], v);
#pragma unroll
        for (int i = 0; i < VEC; i += 2) lm = __builtin_fmaxf(lm, __builtin_fmaxf(v[i], v[i + 1]));
    }
    const float mx = group_allreduce<W>(lm, MaxOp(), red[0], wv, lane);
    const float cj = exp_offset(mx, s2);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        uint4 r = raw[k];
        if constexpr (DT != DT_F32)   // widen again rather than keep the first pass's values
            asm volatile("" : "+v"(r.x), "+v"(r.y), "+v"(r.z), "+v"(r.w));
        float v[VEC];
        unpack<DT>(r, v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) s += __builtin_amdgcn_exp2f(__builtin_fmaf(v[i], s2, -cj));
    }
    s = group_allreduce<W>(s, SumOp(), red[1], wv, lane);
    if (mx == -__builtin_inff()) s = 0.f;    // a fully masked chunk holds no mass
    return make_float2(mx, s);
}

// chunk_stats of a chunk that is not in registers (the cooperative kernel's
// recomputation of a missing record), reading it one 16-byte slice per lane
// at a time, twice: slice k holds exactly the words slot k of a whole-chunk
// load would (every slot depends only on its own chunk index), and the
// arithmetic runs in the same order, so the pair is bitwise chunk_stats'.
template <int DT, int W, int K, bool AL, bool CAUSAL>
__device__ __forceinline__ float2 chunk_stats_reload(const RowGeom<DT, AL> &geo, const char *xr, int t,
                                                        int32_t N, int32_t L, int64_t qbase,
                                                        float (&red)[2][W], int wv, int lane, float s2) {
    constexpr int VEC = dt_info<DT>::VEC, TPR = 64 * W;
    float lm = -__builtin_inff();
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
        uint4 r[1];
        softmax_issue<DT, AL, 1, TPR, CAUSAL>(r, geo, xr, t, N, L, qbase + (int64_t)k * TPR);
        softmax_finish<DT, AL, 1, TPR, CAUSAL>(r, geo, xr, t, N, L, qbase + (int64_t)k * TPR);
        float v[VEC];
        unpack<DT>(r[0], v);
#pragma unroll
        for (int i = 0; i < VEC; i += 2) lm = __builtin_fmaxf(lm, __builtin_fmaxf(v[i], v[i + 1]));
    }
    const float mx = group_allreduce<W>(lm, MaxOp(), red[0], wv, lane);
    const float cj = exp_offset(mx, s2);
    float s = 0.f;
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
        uint4 r[1];
        softmax_issue<DT, AL, 1, TPR, CAUSAL>(r, geo, xr, t, N, L, qbase + (int64_t)k * TPR);
        softmax_finish<DT, AL, 1, TPR, CAUSAL>(r, geo, xr, t, N, L, qbase + (int64_t)k * TPR);
        float v[VEC];
        unpack<DT>(r[0], v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) s += __builtin_amdgcn_exp2f(__builtin_fmaf(v[i], s2, -cj));
    }
    s = group_allreduce<W>(s, SumOp(), red[1], wv, lane);
    if (mx == -__builtin_inff()) s = 0.f;
    return make_float2(mx, s);
}

// Merge of a row's P chunk pairs q[0..P) (global or LDS) by one wave, in a
// fixed order: m = max_j m_j, l = sum_j l_j * 2^(c_j - c) with
// c = exp_offset(m) and c_j = exp_offset(m_j), the offsets the pairs were
// computed with (the online-normalizer rescaling).  Returns c and 1/l.
// Every wave that calls it on the same pairs gets the same bits.
template <class Q>
__device__ __forceinline__ void merge_pairs(Q q, int32_t P, int lane, float &c, float &inv, float s2 = LOG2E) {
    float m = -__builtin_inff();
    for (int p = lane; p < P; p += 64) m = __builtin_fmaxf(m, q[p].x);
    m = wave_allreduce(m, MaxOp());
    float l = 0.f;
    {
#pragma clang fp contract(off)
        c = exp_offset(m, s2);
        for (int p = lane; p < P; p += 64) {
            const float2 e = q[p];
            const float cj = exp_offset(e.x, s2);       // as chunk_stats computed it
            l += (e.x == -__builtin_inff()) ? 0.f : e.y * __builtin_amdgcn_exp2f(cj - c);
        }
    }
    l = wave_allreduce(l, SumOp());
    if (m == -__builtin_inff()) l = __builtin_nanf("");   // all -inf row: NaN, as the formula
    inv = rcp_approx(l);
}

// Output of one chunk: y = 2^(x*s2 - c) * (1/l), rounded once to the type.
template <int DT, int W, int K, bool AL>
__device__ __forceinline__ void softmax_chunk_out(const uint4 (&raw)[K], const RowGeom<DT, AL> &geo, char *yr, int t,
                                                  int32_t N, bool yvec, int64_t cbase, float c, float inv,
                                                  float s2 = LOG2E) {
    constexpr int VEC = dt_info<DT>::VEC, TPR = 64 * W;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float v[VEC];
        unpack<DT>(raw[k], v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[i], s2, -c)) * inv;
        store_slice<DT, AL, TPR>(geo, yr, k, t, N, yvec, pack<DT>(v), cbase);
    }
}

// Two-kernel form: the partial kernel writes each chunk's (m_j, l_j) to the
// workspace, the finalize kernel merges a row's pairs and writes the chunk's
// outputs (reading x a second time).

template <int DT, int W, int K, bool AL, bool CAUSAL = false>
__global__ void __launch_bounds__(64 * W)
softmax_split_partial(RowArgs a) {
    using I = dt_info<DT>;
    constexpr int TPR = 64 * W;
    const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
    const int32_t N = a.N, P = a.P;
    const int64_t row = blockIdx.x / P;
    const int64_t j = blockIdx.x - row * P;
    const char *xr = a.x + row * (int64_t)N * I::E;
    const RowGeom<DT, AL> geo(xr, N);
    __shared__ float red[2][W];

    uint4 raw[K];
    const int64_t cbase = j * (int64_t)(TPR * K);
    const int32_t L = CAUSAL ? visible_len(a, row) : N;
    const float s2 = CAUSAL ? a.s2 : LOG2E;
    // temporal loads: the finalize kernel reads this chunk again
    softmax_issue<DT, AL, K, TPR, CAUSAL, false>(raw, geo, xr, t, N, L, cbase);
    softmax_finish<DT, AL, K, TPR, CAUSAL>(raw, geo, xr, t, N, L, cbase);
    const float2 q = chunk_stats<DT, W, K>(raw, red, wv, lane, s2);
    if (t == 0) a.ws[row * P + j] = q;
}

template <int DT, int W, int K, bool AL, bool CAUSAL = false>
__global__ void __launch_bounds__(64 * W)
softmax_split_finalize(RowArgs a) {
    using I = dt_info<DT>;
    constexpr int TPR = 64 * W;
    const int t = threadIdx.x, lane = t & 63;
    const int32_t N = a.N, P = a.P;
    const int64_t row = blockIdx.x / P;
    const int64_t j = blockIdx.x - row * P;
    const int64_t rowbytes = (int64_t)N * I::E;
    const char *xr = a.x + row * rowbytes;
    char *yr = a.y + row * rowbytes;
    const RowGeom<DT, AL> geo(xr, N);
    bool yvec = true;
    if constexpr (!AL) yvec = (((uintptr_t)yr ^ (uintptr_t)xr) & 15) == 0;

    // issue the chunk loads first so their latency overlaps the merge
    uint4 raw[K];
    const int64_t cbase = j * (int64_t)(TPR * K);
    const int32_t L = CAUSAL ? visible_len(a, row) : N;
    const float s2 = CAUSAL ? a.s2 : LOG2E;
    softmax_issue<DT, AL, K, TPR, CAUSAL>(raw, geo, xr, t, N, L, cbase);

    // every wave merges the row's pairs redundantly, in the same order
    float c, inv;
    merge_pairs(a.ws + row * P, P, lane, c, inv, s2);
    softmax_finish<DT, AL, K, TPR, CAUSAL>(raw, geo, xr, t, N, L, cbase);
    softmax_chunk_out<DT, W, K, AL>(raw, geo, yr, t, N, yvec, cbase, c, inv, s2);
}

// ---------------------------------------------------------------------------
// Cooperative split softmax: the same chunks and arithmetic as the two
// kernels above in ONE pass, so x is read once.  Each workgroup loads its
// chunk, computes (m_j, l_j), and publishes it as a record of two 64-bit
// words {tag, bits of m_j} and {tag, bits of l_j}, each written and read as
// one relaxed device-scope atomic; `tag` is unique to the call, so a record
// is valid only if both words carry it and the workspace needs no clearing.
// Wave 0 then polls the row's other records.  A record still missing after
// `spin` polls is recomputed from x by this workgroup itself (chunk_stats on
// the same chunk gives the same bits), so the result never depends on which
// workgroups run at the same time and every wait is bounded.  The merge and
// the output are those of the finalize kernel, so both paths agree bitwise.
// x must not alias y: a recomputed chunk may already have been overwritten.
// ---------------------------------------------------------------------------

constexpr int COOP_PMAX = 128;    // chunks per row the cooperative kernel accepts

template <int DT, int W, int K, bool AL, bool CAUSAL = false>
__global__ void __launch_bounds__(64 * W)
softmax_coop(RowArgs a) {
    using I = dt_info<DT>;
    constexpr int TPR = 64 * W, NB = COOP_PMAX / 64;
    const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
    const int32_t N = a.N, P = a.P;
    const int64_t row = blockIdx.x / P;
    const int j = (int)(blockIdx.x - row * P);
    const int64_t rowbytes = (int64_t)N * I::E;
    const char *xr = a.x + row * rowbytes;
    char *yr = a.y + row * rowbytes;
    const RowGeom<DT, AL> geo(xr, N);
    bool yvec = true;
    if constexpr (!AL) yvec = (((uintptr_t)yr ^ (uintptr_t)xr) & 15) == 0;
    __shared__ float red[2][W];
    __shared__ float2 qs[COOP_PMAX];
    __shared__ uint64_t miss[NB];

    uint4 raw[K];
    const int64_t cbase = (int64_t)j * (TPR * K);
    const int32_t L = CAUSAL ? visible_len(a, row) : N;
    const float s2 = CAUSAL ? a.s2 : LOG2E;
    softmax_issue<DT, AL, K, TPR, CAUSAL>(raw, geo, xr, t, N, L, cbase);
    softmax_finish<DT, AL, K, TPR, CAUSAL>(raw, geo, xr, t, N, L, cbase);
    const float2 mine = chunk_stats<DT, W, K>(raw, red, wv, lane, s2);

    uint64_t *rec = reinterpret_cast<uint64_t *>(a.ws) + row * P * 2;
    const uint32_t tag = call_tag(a);
    const uint64_t tg = (uint64_t)tag << 32;
    if (t == 0) {
        __hip_atomic_store(rec + 2 * j, tg | __float_as_uint(mine.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(rec + 2 * j + 1, tg | __float_as_uint(mine.y), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        qs[j] = mine;
    }
    if (wv == 0) {
        // bit b of `pending`: this lane's record b*64 + lane is still missing
        uint32_t pending = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int p = b * 64 + lane;
            if (p < P && p != j) pending |= 1u << b;
        }
        for (int it = 0;; ++it) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (pending >> b & 1) {
                    const int p = b * 64 + lane;
                    const uint64_t w0 = __hip_atomic_load(rec + 2 * p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const uint64_t w1 =
                        __hip_atomic_load(rec + 2 * p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if ((w0 >> 32) == tag && (w1 >> 32) == tag) {
                        qs[p] = make_float2(__uint_as_float((uint32_t)w0), __uint_as_float((uint32_t)w1));
                        pending &= ~(1u << b);
                    }
                }
            }
            if (__ballot(pending != 0) == 0 || it >= a.spin) break;
            __builtin_amdgcn_s_sleep(2);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint64_t m = __ballot((pending >> b) & 1);
            if (lane == 0) miss[b] = m;
        }
    }
    __syncthreads();
    // records that did not arrive: recompute them here (uniform loop)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        uint64_t m = miss[b];
        while (m) {
            const int q = b * 64 + __builtin_ctzll(m);
            m &= m - 1;
            const float2 e = chunk_stats_reload<DT, W, K, AL, CAUSAL>(geo, xr, t, N, L, (int64_t)q * (TPR * K), red,
                                                                      wv, lane, s2);
            if (t == 0) qs[q] = e;
        }
    }
    __syncthreads();
    float c, inv;
    merge_pairs(static_cast<const float2 *>(qs), P, lane, c, inv, s2);
    softmax_chunk_out<DT, W, K, AL>(raw, geo, yr, t, N, yvec, cbase, c, inv, s2);
}

// ---------------------------------------------------------------------------
// The cooperative split softmax with two rows per workgroup: workgroup
// (g, j) takes chunk j of rows g and g + G (G = ceil(M / 2)), one after the
// other, with the same record protocol as softmax_coop.  The second row's
// loads are issued as soon as the first row's record is published, so they
// are in flight while the first row's other records arrive and its output
// is written: one row's reads overlap the other row's writes, where one row
// per workgroup reads every row first and writes every row after.  Both
// rows give the bits softmax_coop gives (same chunk_stats, merge, output).
// ---------------------------------------------------------------------------

template <int DT, int W, int K, bool AL, bool CAUSAL = false>
__global__ void __launch_bounds__(64 * W)
softmax_coop2(RowArgs a) {
    using I = dt_info<DT>;
    constexpr int TPR = 64 * W, NB = COOP_PMAX / 64;
    const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
    const int32_t N = a.N, P = a.P;
    const int64_t G = (a.M + 1) / 2;
    const int64_t g = blockIdx.x / P;
    const int j = (int)(blockIdx.x - g * P);
    const int64_t rowbytes = (int64_t)N * I::E;
    const int64_t cbase = (int64_t)j * (TPR * K);
    const float s2 = CAUSAL ? a.s2 : LOG2E;
    const uint32_t tag = call_tag(a);
    const uint64_t tg = (uint64_t)tag << 32;
    const bool two = g + G < a.M;                  // uniform: a second row exists
    __shared__ float red[2][W];
    __shared__ float2 qs[COOP_PMAX];
    __shared__ uint64_t miss[NB];

    uint4 raw[2][K];
    {
        const char *xr = a.x + g * rowbytes;
        softmax_issue<DT, AL, K, TPR, CAUSAL>(raw[0], RowGeom<DT, AL>(xr, N), xr, t, N,
                                              CAUSAL ? visible_len(a, g) : N, cbase);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (i == 1 && !two) break;
        const int64_t row = g + i * G;
        const char *xr = a.x + row * rowbytes;
        char *yr = a.y + row * rowbytes;
        const RowGeom<DT, AL> geo(xr, N);
        bool yvec = true;
        if constexpr (!AL) yvec = (((uintptr_t)yr ^ (uintptr_t)xr) & 15) == 0;
        const int32_t L = CAUSAL ? visible_len(a, row) : N;
        softmax_finish<DT, AL, K, TPR, CAUSAL>(raw[i], geo, xr, t, N, L, cbase);
        const float2 mine = chunk_stats<DT, W, K>(raw[i], red, wv, lane, s2);

        uint64_t *rec = reinterpret_cast<uint64_t *>(a.ws) + row * P * 2;
        if (t == 0) {
            __hip_atomic_store(rec + 2 * j, tg | __float_as_uint(mine.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(rec + 2 * j + 1, tg | __float_as_uint(mine.y), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            qs[j] = mine;
        }
        if (i == 0 && two) {
            // the second row's loads, in flight during this row's exchange and output
            asm volatile("" ::: "memory");
            const char *xn = a.x + (g + G) * rowbytes;
            softmax_issue<DT, AL, K, TPR, CAUSAL>(raw[1], RowGeom<DT, AL>(xn, N), xn, t, N,
                                                  CAUSAL ? visible_len(a, g + G) : N, cbase);
            asm volatile("" ::: "memory");
        }
        if (wv == 0) {
            uint32_t pending = 0;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int p = b * 64 + lane;
                if (p < P && p != j) pending |= 1u << b;
            }
            for (int it = 0;; ++it) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (pending >> b & 1) {
                        const int p = b * 64 + lane;
                        const uint64_t w0 = __hip_atomic_load(rec + 2 * p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        const uint64_t w1 =
                            __hip_atomic_load(rec + 2 * p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if ((w0 >> 32) == tag && (w1 >> 32) == tag) {
                            qs[p] = make_float2(__uint_as_float((uint32_t)w0), __uint_as_float((uint32_t)w1));
                            pending &= ~(1u << b);
                        }
                    }
                }
                if (__ballot(pending != 0) == 0 || it >= a.spin) break;
                __builtin_amdgcn_s_sleep(2);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint64_t m = __ballot((pending >> b) & 1);
                if (lane == 0) miss[b] = m;
            }
        }
        __syncthreads();
        // records that did not arrive: recompute them here (uniform loop)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            uint64_t m = miss[b];
            while (m) {
                const int q = b * 64 + __builtin_ctzll(m);
                m &= m - 1;
                const float2 e = chunk_stats_reload<DT, W, K, AL, CAUSAL>(geo, xr, t, N, L, (int64_t)q * (TPR * K),
                                                                          red, wv, lane, s2);
                if (t == 0) qs[q] = e;
            }
        }
        __syncthreads();
        float c, inv;
        merge_pairs(static_cast<const float2 *>(qs), P, lane, c, inv, s2);
        softmax_chunk_out<DT, W, K, AL>(raw[i], geo, yr, t, N, yvec, cbase, c, inv, s2);
        __syncthreads();                           // qs and miss are the next row's
    }
}

// ---------------------------------------------------------------------------
// Cooperative split norm: the split norm's chunks and arithmetic in ONE
// pass, so x is read once.  The record exchange is the cooperative softmax's
// (tagged 64-bit words, written and read as relaxed device-scope atomics, a
// bounded poll by wave 0, then recomputation of whatever did not arrive),
// with fp64 sums: a record is four words {tag, low or high half of s1 or
// s2}.  The row's sums are combined in the finalize kernel's order, so both
// forms give the same bits.  x must not alias y (a recomputed chunk may
// already hold outputs), and the parameters are loaded with the chunk.
// ---------------------------------------------------------------------------

template <int OP, int DT, int W, int K, bool AL>
__global__ void __launch_bounds__(64 * W)
norm_coop(RowArgs a) {
    static_assert(OP == OP_LAYERNORM || OP == OP_RMSNORM, "split norm");
    using I = dt_info<DT>;
    constexpr int VEC = I::VEC, TPR = 64 * W, NB = COOP_PMAX / 64;
    constexpr int NW = OP == OP_LAYERNORM ? 4 : 2;      // record words: s1 (LayerNorm) and s2, two halves each
    const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
    const int32_t N = a.N, P = a.P;
    const int64_t row = blockIdx.x / P;
    const int j = (int)(blockIdx.x - row * P);
    const int64_t rowbytes = (int64_t)N * I::E;
    const char *xr = a.x + row * rowbytes;
    char *yr = a.y + row * rowbytes;
    const RowGeom<DT, AL> geo(xr, N);
    bool yvec = true;
    if constexpr (!AL) yvec = (((uintptr_t)yr ^ (uintptr_t)xr) & 15) == 0;
    const bool has_p0 = a.p0 != nullptr, has_p1 = a.p1 != nullptr;
    __shared__ double2 red[2][W];
    __shared__ double2 qs[COOP_PMAX];
    __shared__ uint64_t miss[NB];

    const int64_t cbase = (int64_t)j * (TPR * K);
    uint32_t padw = 0;
    if constexpr (OP == OP_LAYERNORM) padw = pivot_word<DT>(xr);
    const double pv = (double)elem_of_word<DT>(padw);
    uint4 raw[K], g4[K], b4[(OP == OP_LAYERNORM) ? K : 1];
    load_row<DT, AL, K, TPR>(raw, geo, t, N, cbase);
    if (has_p0) load_params<DT, AL, K, TPR>(g4, geo, a.p0, t, N, cbase);
    if constexpr (OP == OP_LAYERNORM) {
        if (has_p1) load_params<DT, AL, K, TPR>(b4, geo, a.p1, t, N, cbase);
    }
    finish_row<DT, AL, K, TPR>(raw, geo, xr, t, N, padw, cbase);
    const double2 mine = norm_chunk_sums<OP, DT, W, K>(raw, pv, red[0], wv, lane);

    uint64_t *rec = reinterpret_cast<uint64_t *>(a.wsd) + row * P * NW;
    const uint32_t tag = call_tag(a);
    const uint64_t tg = (uint64_t)tag << 32;
    if (t == 0) {
        const uint64_t b1 = (uint64_t)__double_as_longlong(mine.x), b2 = (uint64_t)__double_as_longlong(mine.y);
        uint64_t *r = rec + (int64_t)NW * j;
        __hip_atomic_store(r, tg | (b2 & 0xffffffffu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(r + 1, tg | (b2 >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (NW == 4) {
            __hip_atomic_store(r + 2, tg | (b1 & 0xffffffffu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(r + 3, tg | (b1 >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        qs[j] = mine;
    }
    if (wv == 0) {
        // bit b of `pending`: this lane's record b*64 + lane is still missing
        uint32_t pending = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int p = b * 64 + lane;
            if (p < P && p != j) pending |= 1u << b;
        }
        for (int it = 0;; ++it) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (pending >> b & 1) {
                    const uint64_t *r = rec + (int64_t)NW * (b * 64 + lane);
                    uint64_t w[NW];
                    bool ok = true;
#pragma unroll
                    for (int q = 0; q < NW; ++q) {
                        w[q] = __hip_atomic_load(r + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        ok = ok && (w[q] >> 32) == tag;
                    }
                    if (ok) {
                        const double s2 = __longlong_as_double((long long)((w[0] & 0xffffffffu) | (w[1] << 32)));
                        double s1 = 0.0;
                        if constexpr (NW == 4)
                            s1 = __longlong_as_double((long long)((w[2] & 0xffffffffu) | (w[3] << 32)));
                        qs[b * 64 + lane] = double2{s1, s2};
                        pending &= ~(1u << b);
                    }
                }
            }
            if (__ballot(pending != 0) == 0 || it >= a.spin) break;
            __builtin_amdgcn_s_sleep(2);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint64_t m = __ballot((pending >> b) & 1);
            if (lane == 0) miss[b] = m;
        }
    }
    __syncthreads();
    // records that did not arrive: recompute them here (uniform loop; the
    // reductions alternate between the two LDS slots)
    int par = 1;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        uint64_t m = miss[b];
        while (m) {
            const int q = b * 64 + __builtin_ctzll(m);
            m &= m - 1;
            const double2 e = norm_chunk_sums_reload<OP, DT, W, K, AL>(geo, xr, t, N, padw, pv,
                                                                       (int64_t)q * (TPR * K), red[par], wv, lane);
            par ^= 1;
            if (t == 0) qs[q] = e;
        }
    }
    __syncthreads();

    // the row's sums in the finalize kernel's order: lane l takes l, l + 64, ...
    double s1 = 0.0, s2 = 0.0;
    for (int q = lane; q < P; q += 64) {
        s1 += qs[q].x;
        s2 += qs[q].y;
    }
    const double2 st = wave_allreduce(double2{s1, s2}, SumOp());
    double m1 = 0.0, scale;
    if constexpr (OP == OP_LAYERNORM) {
        m1 = st.x * a.inv_nd;
        const double var = __builtin_fmax(st.y * a.inv_nd - m1 * m1, 0.0);
        scale = rsqrt_f64(var + (double)a.eps);
        if (j == 0 && t == 0) {
            if (a.mean) a.mean[row] = (float)(pv + m1);
            if (a.rstd) a.rstd[row] = (float)scale;
        }
    } else {
        scale = rsqrt_f64(st.y * a.inv_nd + (double)a.eps);
    }
    const float scale_f = (float)scale;
    const double nm = -m1 * scale;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float v[VEC], g[VEC], b[VEC];
        unpack<DT>(raw[k], v);
        if (has_p0) unpack<DT>(g4[k], g);
        if constexpr (OP == OP_LAYERNORM) {
            if (has_p1) unpack<DT>(b4[k], b);
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const float gi = has_p0 ? g[i] : 1.0f;
            if constexpr (OP == OP_LAYERNORM) {
                const double d = (double)v[i] - pv;
                v[i] = (float)__builtin_fma(__builtin_fma(d, scale, nm), (double)gi, has_p1 ? (double)b[i] : 0.0);
            } else {
                v[i] = (v[i] * scale_f) * gi;
            }
        }
        store_slice<DT, AL, TPR>(geo, yr, k, t, N, yvec, pack<DT>(v), cbase);
    }
}

}  // namespace ntk
