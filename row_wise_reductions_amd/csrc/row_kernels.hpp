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
// Two variants of every kernel exist:
//   AL = true   every row start, x, y and the parameter vectors are 16-byte
//               aligned and N*sizeof(T) is a multiple of 16: whole chunks only.
//   AL = false  rows start anywhere (element-aligned).  Chunks are cut on the
//               16-byte grid of x; the partial first and last chunk of a row
//               are gathered and scattered element by element, and the
//               parameter vectors are read per element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ntk {

enum { OP_SOFTMAX = 0, OP_LAYERNORM = 1, OP_RMSNORM = 2 };
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
    const char *p0;      // gamma (LayerNorm) or weight (RMSNorm); may be null
    const char *p1;      // beta (LayerNorm); may be null
    float *mean;         // LayerNorm statistics outputs; may be null
    float *rstd;
    float2 *ws;          // split softmax: (max, denominator) per (row, chunk)
    int64_t M;
    int32_t N;
    int32_t P;           // split softmax: chunks per row
    float eps;
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// 16-byte chunk <-> fp32 values
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint4 ld16(const char *p) {
    return *reinterpret_cast<const uint4 *>(p);
}
__device__ __forceinline__ void st16(char *p, uint4 v) {
    *reinterpret_cast<uint4 *>(p) = v;
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
        // bf16 is the top half of a binary32: widening is a shift.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
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

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = dpp_i<CTRL>((int)(uint32_t)u);
    const int hi = dpp_i<CTRL>((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
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

struct SumOp {
    template <class V> __device__ __forceinline__ V operator()(V a, V b) const { return a + b; }
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

// Store chunk c of a row.  `yvec` tells whether y shares x's 16-byte phase
// (then whole chunks are stored as vectors).
template <int DT, bool AL>
__device__ __forceinline__ void store_chunk(const RowGeom<DT, AL> &g, char *yr, int64_t c, int32_t N,
                                            bool yvec, uint4 v) {
    if (c < g.nch) {
        if constexpr (AL) {
            st16(yr + c * 16, v);
        } else {
            if (yvec && g.full(c, N))
                st16(yr - (int64_t)g.head * dt_info<DT>::E + c * 16, v);
            else
                scatter<DT>(yr, g.col0(c), N, v);
        }
    }
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

__device__ __forceinline__ float fast_exp(float t) {
    // e^t = 2^(t * log2 e); v_exp_f32 evaluates 2^x.
    return __builtin_amdgcn_exp2f(t * LOG2E);
}

// ---------------------------------------------------------------------------
// Single-pass kernel: one row per group of W waves, row held in VGPRs.
// W == 1: four independent rows per 256-thread workgroup, no LDS or barrier.
// W >= 2: one row per workgroup of 64*W threads.
// ---------------------------------------------------------------------------

template <int W>
struct GroupShape {
    static constexpr int G = (W == 1) ? 4 : 1;           // rows per workgroup
    static constexpr int THREADS = 64 * W * G;
};

template <int OP, int DT, int W, int K, bool AL>
__global__ void __launch_bounds__(GroupShape<W>::THREADS)
row_resident(RowArgs a) {
    using I = dt_info<DT>;
    constexpr int VEC = I::VEC, TPR = 64 * W, G = GroupShape<W>::G;
    const int tid = threadIdx.x;
    const int g = (W == 1) ? (tid >> 6) : 0;
    const int t = (W == 1) ? (tid & 63) : tid;
    const int wv = t >> 6, lane = t & 63;
    const int32_t N = a.N;
    const int64_t rowbytes = (int64_t)N * I::E;
    const uint32_t fill = (OP == OP_SOFTMAX) ? I::NEG_INF_WORD : 0u;

    __shared__ float red_f[2][2][W];
    __shared__ double red_d[2][2][W];

    const int64_t nrb = (a.M + G - 1) / G;
    int par = 0;
    for (int64_t rb = blockIdx.x; rb < nrb; rb += gridDim.x, par ^= 1) {
        const int64_t row = rb * G + g;
        if (row >= a.M) break;   // only possible when W == 1 (no barriers there)
        const char *xr = a.x + row * rowbytes;
        char *yr = a.y + row * rowbytes;
        const RowGeom<DT, AL> geo(xr, N);
        bool yvec = true;
        if constexpr (!AL) yvec = (((uintptr_t)yr ^ (uintptr_t)xr) & 15) == 0;

        // ---- load the whole row: K chunks per lane, all in flight at once
        uint4 raw[K];
#pragma unroll
        for (int k = 0; k < K; ++k) raw[k] = load_chunk<DT, AL>(geo, xr, (int64_t)k * TPR + t, N, fill);
        uint4 p0[(OP == OP_SOFTMAX) ? 1 : K];
        uint4 p1[(OP == OP_LAYERNORM) ? K : 1];
        if constexpr (OP != OP_SOFTMAX) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int64_t c = (int64_t)k * TPR + t;
                p0[k] = a.p0 ? load_param<DT, AL>(geo, a.p0, c, N) : make_uint4(0, 0, 0, 0);
                if constexpr (OP == OP_LAYERNORM)
                    p1[k] = a.p1 ? load_param<DT, AL>(geo, a.p1, c, N) : make_uint4(0, 0, 0, 0);
            }
        }
        float v[K][VEC];
#pragma unroll
        for (int k = 0; k < K; ++k) unpack<DT>(raw[k], v[k]);

        if constexpr (OP == OP_SOFTMAX) {
            // ---- max, shift, exp, sum, scale
            float mx = -__builtin_inff();
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int i = 0; i < VEC; ++i) mx = __builtin_fmaxf(mx, v[k][i]);
            mx = group_allreduce<W>(mx, MaxOp(), red_f[par][0], wv, lane);
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    v[k][i] = fast_exp(v[k][i] - mx);
                    s += v[k][i];
                }
            s = group_allreduce<W>(s, SumOp(), red_f[par][1], wv, lane);
            const float inv = 1.0f / s;
#pragma unroll
            for (int k = 0; k < K; ++k) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) v[k][i] *= inv;
                store_chunk<DT, AL>(geo, yr, (int64_t)k * TPR + t, N, yvec, pack<DT>(v[k]));
            }
        } else if constexpr (OP == OP_RMSNORM) {
            // ---- sum of squares (fp32), scale by the row's 1/rms and the weight
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int i = 0; i < VEC; ++i) ss = __builtin_fmaf(v[k][i], v[k][i], ss);
            ss = group_allreduce<W>(ss, SumOp(), red_f[par][0], wv, lane);
            const float inv = (float)(1.0 / __builtin_sqrt((double)ss / (double)N + (double)a.eps));
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float w[VEC];
                if (a.p0) {
                    unpack<DT>(p0[k], w);
                } else {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) w[i] = 1.0f;
                }
#pragma unroll
                for (int i = 0; i < VEC; ++i) v[k][i] = (v[k][i] * inv) * w[i];
                store_chunk<DT, AL>(geo, yr, (int64_t)k * TPR + t, N, yvec, pack<DT>(v[k]));
            }
        } else {
            // ---- LayerNorm: row sums and the affine step in fp64
            double s1 = 0.0;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int i = 0; i < VEC; ++i) s1 += (double)v[k][i];   // padding is 0
            s1 = group_allreduce<W>(s1, SumOp(), red_d[par][0], wv, lane);
            const double mean = s1 / (double)N;
            double s2 = 0.0;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const double d = (double)v[k][i] - mean;
                    s2 = in_row<DT, AL>(geo, (int64_t)k * TPR + t, i, N) ? __builtin_fma(d, d, s2) : s2;
                }
            s2 = group_allreduce<W>(s2, SumOp(), red_d[par][1], wv, lane);
            const double rstd = 1.0 / __builtin_sqrt(s2 / (double)N + (double)a.eps);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float gm[VEC], bt[VEC];
                if (a.p0) {
                    unpack<DT>(p0[k], gm);
                } else {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) gm[i] = 1.0f;
                }
                if (a.p1) {
                    unpack<DT>(p1[k], bt);
                } else {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) bt[i] = 0.0f;
                }
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const double d = ((double)v[k][i] - mean) * rstd;
                    v[k][i] = (float)__builtin_fma(d, (double)gm[i], (double)bt[i]);
                }
                store_chunk<DT, AL>(geo, yr, (int64_t)k * TPR + t, N, yvec, pack<DT>(v[k]));
            }
            if (t == 0) {
                if (a.mean) a.mean[row] = (float)mean;
                if (a.rstd) a.rstd[row] = (float)rstd;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Split online softmax for rows too wide for one group's registers.
// The row is cut into P chunks of 64*W*K 16-byte pieces; workgroup b handles
// chunk j = b mod P of row r = b / P.
//   split_partial:  (m_j, l_j) = (max of chunk, sum exp(x - m_j)) -> ws[r*P + j]
//   split_finalize: m = max_j m_j, l = sum_j l_j * exp(m_j - m) (the online
//                   normalizer merge), then y = exp(x - m) / l on its chunk.
// ---------------------------------------------------------------------------

template <int DT, int W, int K, bool AL>
__global__ void __launch_bounds__(64 * W)
softmax_split_partial(RowArgs a) {
    using I = dt_info<DT>;
    constexpr int VEC = I::VEC, TPR = 64 * W;
    const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
    const int32_t N = a.N, P = a.P;
    const int64_t row = blockIdx.x / P;
    const int64_t j = blockIdx.x - row * P;
    const char *xr = a.x + row * (int64_t)N * I::E;
    const RowGeom<DT, AL> geo(xr, N);
    __shared__ float red[2][W];

    uint4 raw[K];
    const int64_t cbase = j * (int64_t)(TPR * K);
#pragma unroll
    for (int k = 0; k < K; ++k)
        raw[k] = load_chunk<DT, AL>(geo, xr, cbase + (int64_t)k * TPR + t, N, I::NEG_INF_WORD);
    float v[K][VEC];
#pragma unroll
    for (int k = 0; k < K; ++k) unpack<DT>(raw[k], v[k]);
    float mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) mx = __builtin_fmaxf(mx, v[k][i]);
    mx = group_allreduce<W>(mx, MaxOp(), red[0], wv, lane);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int i = 0; i < VEC; ++i) s += fast_exp(v[k][i] - mx);
    s = group_allreduce<W>(s, SumOp(), red[1], wv, lane);
    if (mx == -__builtin_inff()) s = 0.f;    // a fully masked chunk holds no mass
    if (t == 0) a.ws[row * P + j] = make_float2(mx, s);
}

template <int DT, int W, int K, bool AL>
__global__ void __launch_bounds__(64 * W)
softmax_split_finalize(RowArgs a) {
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

    // issue the chunk loads first so their latency overlaps the merge
    uint4 raw[K];
    const int64_t cbase = j * (int64_t)(TPR * K);
#pragma unroll
    for (int k = 0; k < K; ++k)
        raw[k] = load_chunk<DT, AL>(geo, xr, cbase + (int64_t)k * TPR + t, N, I::NEG_INF_WORD);

    // merge the row's P partials; every wave does it redundantly, in the
    // same order, so every workgroup of the row gets identical (m, l)
    const float2 *wr = a.ws + row * P;
    float m = -__builtin_inff();
    for (int p = lane; p < P; p += 64) m = __builtin_fmaxf(m, wr[p].x);
    m = wave_allreduce(m, MaxOp());
    float l = 0.f;
    for (int p = lane; p < P; p += 64) {
        const float2 q = wr[p];
        l += (q.x == -__builtin_inff()) ? 0.f : q.y * fast_exp(q.x - m);
    }
    l = wave_allreduce(l, SumOp());
    if (m == -__builtin_inff()) l = __builtin_nanf("");   // all -inf row: NaN, as the formula
    const float inv = 1.0f / l;

#pragma unroll
    for (int k = 0; k < K; ++k) {
        float v[VEC];
        unpack<DT>(raw[k], v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[i] = fast_exp(v[i] - m) * inv;
        store_chunk<DT, AL>(geo, yr, cbase + (int64_t)k * TPR + t, N, yvec, pack<DT>(v));
    }
}

}  // namespace ntk
