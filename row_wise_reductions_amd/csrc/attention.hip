// Attention forward with the online softmax, for gfx950 (MI355X, CDNA4):
//   o[b, i, :] = softmax_j(scale * q[b, i, :] . k[b, j, :]) v[b, j, :]
// over the keys j visible to query i (all Lk, or j <= i + offset when
// causal), without materializing the scores: the loop over key/value tiles
// of "Triton: Block-Level GPU Programming Without CUDA", section "How Flash
// Attention Uses Triton" (per tile: the scores, the running max, the rescale
// alpha = 2^(m_prev - m_new) of the accumulator and of the denominator, the
// P V product), on the matrix cores.
//
// Workgroup: 4 waves, 128 queries of one head (32 per wave); key tiles of 64.
// Per tile the workgroup stages K (row-major, rows padded by 16 bytes) and V
// transposed (one row per head-dimension index, padded by 8 bytes) in LDS,
// while the next tile's rows are already being loaded into registers.
//
// Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16 (A = K rows from
// LDS, B = Q^T: the wave's 32 query rows held in registers for the whole
// kernel).  In the accumulator layout of that instruction lane l holds, for
// query l mod 32, the scores of keys 8*(r/4) + 4*(l/32) + r%4 of a 32-key
// block (r = 0..15), so a query's row max and sum need one exchange between
// lanes l and l^32, and the accumulator rescale is one multiply per
// register.  The weights P^T (fp32) are split into P_hi + P_lo, both 16-bit
// (each value kept to 16 significant bits, the bfloat16x2 / half x2 split of
// Henry, Tang and Heinecke, "Leveraging the bfloat16 Artificial Intelligence
// Datatype For Higher-Precision Computations", 2019), and fed straight from
// those registers as the B operand of O^T += V^T P_hi + V^T P_lo: the 8 key
// slots an MFMA step takes from lane l are the keys that lane already holds,
// and V^T's A operand reads the same keys from LDS.  Products are exact and
// every sum is accumulated in fp32 ("Portable Triton Kernels", "Numerics":
// fp32 accumulation).
//
// Causal and ragged tiles: scores of keys >= Lk or > query + offset become
// -inf (their weights exactly 0); only the tiles that can hold such keys are
// masked.  Loads of rows past Lq or Lk are clamped to the last row (never
// out of bounds); their results are discarded.  Query blocks are dealt
// heaviest first (most key tiles under a causal mask), heads interleaved.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attention.hpp"
#include "row_kernels.hpp"

namespace ntk {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

template <int DT> struct Mma;
template <> struct Mma<DT_BF16> {
    typedef bf16x8 E8;
    typedef bf16x2v E2;
    static __device__ __forceinline__ f32x16 mma(E8 a, E8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<DT_F16> {
    typedef f16x8 E8;
    typedef f16x2v E2;
    static __device__ __forceinline__ f32x16 mma(E8 a, E8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int BM = 128;       // queries per workgroup
constexpr int BN = 64;        // keys per tile
constexpr int NT = 256;       // threads per workgroup

// Eight consecutive 16-bit values at p (16-byte aligned) as an operand.
template <class E8>
__device__ __forceinline__ E8 ld8(const char *p) {
    return __builtin_bit_cast(E8, *reinterpret_cast<const uint4 *>(p));
}

// Two 4-element halves (8-byte aligned each) as one 8-element operand.
template <class E8>
__device__ __forceinline__ E8 ld4x2(const char *p0, const char *p1) {
    const uint2 a = *reinterpret_cast<const uint2 *>(p0), b = *reinterpret_cast<const uint2 *>(p1);
    return __builtin_bit_cast(E8, make_uint4(a.x, a.y, b.x, b.y));
}

// p (8 weights) = hi + lo, both in the 16-bit type, each rounded to nearest:
// hi holds p's leading bits, lo the next ones (p - hi is exact in fp32).
template <int DT>
__device__ __forceinline__ void split16(const float (&p)[8], typename Mma<DT>::E8 &hi, typename Mma<DT>::E8 &lo) {
    typedef typename Mma<DT>::E2 E2;
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x2 v = {p[2 * j], p[2 * j + 1]};
        const E2 h = __builtin_convertvector(v, E2);
        const f32x2 hf = __builtin_convertvector(h, f32x2);
        const f32x2 r = {v.x - hf.x, v.y - hf.y};
        wh[j] = __builtin_bit_cast(uint32_t, h);
        wl[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, E2));
    }
    hi = __builtin_bit_cast(typename Mma<DT>::E8, make_uint4(wh[0], wh[1], wh[2], wh[3]));
    lo = __builtin_bit_cast(typename Mma<DT>::E8, make_uint4(wl[0], wl[1], wl[2], wl[3]));
}

// Issue the loads of one key tile's K and V rows (keys j0 .. j0 + 63, clamped
// to the last key): K as contiguous 16-byte chunks per thread, V one key per
// lane, so that a wave's transposed LDS writes fill consecutive bytes.
template <int D, int KCH, int VCH>
__device__ __forceinline__ void load_tile(u32x4 (&kr)[KCH], uint4 (&vr)[VCH], const char *kb0, const char *vb0,
                                          int64_t j0, int64_t Lk, int tid) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const int idx = tid + NT * c, key = idx / (D / 8), dc = idx % (D / 8);
        int64_t kj = j0 + key;
        kj = kj < Lk ? kj : Lk - 1;
        kr[c] = *reinterpret_cast<const u32x4 *>(kb0 + (kj * D + dc * 8) * 2);
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
        const int key = tid % BN, dc = tid / BN + (NT / BN) * c;
        int64_t kj = j0 + key;
        kj = kj < Lk ? kj : Lk - 1;
        vr[c] = *reinterpret_cast<const uint4 *>(vb0 + (kj * D + dc * 8) * 2);
    }
}

// The reference max of a query's weights moves only when a tile's scores
// exceed it by more than 2^RESCALE_SLACK (base-2 exponent); until then the
// weights are 2^(s - m_ref) <= 2^RESCALE_SLACK, far inside fp32 and both
// 16-bit types, and the accumulator is not rescaled.  Any reference gives
// the same result in real arithmetic (the rescale factor cancels).
constexpr float RESCALE_SLACK = 8.0f;

// Two waves per SIMD (one to issue matrix instructions while the other runs
// the softmax): the compiler keeps the kernel within 256 registers, the
// accumulators in architectural VGPRs, where the rescale can reach them.
template <int DT, int D>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) attention_fwd(AttnArgs a) {
    typedef typename Mma<DT>::E8 E8;
    constexpr int KSTR = D * 2 + 16;               // bytes per K row in LDS
    constexpr int VSTR = BN * 2 + 8;               // bytes per V^T row (one head-dim index) in LDS
    constexpr int KCH = BN * D * 2 / 16 / NT;      // 16-byte K chunks per thread per tile
    constexpr int VCH = D / 8 / (NT / BN);         // 16-byte V chunks per thread per tile
    static_assert(KCH >= 1 && VCH >= 1, "tile shape");
    __shared__ __attribute__((aligned(16))) char ks[BN * KSTR];
    __shared__ __attribute__((aligned(16))) char vs[D * VSTR];

    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, h = lane >> 5, ql = lane & 31;
    const int64_t nblk = a.BH * a.nqb;
    if ((int64_t)blockIdx.x >= nblk) return;
    const int64_t qblk = a.nqb - 1 - (int64_t)blockIdx.x / a.BH;     // heaviest first
    const int64_t b = (int64_t)blockIdx.x % a.BH;
    const int64_t q0 = qblk * BM;
    const int64_t qw = q0 + wv * 32;                                 // the wave's first query
    const int64_t qi = qw + ql;                                      // this lane's query
    const int64_t qc = qi < a.Lq ? qi : a.Lq - 1;

    // Q^T operand: 8 head-dim values per 16-wide step, d = 16 st + 8 h + 0..7
    E8 qf[D / 16];
    {
        const char *qrow = a.q + (b * a.Lq + qc) * (int64_t)D * 2;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) qf[st] = ld8<E8>(qrow + (16 * st + 8 * h) * 2);
    }

    // keys any query of this workgroup can see
    int64_t kend = a.Lk;
    if (a.causal) {
        const int64_t lim = q0 + BM + a.offset;                      // last query's keys: < q0 + BM - 1 + offset + 1
        if (lim < kend) kend = lim;
    }
    const int64_t ntiles = (kend + BN - 1) / BN;

    // tile loads: K rows contiguous per thread (coalesced), V rows one key
    // per lane (so the transposed LDS writes of a wave fill one row)
    const char *kb0 = a.k + b * a.Lk * (int64_t)D * 2;
    const char *vb0 = a.v + b * a.Lk * (int64_t)D * 2;
    // (K chunks as vector-typed values: held in registers across the loop)
    u32x4 kr[KCH];
    uint4 vr[VCH];
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m_run = -__builtin_inff(), l_run = 0.f;           // running max (scaled, base 2) and this lane's sum
    const float s2 = a.s2;

    load_tile<D, KCH, VCH>(kr, vr, kb0, vb0, 0, a.Lk, tid);
    for (int64_t t = 0; t < ntiles; ++t) {
        const int64_t j0 = t * BN;
        __syncthreads();                                    // previous tile's LDS reads are done
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int idx = tid + NT * c, key = idx / (D / 8), dc = idx % (D / 8);
            *reinterpret_cast<u32x4 *>(ks + key * KSTR + dc * 16) = kr[c];
        }
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
            const int key = tid % BN, dc = tid / BN + (NT / BN) * c;
            const uint32_t w[4] = {vr[c].x, vr[c].y, vr[c].z, vr[c].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *reinterpret_cast<uint16_t *>(vs + (dc * 8 + e) * VSTR + key * 2) =
                    (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
        __syncthreads();
        // next tile's rows in flight during this one's math (after the last
        // tile: a clamped, unused reload)
        load_tile<D, KCH, VCH>(kr, vr, kb0, vb0, t + 1 < ntiles ? j0 + BN : j0, a.Lk, tid);

        // ---- S^T = K Q^T for both 32-key blocks of the tile first, so the
        // matrix cores work on the second block's scores while the vector
        // ALUs run the first block's softmax
        f32x16 sb[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sb[kb][r] = 0.f;
            const char *krow = ks + (kb * 32 + ql) * KSTR + 8 * h * 2;
#pragma unroll
            for (int st = 0; st < D / 16; ++st) sb[kb] = Mma<DT>::mma(ld8<E8>(krow + 32 * st), qf[st], sb[kb]);
        }

        // ---- per 32-key block: mask, online softmax update, P^T (two
        // 16-bit parts), O^T += V^T P^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 s = sb[kb];
            // this block's V^T operands, read from LDS ahead of the softmax so
            // their latency is hidden behind it: the keys lane l holds for
            // MFMA step ss are kk + 4h + 0..3 and kk + 8 + 4h + 0..3
            E8 va[2][D / 32];
#pragma unroll
            for (int ss = 0; ss < 2; ++ss) {
                const int kk = kb * 32 + 16 * ss;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const char *vrow = vs + (db * 32 + ql) * VSTR;
                    va[ss][db] = ld4x2<E8>(vrow + (kk + 4 * h) * 2, vrow + (kk + 8 + 4 * h) * 2);
                }
            }

            // mask: blocks past Lk, or reaching past the wave's first query's diagonal
            const int64_t jb = j0 + kb * 32;
            if (jb + 32 > a.Lk || (a.causal && jb + 31 > qw + a.offset)) {
                const int64_t lim = a.causal ? (qi + a.offset < a.Lk - 1 ? qi + a.offset : a.Lk - 1) : a.Lk - 1;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t key = jb + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (key > lim) s[r] = -__builtin_inff();
                }
            }

            // online softmax: the block's max of scale*s (base 2); the
            // reference max m_run moves (and the accumulator and the sum are
            // rescaled by alpha = 2^(m_old - m_new)) only when some query of
            // the wave needs it: on its first keys, or when a score exceeds
            // the reference by more than the slack
            float mloc = -__builtin_inff();
#pragma unroll
            for (int r = 0; r < 16; ++r) mloc = __builtin_fmaxf(mloc, s[r]);
            mloc = __builtin_fmaxf(mloc, __shfl_xor(mloc, 32)) * s2;
            const bool move = !(mloc <= m_run + RESCALE_SLACK);            // also when m_run is -inf
            if (__ballot(move)) {
                const float m_new = move ? __builtin_fmaxf(m_run, mloc) : m_run;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 the first time, 1 if unmoved
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            }

#pragma unroll
            for (int ss = 0; ss < 2; ++ss) {
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * ss + j], s2, -m_run));
                    l_run += p[j];
                }
                E8 phi, plo;
                split16<DT>(p, phi, plo);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    acc[db] = Mma<DT>::mma(va[ss][db], phi, acc[db]);
                    acc[db] = Mma<DT>::mma(va[ss][db], plo, acc[db]);
                }
            }
        }
    }

    // ---- o = acc / l; lane l writes head-dims db*32 + 8g + 4h + 0..3 of its query
    const float l = l_run + __shfl_xor(l_run, 32);
    const float inv = __builtin_amdgcn_rcpf(l);
    if (qi < a.Lq) {
        char *orow = a.o + (b * a.Lq + qi) * (int64_t)D * 2;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = acc[db][4 * g + r] * inv;
#pragma unroll
                for (int r = 4; r < 8; ++r) v[r] = 0.f;
                const uint4 w = pack<DT>(v);
                *reinterpret_cast<uint2 *>(orow + (db * 32 + 8 * g + 4 * h) * 2) = make_uint2(w.x, w.y);
            }
    }
}

template <int DT, int D>
hipError_t go(const AttnArgs &a, hipStream_t s) {
    void *args[] = {const_cast<AttnArgs *>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void *>(attention_fwd<DT, D>), dim3((uint32_t)(a.BH * a.nqb)),
                           dim3(NT), args, 0, s);
}

}  // namespace

hipError_t launch_attention(int dt, int D, const AttnArgs &a, hipStream_t s) {
    if (dt == DT_BF16 && D == 128) return go<DT_BF16, 128>(a, s);
    if (dt == DT_BF16 && D == 64) return go<DT_BF16, 64>(a, s);
    if (dt == DT_F16 && D == 128) return go<DT_F16, 128>(a, s);
    if (dt == DT_F16 && D == 64) return go<DT_F16, 64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace ntk
