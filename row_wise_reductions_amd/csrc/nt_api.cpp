// C ABI of the row-reduction library: argument validation, launch planning
// and dispatch to the gfx950 kernels.  Declared in include/nt.h.
//
// Planning rule (per element type and row width):
//   * the row is cut into 16-byte chunks; a group of W waves (64*W lanes)
//     holding K chunks per lane covers 64*W*K chunks;
//   * the first (smallest) shape of the type's menu that covers the row is
//     used for the single-pass kernel (one HBM read and one write per
//     element, as in the fused softmax of the stanleyjacob.dev Triton guide,
//     Part II "Worked example: fused softmax");
//   * softmax rows wider than the widest shape take the split online path
//     ("Triton: Block-Level GPU Programming Without CUDA", section "How Flash
//     Attention Uses Triton"): chunks of one workgroup each, partial
//     (max, denominator) pairs in the caller's workspace, then a merge -- in
//     one cooperative kernel up to 128 chunks per row, else in two kernels.
//     LayerNorm and RMSNorm rows wider than the widest shape take a looped
//     kernel: one workgroup per row reads the row twice in tiles (statistics,
//     then output), so no workspace is needed;
//   * norms on aligned rows with every parameter vector present run
//     persistent workgroups (parameters widened once, next row prefetched).
// The fused residual add + norm entry points and the causal softmax entry
// point plan as their norm / the softmax, with the limits noted where they
// differ (values per lane, the causal 16-bit menu exception).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>

#include "../../include/nt.h"
#include "attention.hpp"
#include "launch.hpp"

namespace {

struct Shape {
    int W, K;
    int cap = 0;     // menu entries: most chunks per row it is chosen for (0: its capacity, 64*W*K)
};

// Single-pass shapes in order of capacity (64*W*K chunks of 16 bytes).  None
// of them spills registers.  A lane holds at most 64 values of a row, and
// LayerNorm at most 16 (its fp64 arithmetic needs more registers) except 32
// at 8 waves (rows of up to 16384 elements, where the looped kernel ran at
// 0.6-0.9x torch's layer_norm; fp32 at 32 values is never persistent, which
// would spill); wider LayerNorm and RMSNorm rows take the looped kernel, wider
// softmax rows the split path.
struct Menu {
    const Shape *s;
    int n;
};
// Chosen from launch-shape sweeps on MI355X (every shape that covers the row,
// timed interleaved at M = 4096 and at 2^27 elements per matrix, and on the
// workloads): about one or two 16-byte chunks per lane with up to 8 waves per
// row stream best.  For softmax rows of 257..512 chunks 4 waves with 2 chunks
// each beat 8 waves with 1 by 3-15% (no idle lanes on part-filled rows, twice
// the rows in flight; on causal rows, whose loads stop at the diagonal, by
// 27%).  Exception: 16-bit softmax rows that fill all 512 chunks (4096
// elements) keep 8 waves with 1 chunk, which streams the 131072-row
// causal-score workload about 1-2% faster (full_row_shape).  RMSNorm: 4 waves
// x 1 chunk for rows of 129..256 chunks (3% over one wave x 4 at large M),
// 8 x 1 for 257..512 (6% over 1 x 8), fp32 16 x 2 for 1025..2048.  LayerNorm,
// whose fp64 statistics lengthen each row's compute, prefers fewer waves:
// f16 2 x 2 for 129..256 chunks, fp32 2 x 4 for 257..512 (2-5%); and it
// takes 5-7 waves (12 for fp32 with 4 chunks) where a power of two would
// leave lanes idle: 16-bit 7 x 2 for 513..896 chunks (1-3% over 8 x 2),
// 5 x 4 to 1216 chunks, 6 x 4 to 1408, 7 x 4 from 1473 to 1792 (2-5% over
// 8 x 4; near the top of its capacity 5 x 4 and 6 x 4 fell 2-7% behind
// 8 x 4, hence the caps), fp32 4 x 4 for 513..640 chunks (1-8% over 8 x 2),
// 12 x 4 for 2049..3072 (2-8% over 8 x 8; two M = 4096 sweeps of the
// pages' widths).  The fused residual add + norm
// entries have menus of their own (below).
const Shape kSoftmax32[] = {{1, 1}, {1, 2}, {1, 4}, {4, 2}, {8, 2}, {8, 4}, {8, 8}, {8, 16}};
const Shape kSoftmax16[] = {{1, 1}, {1, 2}, {1, 4}, {4, 2}, {8, 2}, {8, 4}, {8, 8}};
const Shape kRms32[] = {{1, 1}, {1, 2}, {1, 4}, {8, 1}, {8, 2}, {16, 2}, {8, 8}, {8, 16}};
const Shape kRms16[] = {{1, 1}, {1, 2}, {4, 1}, {8, 1}, {8, 2}, {8, 4}, {8, 8}};
const Shape kLn32[] = {{1, 1}, {1, 2}, {1, 4}, {2, 4}, {4, 4, 640}, {8, 2}, {8, 4}, {12, 4}, {8, 8}};
const Shape kLn16[] = {{1, 1},       {1, 2},       {2, 2},       {4, 2}, {7, 2}, {8, 2},
                       {5, 4, 1216}, {6, 4, 1408}, {8, 4, 1472}, {7, 4}, {8, 4}};
// Fused residual add + norm (two input and two output streams per row): more
// waves per row than the plain norms at the same width.  16-bit RMSNorm rows
// of 1025..2048 chunks take 16 waves x 2 (7% over 8 x 4); f16 LayerNorm rows
// of up to 512 chunks 4 x 1 and 8 x 1 (3-4% over 4 x 2); fp32 RMSNorm uses
// the plain menu (wider shapes are cut at 32 values per lane by shape_fits).
const Shape kAddRms16[] = {{1, 1}, {1, 2}, {4, 1}, {8, 1}, {8, 2}, {16, 2}};
const Shape kAddLn32[] = {{1, 1}, {1, 2}, {1, 4}, {4, 2}, {8, 2}, {8, 4}, {8, 8}};
const Shape kAddLn16[] = {{1, 1}, {1, 2}, {4, 1}, {8, 1}, {8, 2}, {8, 4}};
#define NT_MENU(a) Menu{a, (int)(sizeof(a) / sizeof(*(a)))}
Menu menu_for(nt_op op, nt_dtype dt, bool res) {
    const bool wide = dt == NT_F32;
    switch (op) {
    case NT_OP_SOFTMAX: return wide ? NT_MENU(kSoftmax32) : NT_MENU(kSoftmax16);
    case NT_OP_RMSNORM:
        if (res && !wide) return NT_MENU(kAddRms16);
        return wide ? NT_MENU(kRms32) : NT_MENU(kRms16);
    default:
        if (res) return wide ? NT_MENU(kAddLn32) : NT_MENU(kAddLn16);
        return wide ? NT_MENU(kLn32) : NT_MENU(kLn16);
    }
}
#undef NT_MENU
// Split-path chunk shapes.  Up to COOP_PMAX chunks per row, large chunks for
// the cooperative kernel, so few workgroups per row wait on each other: fp32
// 8 waves x 8 chunks (32 values per lane), 16-bit 4 waves x 8 chunks (64
// values per lane; 3% ahead of 8 x 4 on 64 x 262144 bf16 rows); wider rows:
// 4 waves, 4 chunks per lane, two kernels.  The shape does not depend on
// whether the cooperative kernel is enabled, so neither does the workspace.
const Shape kSplitCoop32 = {8, 8};
const Shape kSplitCoop16 = {4, 8};
const Shape kSplitWide = {4, 4};
// Looped norm kernel: 512 threads, tiles of 4 chunks per lane.
const Shape kLooped = {8, 4};
// Split norm chunk shapes, largest first: the first that gives the call at
// least kNormSplitGrid workgroups is used (8 per CU on 256 CUs).
const Shape kNormSplit[] = {{8, 4}, {8, 1}, {4, 1}};
constexpr int64_t kNormSplitGrid = 2048;
constexpr int64_t kNormCoopPMax = 16;
// Rows below which the split is used.  The looped kernel gives each row one
// workgroup, so it fills the 256 CUs from 256 rows on; measured on MI355X
// (rows of 64 KiB to 2 MiB), the split is 2-7x faster below 64 rows, even at
// 256, and from there on 0-8% faster for RMSNorm but up to 8% slower for
// LayerNorm, whose finalize kernel holds the parameters as well.
constexpr int64_t kNormSplitRowsLN = 256;
constexpr int64_t kNormSplitRowsRMS = 2048;

int elem_bytes(nt_dtype dt) { return dt == NT_F32 ? 4 : 2; }
int elems_per_chunk(nt_dtype dt) { return 16 / elem_bytes(dt); }

bool valid_dtype(int dt) { return dt == NT_F32 || dt == NT_F16 || dt == NT_BF16; }

bool valid_shape(int64_t M, int64_t N) {
    if (M < 0 || N <= 0 || N > INT32_MAX) return false;
    if (M > 0 && N > INT64_MAX / 4 / M) return false;   // M*N*4 bytes must fit int64
    return true;
}

bool aligned_to(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// ---------------------------------------------------------------------------
// Tuning overrides (tests and launch-shape sweeps).  Each is read once from
// the NT_* environment variable of the same name when the library is loaded;
// nt_set_override() changes it afterwards.  The per-call path only reads
// these atomics.  Shapes are packed as (W << 32) | K, 0 = none.
// ---------------------------------------------------------------------------
enum TuneKey {
    T_FORCE_PATH,       // NT_FORCE_PATH: 0 none, 1 "split" (softmax), 2 "looped" (norms)
    T_FORCE_SHAPE,      // NT_FORCE_SHAPE "W,K": single-pass shape (ignored if it does not fit the row)
    T_SPLIT_SHAPE,      // NT_SPLIT_SHAPE "W,K": split softmax chunk shape
    T_COOP,             // NT_COOP: "0" two-kernel split forms; "rows1" / "rows2": the cooperative
                        // softmax with one / two rows per workgroup; else the planner's choice
    T_COOP_SPIN,        // NT_COOP_SPIN: polls before a missing record is recomputed (0..65536)
    T_PERSISTENT,       // NT_PERSISTENT: "0" never, "always" wherever built, "1" where it pays
    T_PERSIST_GRID,     // NT_PERSIST_GRID: workgroups of the persistent norm kernel (> 0)
    T_NORM_SPLIT_ROWS,  // NT_NORM_SPLIT_ROWS: rows below which a wide norm is split (>= 0)
    T_DEBUG,            // NT_DEBUG: print each plan to stderr
    T_COUNT
};
const char *const kTuneNames[T_COUNT] = {"NT_FORCE_PATH",   "NT_FORCE_SHAPE",     "NT_SPLIT_SHAPE",
                                         "NT_COOP",         "NT_COOP_SPIN",       "NT_PERSISTENT",
                                         "NT_PERSIST_GRID", "NT_NORM_SPLIT_ROWS", "NT_DEBUG"};
constexpr int64_t kTuneDefault[T_COUNT] = {0, 0, 0, 1, 1024, 1, 0, -1, 0};
std::atomic<int64_t> g_tune[T_COUNT];
int64_t g_tune_loaded[T_COUNT];      // the values read at load (what a reset restores)

// Parse a setting (NULL or "" gives the default); false for a malformed
// value, which the environment reader replaces by the default and the
// setter refuses.
bool parse_tune(int key, const char *s, int64_t *out) {
    if (!s || !*s) {
        *out = kTuneDefault[key];
        return true;
    }
    switch (key) {
    case T_FORCE_PATH:
        if (std::strcmp(s, "split") == 0) *out = 1;
        else if (std::strcmp(s, "looped") == 0) *out = 2;
        else return false;
        return true;
    case T_FORCE_SHAPE:
    case T_SPLIT_SHAPE: {
        int w = 0, k = 0;
        char tail = 0;
        if (std::sscanf(s, "%d,%d%c", &w, &k, &tail) != 2 || w <= 0 || k <= 0) return false;
        *out = ((int64_t)w << 32) | (int64_t)k;
        return true;
    }
    case T_COOP:
        if (std::strcmp(s, "0") == 0) *out = 0;
        else if (std::strcmp(s, "rows1") == 0) *out = 2;
        else if (std::strcmp(s, "rows2") == 0) *out = 3;
        else *out = 1;
        return true;
    case T_DEBUG:
        *out = std::strcmp(s, "0") == 0 ? 0 : 1;
        return true;
    case T_PERSISTENT:
        if (std::strcmp(s, "0") == 0) *out = 0;
        else if (std::strcmp(s, "1") == 0) *out = 1;
        else if (std::strcmp(s, "always") == 0) *out = 2;
        else return false;
        return true;
    default: {
        char *end = nullptr;
        const long long v = std::strtoll(s, &end, 10);
        if (end == s || *end) return false;
        if (key == T_COOP_SPIN && (v < 0 || v > 65536)) return false;
        if (key == T_PERSIST_GRID && v <= 0) return false;
        if (key == T_NORM_SPLIT_ROWS && v < 0) return false;
        *out = (int64_t)v;
        return true;
    }
    }
}

// Runs once, when the library is loaded.
struct TuneInit {
    TuneInit() {
        for (int k = 0; k < T_COUNT; ++k) {
            int64_t v = kTuneDefault[k];
            if (!parse_tune(k, std::getenv(kTuneNames[k]), &v)) v = kTuneDefault[k];
            g_tune_loaded[k] = v;
            g_tune[k].store(v, std::memory_order_relaxed);
        }
    }
} g_tune_init;

int64_t tune(TuneKey k) { return g_tune[k].load(std::memory_order_relaxed); }

bool tune_shape(TuneKey k, Shape *out) {
    const int64_t v = tune(k);
    if (v == 0) return false;
    *out = {(int)(v >> 32), (int)(v & 0xffffffff)};
    return true;
}

bool debug_on() { return tune(T_DEBUG) != 0; }

// Cooperative split forms (one pass over x) unless NT_COOP=0.
bool coop_enabled() { return tune(T_COOP) != 0; }

// Rows per workgroup of the cooperative softmax for M rows of P chunks
// (NT_COOP=rows1 / rows2 force one or the other).  Two rows (softmax_coop2:
// one row's writes overlap the next row's reads) for fp32 rows from 1024
// (row, chunk) pairs on: 1.10x on 64 x 262144, 1.08x on 256 x 65536,
// 1.01-1.04x at 2048-4096 pairs; below 1024 pairs half the workgroups leave
// CUs idle (0.78-0.88x at 256-512 pairs), and the 16-bit form, at 142
// instead of 108 VGPRs, was slower at every size tried (0.83-0.94x).
int coop_rows(int64_t M, int64_t P, nt_dtype dt) {
    const int64_t v = tune(T_COOP);
    if (M < 2 || v == 2) return 1;
    if (v == 3) return 2;
    return dt == NT_F32 && M * P >= 1024 ? 2 : 1;
}

// Polls of the cooperative kernels before they recompute a missing chunk's
// record themselves (0 recomputes every record not there at the first look,
// which tests use).
int32_t coop_spin() { return (int32_t)tune(T_COOP_SPIN); }

// Bytes after a split plan's records that hold the tag word of a cooperative
// call captured into a graph (the workspace sizes include them).
constexpr int64_t kTagBytes = 16;

// One thread advances the tag word of a captured cooperative call; in the
// graph it runs right before the cooperative launch, so every replay tags
// its records with a value no earlier replay used (vector load and store).
__global__ void __launch_bounds__(64) nt_tag_bump(uint32_t *p) {
    if (threadIdx.x == 0) {
        const uint32_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p, v + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

hipError_t bump_tag(const uint32_t *p, hipStream_t s) {
    uint32_t *q = const_cast<uint32_t *>(p);
    void *args[] = {&q};
    return hipLaunchKernel(reinterpret_cast<const void *>(nt_tag_bump), dim3(1), dim3(64), args, 0, s);
}


// Compute units of each device, queried on the first call made on it.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        g_cus[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

// Tag of the cooperative kernel's workspace records: unique per call within
// a process (a counter), and with a random start so that records left in a
// reused buffer by another process are not taken for this call's.
uint32_t next_tag() {
    static std::atomic<uint32_t> counter{[] {
        std::random_device rd;
        return (uint32_t)rd();
    }()};
    return counter.fetch_add(1, std::memory_order_relaxed);
}

// Is `stream` capturing a graph?  A replay would reuse the call's record
// tag, and could take the previous replay's records for its own.
nt_status stream_capturing(void *stream, bool *capturing) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(reinterpret_cast<hipStream_t>(stream), &cs) != hipSuccess) return NT_ERR_HIP;
    *capturing = cs != hipStreamCaptureStatusNone;
    return NT_OK;
}

// The record tag of a cooperative call: from the host, unique per call; or,
// while the stream is being captured into a graph (whose replays repeat the
// call's arguments), the device word after the records, which run() has a
// one-thread kernel advance right before the cooperative launch.
nt_status set_coop_tag(void *stream, char *ws, int64_t records_bytes, ntk::RowArgs &a) {
    bool cap = false;
    const nt_status st = stream_capturing(stream, &cap);
    if (st != NT_OK) return st;
    if (cap)
        a.tagp = reinterpret_cast<const uint32_t *>(ws + records_bytes);
    else
        a.tag = next_tag();
    a.spin = coop_spin();
    return NT_OK;
}

// Chunks a row can touch: N*e/16 when aligned, else up to one more for the
// partial chunk in front of a misaligned row start.
int64_t row_chunks(int64_t N, nt_dtype dt, bool aligned) {
    const int64_t vec = elems_per_chunk(dt);
    if (aligned) return N / vec;
    return (N + vec - 1 + vec - 1) / vec;
}

// Rows below which a norm too wide for one pass is split over workgroups
// (given a workspace); NT_NORM_SPLIT_ROWS overrides (tuning).
int64_t norm_split_rows(nt_op op) {
    const int64_t v = tune(T_NORM_SPLIT_ROWS);
    if (v >= 0) return v;
    return op == NT_OP_LAYERNORM ? kNormSplitRowsLN : kNormSplitRowsRMS;
}

// Persistent norm kernels: NT_PERSISTENT=0 never, "always" wherever the
// kernel is built (tuning), else where it pays (persistent_pays).
int persistent_mode() { return (int)tune(T_PERSISTENT); }

// Whether persistent workgroups beat one workgroup per row, from sweeps with
// both forced on every planned shape and row fill (M = 4096 and 256 MiB
// matrices).  The persistent kernel overlaps the next row's loads with this
// row's arithmetic but holds two rows in registers, so fewer waves fit.
//  - LayerNorm (fp64 statistics, long per-row arithmetic): always, by 4-54%.
//  - Fused add + LayerNorm: when a lane holds 16 values or more (9-29%);
//    with fewer, one row per workgroup is 1-14% faster.
//  - 16-bit RMSNorm: rows of 1024 chunks or more (a tie at 1024, 5-13% from
//    1280); narrower rows stream 2-12% faster one row per workgroup.
//  - fp32 RMSNorm: only the part-filled 8 x 8 shape (2049..3072 chunks,
//    2-8%); the fused add + RMSNorm never (its two input streams keep enough
//    bytes in flight without it).
bool persistent_built(nt_op op, nt_dtype dt, bool res, Shape sh) {
    if (op == NT_OP_LAYERNORM) return !(dt == NT_F32 && sh.K * elems_per_chunk(dt) > 16);
    return !res && (dt != NT_F32 || (sh.W == 8 && sh.K == 8));
}

bool persistent_pays(nt_op op, nt_dtype dt, bool res, Shape sh, int64_t nch) {
    if (op == NT_OP_LAYERNORM) return !res || sh.K * elems_per_chunk(dt) >= 16;
    if (res) return false;
    return dt != NT_F32 ? nch >= 1024 : (sh.W == 8 && sh.K == 8 && nch <= 3072);
}

// Grid of the persistent norm kernel: k workgroups per compute unit, k from
// the bytes of one row (interleaved kernel-trace sweeps of k = 1..8 with an
// A/A control).  LayerNorm streams fastest with about 16 KiB of rows per CU
// and at least two workgroups: k = max(2, ceil(16 KiB / row)), so 2 on
// 4096-element 16-bit rows (3.7% over the 3 that fit), 3 on 3584-element
// ones, 4 on 2048-element ones (6% over the 8 that fit), 2 on 2048-element
// fp32 rows (10% over 6).  RMSNorm (16 to 48 KiB rows) is fastest with
// floor(32 KiB / row), at least 1: half the workgroups that fit.  The
// launcher caps k at the kernel's occupancy; NT_PERSIST_GRID sets the grid
// itself, uncapped (tuning).
int64_t persistent_grid(nt_op op, nt_dtype dt, int64_t M, int64_t N, int cus) {
    const int64_t forced = tune(T_PERSIST_GRID);
    if (forced > 0) return std::min(M, forced);
    const int64_t row = N * elem_bytes(dt);
    const int64_t k = op == NT_OP_RMSNORM ? std::max<int64_t>(1, 32768 / row)
                                           : std::max<int64_t>(2, (16384 + row - 1) / row);
    return std::min(M, k * cus);
}

// `res`: the fused residual add + norm, whose lanes also hold the residual's
// words (at most 32 values per lane for RMSNorm; LayerNorm is capped at 16).
// LayerNorm is built with at most 12 waves per row.
// Only shapes with a kernel fit: the single-pass kernels are instantiated for
// W x K in {1 x 1..16, 2 x 2..8, 4 x 1..8, 8 x 1..16, 16 x 1..2} (K a power of
// two), plus LayerNorm's 7 x 2 and 5..7 x 4 (16-bit) and 12 x 4 (fp32);
// LayerNorm has at most 12 waves per row and keeps at most 16 values per
// lane, or 32 at 5 to 8 waves.
bool shape_fits(nt_op op, nt_dtype dt, bool res, Shape sh) {
    const int W = sh.W, K = sh.K, V = K * (int)elems_per_chunk(dt);
    const bool pow2k = K >= 1 && K <= 16 && (K & (K - 1)) == 0;
    bool built = (W == 1 && pow2k) || (W == 2 && pow2k && K >= 2 && K <= 8) || (W == 4 && pow2k && K <= 8) ||
                 (W == 8 && pow2k) || (W == 16 && K <= 2 && pow2k);
    if (op == NT_OP_LAYERNORM) {
        if (dt != NT_F32) built = built || (W == 7 && K == 2) || (W >= 5 && W <= 7 && K == 4);
        else built = built || (W == 12 && K == 4);
        built = built && W <= 12 && (V <= 16 || (W >= 5 && W <= 8 && V == 32));
    } else {
        built = built && V <= (res ? 32 : 64);
    }
    return built;
}

// 16-bit softmax rows of exactly 512 chunks (not causal): 8 waves, 1 chunk.
bool full_row_shape(nt_op op, nt_dtype dt, int64_t nch, bool causal, Shape *s) {
    if (op != NT_OP_SOFTMAX || dt == NT_F32 || causal || nch != 512) return false;
    *s = {8, 1};
    return true;
}

// Narrow rows (at most 256 chunks), where the menus give one wave per row
// with 1 to 4 chunks per lane, take more waves per row in two cases
// (softmax, RMSNorm, LayerNorm; the causal entry plans as the softmax; not
// the fused add + norm entries, whose menus were swept separately):
//  - few rows (M <= 1024: one wave per row would leave most of the 1024
//    SIMDs with at most one wave): 4 waves x 1 chunk, 2-32% faster on rows
//    of 40-256 chunks at 512 and 1024 rows, every op and type;
//  - rows that are not 16-byte aligned, 65-256 chunks: 2 waves x 2 chunks up
//    to 128 chunks, and for 16-bit softmax up to 256; 4 x 1 for fp32 rows
//    and 16-bit norm rows of 129-256 chunks (16-bit LayerNorm keeps 1 x 2 up
//    to 128, 1-16% ahead there).  1.04-1.53x over the one-wave shapes at
//    2048-16384 rows (softmax fp32 781 wide: 1.30x at 16384 rows; bf16 1030
//    wide: 1.53x).  On aligned rows of many rows the one-wave shapes stay
//    ahead (0-5%).
// Kernel-trace sweeps of every covering shape over 512-16384 rows of 40-256
// chunks (softmax fp32/bf16, RMSNorm and LayerNorm fp32/16-bit) on MI355X.
bool narrow_row_shape(nt_op op, nt_dtype dt, bool res, bool aligned, int64_t M, int64_t nch, Shape *s) {
    if (res || nch > 256) return false;
    if (M <= 1024) {
        *s = {4, 1};
        return true;
    }
    if (aligned || nch <= 64) return false;
    const bool wide = dt == NT_F32;
    if (nch <= 128) {
        if (op == NT_OP_LAYERNORM && !wide) return false;
        *s = {2, 2};
        return true;
    }
    *s = (op == NT_OP_SOFTMAX && !wide) ? Shape{2, 2} : Shape{4, 1};
    return true;
}

// The split norm's plan for M rows of nch chunks (norms with a workspace, rows
// too wide for one pass): false for the plain (looped) plan.
//   One pass (cooperative), at any row count, where the row has at most
//   kNormCoopPMax chunks of 8 waves x 4 (32 KiB; fp32 also 8 x 8, 64 KiB:
//   RMSNorm first, LayerNorm second), those give at least kNormSplitGrid
//   workgroups, and the
//   kernel keeps 4 waves per SIMD (not 16-bit LayerNorm, whose 8 x 4 form
//   holds about 200 registers).
//   Else, below norm_split_rows(op) rows, two kernels, with the largest chunk
//   that gives kNormSplitGrid workgroups.
// Measured on MI355X (rows of 64 KiB to 2 MiB, 4 to 2048 rows): the one pass
// reads x once and beats the looped kernel by 8-35% there, but its
// workgroups wait for the slowest of the row's chunks, which costs more than
// the second read saves once a row has 32 chunks or more, or when few rows
// leave the re-read in cache; the two kernels are 2-7x faster than the
// looped kernel below 64 rows.
bool split_norm_plan(nt_op op, nt_dtype dt, int64_t M, int64_t nch, bool coop, Shape *out, int64_t *P,
                     bool *cooperative) {
    if (M <= 0) return false;                            // nothing to split (callers divide by M)
    auto chunks = [nch](const Shape &c) { return (nch + 64 * c.W * c.K - 1) / (64 * c.W * c.K); };
    const Shape big = kNormSplit[0];
    if (coop && !(op == NT_OP_LAYERNORM && dt != NT_F32)) {
        // fp32 RMSNorm first tries 64 KiB chunks (8 x 8, 110 VGPRs, still two
        // workgroups per CU): half the chunks per row wait on each other, and
        // rows up to 262144 elements qualify (11% faster at 2048 x 65536,
        // 27-41% on 262144-wide rows, which the 8 x 4 form left to the looped
        // kernel); 16-bit 8 x 8 holds 174 VGPRs and was not faster.  fp32
        // LayerNorm's 8 x 8 (206 VGPRs, one workgroup per CU) was 5% slower
        // than its 8 x 4 but 3-9% faster than the looped kernel: it comes
        // second, for rows of 17 to 16 x 2 chunks of 32 KiB.
        const Shape big8 = {8, 8};
        const Shape rms32[2] = {big8, big}, ln32[2] = {big, big8}, one[1] = {big};
        const Shape *cands = dt != NT_F32 ? one : op == NT_OP_RMSNORM ? rms32 : ln32;
        const int nc = dt != NT_F32 ? 1 : 2;
        for (int i = 0; i < nc; ++i) {
            const Shape &c = cands[i];
            if (chunks(c) <= kNormCoopPMax && M * chunks(c) >= kNormSplitGrid) {
                *out = c;
                *P = chunks(c);
                *cooperative = true;
                return true;
            }
        }
    }
    if (M >= norm_split_rows(op)) return false;
    Shape s = big;
    for (const Shape &c : kNormSplit) {
        s = c;
        if (M * chunks(c) >= kNormSplitGrid) break;
    }
    *out = s;
    *P = chunks(s);
    *cooperative = false;
    return true;
}

nt_status make_plan(nt_op op, int64_t M, int64_t N, nt_dtype dt, bool aligned, nt_plan *p, bool params = true,
                    bool res = false, bool causal = false, bool norm_split = false) {
    std::memset(p, 0, sizeof *p);
    p->aligned = aligned ? 1 : 0;
    const int64_t nch = row_chunks(N, dt, aligned);
    const Menu menu = menu_for(op, dt, res);
    const int64_t force = tune(T_FORCE_PATH);
    const bool force_split = op == NT_OP_SOFTMAX && force == 1;
    const bool force_loop = op != NT_OP_SOFTMAX && force == 2;

    Shape pick = {0, 0};
    if (!force_split && !force_loop) {
        Shape o;
        if (tune_shape(T_FORCE_SHAPE, &o) && (int64_t)64 * o.W * o.K >= nch && shape_fits(op, dt, res, o)) {
            pick = o;
        } else if (full_row_shape(op, dt, nch, causal, &o)) {
            pick = o;
        } else if (narrow_row_shape(op, dt, res, aligned, M, nch, &o) && shape_fits(op, dt, res, o)) {
            pick = o;
        } else {
            for (int i = 0; i < menu.n; ++i) {
                const Shape &c = menu.s[i];
                if ((c.cap ? c.cap : (int64_t)64 * c.W * c.K) >= nch && shape_fits(op, dt, res, c)) {
                    pick = {c.W, c.K};
                    break;
                }
            }
        }
    }
    if (pick.W) {
        const int G = pick.W == 1 ? 4 : 1;
        p->split = 0;
        p->waves_per_row = pick.W;
        p->chunks_per_lane = pick.K;
        p->rows_per_block = G;
        p->threads_per_block = 64 * pick.W * G;
        // The dispatch packet counts work-items in 32 bits: keep grid*threads
        // below 2^31; the kernel strides over any remaining rows.
        const int64_t max_grid = ((int64_t)1 << 31) / p->threads_per_block;
        int64_t grid = (M + G - 1) / G;
        if (grid > max_grid) grid = max_grid;
        p->grid = grid;
        // Norms on aligned rows with every parameter vector present can keep
        // the parameters widened in registers across rows: persistent
        // workgroups (k per compute unit, persistent_grid; capped at launch
        // by how many fit at once), where that pays (persistent_pays).  At most 32
        // values per lane: the row, its prefetched successor and the cached
        // parameters must fit without spilling; built for 2 to 8 waves.
        if (op != NT_OP_SOFTMAX && aligned && params && pick.W >= 2 && pick.W <= 8 &&
            pick.K * elems_per_chunk(dt) <= 32 && persistent_built(op, dt, res, pick) &&
            (persistent_mode() == 2 || (persistent_mode() == 1 && persistent_pays(op, dt, res, pick, nch)))) {
            p->persistent = 1;
            p->grid = persistent_grid(op, dt, M, N, device_cus());
        }
        return NT_OK;
    }
    Shape ns;
    int64_t nP;
    bool ncoop;
    // (one workgroup per (row, chunk), no striding: else the looped plan)
    if (op != NT_OP_SOFTMAX && norm_split && !res && split_norm_plan(op, dt, M, nch, coop_enabled(), &ns, &nP, &ncoop) &&
        nP <= (((int64_t)1 << 31) / (64 * ns.W)) / M) {
        // few wide rows, or wide rows of few chunks: each row cut into
        // chunks, one workgroup each
        p->split = 3;
        p->waves_per_row = ns.W;
        p->chunks_per_lane = ns.K;
        p->rows_per_block = 1;
        p->threads_per_block = 64 * ns.W;
        p->row_chunks = nP;
        p->grid = M * nP;
        p->cooperative = ncoop ? 1 : 0;
        // four tagged 64-bit words per chunk (the cooperative records; the
        // two kernels use half of that for their (s1, s2) pairs), then a
        // pivot per row
        p->workspace_bytes = M * nP * 32 + M * 8 + kTagBytes;
        return NT_OK;
    }
    if (op != NT_OP_SOFTMAX) {
        // one workgroup per row, the row streamed twice in tiles
        p->split = 2;
        p->waves_per_row = kLooped.W;
        p->chunks_per_lane = kLooped.K;
        p->rows_per_block = 1;
        p->threads_per_block = 64 * kLooped.W;
        const int64_t max_grid = ((int64_t)1 << 31) / p->threads_per_block;
        p->grid = M < max_grid ? M : max_grid;
        return NT_OK;
    }
    Shape s = dt == NT_F32 ? kSplitCoop32 : kSplitCoop16;
    if ((nch + 64 * s.W * s.K - 1) / (64 * s.W * s.K) > ntk::COOP_PMAX) s = kSplitWide;
    Shape o;
    if (tune_shape(T_SPLIT_SHAPE, &o)) s = o;
    const int64_t per = (int64_t)64 * s.W * s.K;
    const int64_t P = (nch + per - 1) / per;
    // one workgroup per (row, chunk), no striding: the grid must fit the packet
    if (P > INT32_MAX || (M > 0 && P > (((int64_t)1 << 31) / (64 * s.W)) / M)) return NT_ERR_SHAPE;
    p->split = 1;
    p->waves_per_row = s.W;
    p->chunks_per_lane = s.K;
    p->rows_per_block = 1;
    p->threads_per_block = 64 * s.W;
    p->row_chunks = P;
    p->grid = M * P;
    // two 64-bit words per (row, chunk): the cooperative kernel's tagged
    // record; the two-kernel form uses the first 8 bytes as its (m_j, l_j);
    // then the tag word of a captured cooperative call
    p->workspace_bytes = M * P * 16 + kTagBytes;
    p->cooperative = (P <= ntk::COOP_PMAX && coop_enabled()) ? 1 : 0;
    if (p->cooperative && coop_rows(M, P, dt) == 2) {
        p->cooperative = 2;
        p->rows_per_block = 2;
        p->grid = (M + 1) / 2 * P;
    }
    return NT_OK;
}

bool all_aligned16(int64_t N, nt_dtype dt, const void *x, const void *y, const void *p0, const void *p1) {
    if ((N * elem_bytes(dt)) % 16 != 0) return false;
    for (const void *q : {x, y, p0, p1})
        if (q && !aligned_to(q, 16)) return false;
    return true;
}

hipError_t launch_resident(nt_dtype dt, int op, const nt_plan &p, const ntk::RowArgs &a, hipStream_t s) {
    const bool al = p.aligned != 0;
    if (p.persistent) {
        // capped at the kernel's occupancy, unless the grid is forced
        const int cap = tune(T_PERSIST_GRID) > 0 ? 0 : device_cus();
        switch (dt) {
        case NT_F32: return ntk::launch_persistent_f32(op, p.waves_per_row, p.chunks_per_lane, a, s, p.grid, cap);
        case NT_F16: return ntk::launch_persistent_f16(op, p.waves_per_row, p.chunks_per_lane, a, s, p.grid, cap);
        case NT_BF16: return ntk::launch_persistent_bf16(op, p.waves_per_row, p.chunks_per_lane, a, s, p.grid, cap);
        }
    }
    switch (dt) {
    case NT_F32: return ntk::launch_resident_f32(op, p.waves_per_row, p.chunks_per_lane, al, a, p.grid, s);
    case NT_F16: return ntk::launch_resident_f16(op, p.waves_per_row, p.chunks_per_lane, al, a, p.grid, s);
    case NT_BF16: return ntk::launch_resident_bf16(op, p.waves_per_row, p.chunks_per_lane, al, a, p.grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_looped(nt_dtype dt, int op, const nt_plan &p, const ntk::RowArgs &a, hipStream_t s) {
    const bool al = p.aligned != 0;
    switch (dt) {
    case NT_F32: return ntk::launch_looped_f32(op, p.waves_per_row, p.chunks_per_lane, al, a, p.grid, s);
    case NT_F16: return ntk::launch_looped_f16(op, p.waves_per_row, p.chunks_per_lane, al, a, p.grid, s);
    case NT_BF16: return ntk::launch_looped_bf16(op, p.waves_per_row, p.chunks_per_lane, al, a, p.grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_split(nt_dtype dt, const nt_plan &p, const ntk::RowArgs &a, hipStream_t s) {
    const bool al = p.aligned != 0;
    const int coop = p.cooperative;
    switch (dt) {
    case NT_F32: return ntk::launch_split_f32(p.waves_per_row, p.chunks_per_lane, al, coop, a, s);
    case NT_F16: return ntk::launch_split_f16(p.waves_per_row, p.chunks_per_lane, al, coop, a, s);
    case NT_BF16: return ntk::launch_split_bf16(p.waves_per_row, p.chunks_per_lane, al, coop, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_norm_split(nt_dtype dt, int op, const nt_plan &p, const ntk::RowArgs &a, hipStream_t s) {
    const bool al = p.aligned != 0, coop = p.cooperative != 0;
    switch (dt) {
    case NT_F32: return ntk::launch_norm_split_f32(op, p.waves_per_row, p.chunks_per_lane, al, coop, a, s);
    case NT_F16: return ntk::launch_norm_split_f16(op, p.waves_per_row, p.chunks_per_lane, al, coop, a, s);
    case NT_BF16: return ntk::launch_norm_split_bf16(op, p.waves_per_row, p.chunks_per_lane, al, coop, a, s);
    }
    return hipErrorInvalidValue;
}

void debug_print(const char *what, int64_t M, int64_t N, nt_dtype dt, const nt_plan &p) {
    std::fprintf(stderr,
                 "[nt] %s M=%lld N=%lld dt=%d: path %s W=%d K=%d rows/block=%d threads=%d aligned=%d"
                 " persistent=%d cooperative=%d grid=%lld chunks/row=%lld ws=%lld\n",
                 what, (long long)M, (long long)N, (int)dt,
                 p.split == 1 ? "split" : p.split == 2 ? "looped" : p.split == 3 ? "split norm" : "single-pass", p.waves_per_row,
                 p.chunks_per_lane, p.rows_per_block, p.threads_per_block, p.aligned, p.persistent, p.cooperative, (long long)p.grid,
                 (long long)p.row_chunks, (long long)p.workspace_bytes);
}

nt_status run(nt_op op, int64_t M, int64_t N, nt_dtype dt, const nt_plan &p, const ntk::RowArgs &a,
              void *stream) {
    if (debug_on())
        debug_print(op == NT_OP_SOFTMAX     ? (a.queries ? "causal softmax" : "softmax")
                    : op == NT_OP_LAYERNORM ? (a.r ? "add+layernorm" : "layernorm")
                                            : (a.r ? "add+rmsnorm" : "rmsnorm"),
                    M, N, dt, p);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // kernel op codes: the causal softmax is a kernel op of its own
    const int kop = (op == NT_OP_SOFTMAX && a.queries > 0) ? (int)ntk::OP_SOFTMAX_CAUSAL : (int)op;
    // a captured cooperative call: advance its tag word on the device first
    if (a.tagp && (p.split == 1 || p.split == 3) && p.cooperative) {
        const hipError_t eb = bump_tag(a.tagp, s);
        if (eb != hipSuccess) {
            if (debug_on()) std::fprintf(stderr, "[nt] launch failed: %s\n", hipGetErrorString(eb));
            return NT_ERR_HIP;
        }
    }
    hipError_t e = p.split == 1   ? launch_split(dt, p, a, s)
                   : p.split == 2 ? launch_looped(dt, kop, p, a, s)
                   : p.split == 3 ? launch_norm_split(dt, kop, p, a, s)
                                  : launch_resident(dt, kop, p, a, s);
    if (e != hipSuccess) {
        if (debug_on()) std::fprintf(stderr, "[nt] launch failed: %s\n", hipGetErrorString(e));
        return NT_ERR_HIP;
    }
    return NT_OK;
}

// Checks shared by every entry point, in the documented order.
// Do the byte ranges [a, a + na) and [b, b + nb) overlap?  (Addresses and
// sizes here stay far below 2^63, so the sums do not wrap.)
bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
    const uint64_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return na && nb && pa < pb + nb && pb < pa + na;
}

uint64_t matrix_bytes(int64_t M, int64_t N, int dt) {
    return (uint64_t)M * (uint64_t)N * (uint64_t)elem_bytes((nt_dtype)dt);
}

nt_status common_checks(int64_t M, int64_t N, int dt, const void *x, const void *y) {
    if (!valid_dtype(dt)) return NT_ERR_DTYPE;
    if (!valid_shape(M, N)) return NT_ERR_SHAPE;
    if (M == 0) return NT_OK;
    if (!x || !y) return NT_ERR_NULL;
    const uintptr_t e = (uintptr_t)elem_bytes((nt_dtype)dt);
    if (!aligned_to(x, e) || !aligned_to(y, e)) return NT_ERR_ALIGN;
    // in place (y == x) is fine; a partial overlap would read outputs as inputs
    const uint64_t b = matrix_bytes(M, N, dt);
    if (x != y && overlaps(x, b, y, b)) return NT_ERR_ALIAS;
    return NT_OK;
}

// A workspace must not overlap x or y.
nt_status workspace_apart(int64_t M, int64_t N, int dt, const void *x, const void *y, const void *ws,
                          size_t wsb) {
    const uint64_t b = matrix_bytes(M, N, dt);
    if (ws && (overlaps(ws, wsb, x, b) || overlaps(ws, wsb, y, b))) return NT_ERR_ALIAS;
    return NT_OK;
}

bool valid_eps(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

}  // namespace

extern "C" {

const char *nt_status_string(nt_status s) {
    switch (s) {
    case NT_OK: return "ok";
    case NT_ERR_NULL: return "a required pointer is NULL";
    case NT_ERR_SHAPE: return "invalid shape (M < 0, N <= 0, N > INT32_MAX, or size overflow)";
    case NT_ERR_DTYPE: return "unknown element type";
    case NT_ERR_EPS: return "eps must be finite and >= 0";
    case NT_ERR_ALIGN: return "pointer not aligned to its element size";
    case NT_ERR_WORKSPACE: return "workspace smaller than nt_softmax_workspace_bytes() / nt_norm_workspace_bytes()";
    case NT_ERR_HIP: return "HIP launch error";
    case NT_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
    case NT_ERR_SCALE: return "scale must be finite and > 0";
    case NT_ERR_OVERRIDE: return "unknown override name or malformed value";
    }
    return "unknown status";
}

nt_status nt_set_override(const char *name, const char *value) {
    if (!name) return NT_ERR_NULL;
    for (int k = 0; k < T_COUNT; ++k) {
        if (std::strcmp(name, kTuneNames[k]) != 0) continue;
        int64_t v = g_tune_loaded[k];
        if (value && !parse_tune(k, value, &v)) return NT_ERR_OVERRIDE;
        g_tune[k].store(v, std::memory_order_relaxed);
        return NT_OK;
    }
    return NT_ERR_OVERRIDE;
}

nt_status nt_plan_launch(nt_op op, int64_t M, int64_t N, nt_dtype dt, int aligned16, nt_plan *out) {
    if (!out) return NT_ERR_NULL;
    if (op != NT_OP_SOFTMAX && op != NT_OP_LAYERNORM && op != NT_OP_RMSNORM && op != NT_OP_ADD_LAYERNORM &&
        op != NT_OP_ADD_RMSNORM && op != NT_OP_SOFTMAX_CAUSAL && op != NT_OP_LAYERNORM_WS && op != NT_OP_RMSNORM_WS)
        return NT_ERR_SHAPE;
    if (!valid_dtype(dt)) return NT_ERR_DTYPE;
    if (!valid_shape(M, N)) return NT_ERR_SHAPE;
    const bool al = aligned16 && (N * elem_bytes(dt)) % 16 == 0;
    const bool res = op == NT_OP_ADD_LAYERNORM || op == NT_OP_ADD_RMSNORM;
    const bool ws = op == NT_OP_LAYERNORM_WS || op == NT_OP_RMSNORM_WS;
    const nt_op base = (op == NT_OP_ADD_LAYERNORM || op == NT_OP_LAYERNORM_WS) ? NT_OP_LAYERNORM
                       : (op == NT_OP_ADD_RMSNORM || op == NT_OP_RMSNORM_WS) ? NT_OP_RMSNORM
                       : op == NT_OP_SOFTMAX_CAUSAL                         ? NT_OP_SOFTMAX
                                                                             : op;
    return make_plan(base, M, N, dt, al, out, true, res, op == NT_OP_SOFTMAX_CAUSAL, ws);
}

size_t nt_softmax_workspace_bytes(int64_t M, int64_t N, nt_dtype dt) {
    if (!valid_dtype(dt) || !valid_shape(M, N) || M == 0) return 0;
    // Sized for the misaligned case, which touches at most one extra chunk
    // per row, so the answer does not depend on the pointers.
    nt_plan p;
    if (make_plan(NT_OP_SOFTMAX, M, N, dt, false, &p) != NT_OK) return 0;
    return (size_t)p.workspace_bytes;
}

// Softmax launch shared by the plain and the causal entry points (a.queries
// > 0 selects the causal kernels); arguments already validated up to the
// workspace.
static nt_status softmax_launch(int64_t M, int64_t N, nt_dtype dt, const void *x, void *y, void *workspace,
                                size_t workspace_bytes, void *stream, ntk::RowArgs &a) {
    const bool al = all_aligned16(N, dt, x, y, nullptr, nullptr);
    nt_plan p;
    nt_status st = make_plan(NT_OP_SOFTMAX, M, N, dt, al, &p, true, false, a.queries > 0);
    if (st != NT_OK) return st;
    a.x = static_cast<const char *>(x);
    a.y = static_cast<char *>(y);
    a.M = M;
    a.N = (int32_t)N;
    a.inv_n = (float)(1.0 / (double)N);
    a.inv_nd = 1.0 / (double)N;
    if (p.split) {
        if (!workspace) return NT_ERR_NULL;
        if (!aligned_to(workspace, 8)) return NT_ERR_ALIGN;
        // The documented requirement (sized for misaligned rows) is enforced,
        // not the possibly smaller need of this particular call.
        const size_t need = nt_softmax_workspace_bytes(M, N, dt);
        if (workspace_bytes < need) return NT_ERR_WORKSPACE;
        if (workspace_apart(M, N, dt, x, y, workspace, workspace_bytes) != NT_OK) return NT_ERR_ALIAS;
        a.ws = static_cast<float2 *>(workspace);
        a.P = (int32_t)p.row_chunks;
        // in place, a chunk recomputed by another workgroup could already
        // hold outputs: the two-kernel form reads x completely first
        if (x == y) p.cooperative = 0;
        if (p.cooperative) {
            // the tag word: the 16 bytes after this plan's records
            const nt_status tst =
                set_coop_tag(stream, static_cast<char *>(workspace), p.workspace_bytes - kTagBytes, a);
            if (tst != NT_OK) return tst;
        }
    }
    return run(NT_OP_SOFTMAX, M, N, dt, p, a, stream);
}

nt_status nt_softmax_rows(int64_t M, int64_t N, nt_dtype dt, const void *x, void *y, void *workspace,
                          size_t workspace_bytes, void *stream) {
    nt_status st = common_checks(M, N, dt, x, y);
    if (st != NT_OK || M == 0) return st;
    ntk::RowArgs a{};
    return softmax_launch(M, N, dt, x, y, workspace, workspace_bytes, stream, a);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Scratch of nt_softmax_rows_noalloc: the split path's workspace (the per
// (row, chunk) records) in a file-scope device array, for callers that
// cannot allocate.  Each device holds its own copy; host code never uses
// the array's name as an address: its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept.  Calls
// that overlap on one device share it and race; nothing in it has to start
// at zero (the records carry a per-call tag, and the two-kernel form writes
// every record before reading any).
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[NT_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<void *> g_scratch[kMaxDevices];

// The scratch array's address on the device `stream` belongs to.
nt_status scratch_for(void *stream, void **out) {
    int dev = 0;
    if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev) != hipSuccess) return NT_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return NT_ERR_HIP;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return NT_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return NT_ERR_HIP;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess || r != hipSuccess || !p) return NT_ERR_HIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return NT_OK;
}

}  // namespace

extern "C" {

nt_status nt_softmax_rows_noalloc(int64_t M, int64_t N, nt_dtype dt, const void *x, void *y, void *stream) {
    nt_status st = common_checks(M, N, dt, x, y);
    if (st != NT_OK || M == 0) return st;
    const size_t need = nt_softmax_workspace_bytes(M, N, dt);
    if (need > (size_t)NT_NOALLOC_SCRATCH_BYTES) return NT_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need) {
        st = scratch_for(stream, &ws);
        if (st != NT_OK) return st;
    }
    ntk::RowArgs a{};
    return softmax_launch(M, N, dt, x, y, ws, need ? (size_t)NT_NOALLOC_SCRATCH_BYTES : 0, stream, a);
}

nt_status nt_softmax_causal_rows(int64_t M, int64_t N, nt_dtype dt, float scale, int64_t queries, int64_t offset,
                                 const void *x, void *y, void *workspace, size_t workspace_bytes, void *stream) {
    if (!valid_dtype(dt)) return NT_ERR_DTYPE;
    if (!valid_shape(M, N)) return NT_ERR_SHAPE;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return NT_ERR_SCALE;
    if (queries < 1 || offset < 0) return NT_ERR_SHAPE;
    nt_status st = common_checks(M, N, dt, x, y);
    if (st != NT_OK || M == 0) return st;
    ntk::RowArgs a{};
    a.queries = queries < M ? queries : M;            // rows r < M: r mod queries is unchanged
    a.offset = offset < N ? offset : N;              // every key visible from there on
    a.s2 = (float)((double)scale * 1.4426950408889634074);
    return softmax_launch(M, N, dt, x, y, workspace, workspace_bytes, stream, a);
}

}  // extern "C"

namespace {

// Workspace of a split-norm plan, or an error status before anything is
// launched; a NULL workspace selected the plain plan already.
// The split norm's workspace checks, and the choice between its one-pass
// (cooperative) and two-kernel forms: in place, the two kernels.
nt_status attach_workspace(nt_plan &p, void *ws, size_t wsb, int64_t M, int64_t N, nt_dtype dt, const void *x,
                           const void *y, void *stream, ntk::RowArgs &a) {
    if (p.split != 3) return NT_OK;
    if (wsb < (size_t)p.workspace_bytes) return NT_ERR_WORKSPACE;
    if (!aligned_to(ws, 8)) return NT_ERR_ALIGN;
    if (workspace_apart(M, N, dt, x, y, ws, wsb) != NT_OK) return NT_ERR_ALIAS;
    a.P = (int32_t)p.row_chunks;
    a.wsd = static_cast<double *>(ws);
    if (x == y) p.cooperative = 0;
    // the tag word: the 16 bytes after this plan's records
    if (p.cooperative) return set_coop_tag(stream, static_cast<char *>(ws), p.workspace_bytes - kTagBytes, a);
    return NT_OK;
}

nt_status layernorm_impl(int64_t M, int64_t N, nt_dtype dt, float eps, const void *x, const void *gamma,
                         const void *beta, void *y, float *mean, float *rstd, void *ws, size_t wsb, void *stream) {
    if (!valid_dtype(dt)) return NT_ERR_DTYPE;
    if (!valid_shape(M, N)) return NT_ERR_SHAPE;
    if (!valid_eps(eps)) return NT_ERR_EPS;
    nt_status st = common_checks(M, N, dt, x, y);
    if (st != NT_OK || M == 0) return st;
    const uintptr_t e = (uintptr_t)elem_bytes(dt);
    if ((gamma && !aligned_to(gamma, e)) || (beta && !aligned_to(beta, e)) || (mean && !aligned_to(mean, 4)) ||
        (rstd && !aligned_to(rstd, 4)))
        return NT_ERR_ALIGN;
    const bool al = all_aligned16(N, dt, x, y, gamma, beta);
    nt_plan p;
    st = make_plan(NT_OP_LAYERNORM, M, N, dt, al, &p, gamma != nullptr && beta != nullptr, false, false,
                   ws != nullptr);
    if (st != NT_OK) return st;
    ntk::RowArgs a{};
    st = attach_workspace(p, ws, wsb, M, N, dt, x, y, stream, a);
    if (st != NT_OK) return st;
    a.x = static_cast<const char *>(x);
    a.y = static_cast<char *>(y);
    a.p0 = static_cast<const char *>(gamma);
    a.p1 = static_cast<const char *>(beta);
    a.mean = mean;
    a.rstd = rstd;
    a.M = M;
    a.N = (int32_t)N;
    a.inv_n = (float)(1.0 / (double)N);
    a.inv_nd = 1.0 / (double)N;
    a.eps = eps;
    return run(NT_OP_LAYERNORM, M, N, dt, p, a, stream);
}

nt_status rmsnorm_impl(int64_t M, int64_t N, nt_dtype dt, float eps, const void *x, const void *weight, void *y,
                       void *ws, size_t wsb, void *stream) {
    if (!valid_dtype(dt)) return NT_ERR_DTYPE;
    if (!valid_shape(M, N)) return NT_ERR_SHAPE;
    if (!valid_eps(eps)) return NT_ERR_EPS;
    nt_status st = common_checks(M, N, dt, x, y);
    if (st != NT_OK || M == 0) return st;
    if (weight && !aligned_to(weight, (uintptr_t)elem_bytes(dt))) return NT_ERR_ALIGN;
    const bool al = all_aligned16(N, dt, x, y, weight, nullptr);
    nt_plan p;
    st = make_plan(NT_OP_RMSNORM, M, N, dt, al, &p, weight != nullptr, false, false, ws != nullptr);
    if (st != NT_OK) return st;
    ntk::RowArgs a{};
    st = attach_workspace(p, ws, wsb, M, N, dt, x, y, stream, a);
    if (st != NT_OK) return st;
    a.x = static_cast<const char *>(x);
    a.y = static_cast<char *>(y);
    a.p0 = static_cast<const char *>(weight);
    a.M = M;
    a.N = (int32_t)N;
    a.inv_n = (float)(1.0 / (double)N);
    a.inv_nd = 1.0 / (double)N;
    a.eps = eps;
    return run(NT_OP_RMSNORM, M, N, dt, p, a, stream);
}

}  // namespace

extern "C" {

nt_status nt_layernorm_rows(int64_t M, int64_t N, nt_dtype dt, float eps, const void *x, const void *gamma,
                            const void *beta, void *y, float *mean, float *rstd, void *stream) {
    return layernorm_impl(M, N, dt, eps, x, gamma, beta, y, mean, rstd, nullptr, 0, stream);
}

nt_status nt_rmsnorm_rows(int64_t M, int64_t N, nt_dtype dt, float eps, const void *x, const void *weight, void *y,
                          void *stream) {
    return rmsnorm_impl(M, N, dt, eps, x, weight, y, nullptr, 0, stream);
}

size_t nt_norm_workspace_bytes(int op, int64_t M, int64_t N, nt_dtype dt) {
    if ((op != NT_OP_LAYERNORM && op != NT_OP_RMSNORM) || !valid_dtype(dt) || !valid_shape(M, N)) return 0;
    size_t need = 0;
    for (const bool al : {true, false}) {      // the larger of the two alignments' plans
        nt_plan p;
        if (make_plan((nt_op)op, M, N, dt, al && (N * elem_bytes(dt)) % 16 == 0, &p, true, false, false, false) !=
                NT_OK ||
            p.split != 2)
            continue;          // rows that fit one pass need nothing
        // and of the two forms' plans, so the size does not depend on NT_COOP
        for (const bool coop : {true, false}) {
            Shape s;
            int64_t P;
            bool c;
            if (split_norm_plan((nt_op)op, dt, M, row_chunks(N, dt, p.aligned != 0), coop, &s, &P, &c) &&
                P <= (((int64_t)1 << 31) / (64 * s.W)) / M && (size_t)(M * P * 32 + M * 8 + kTagBytes) > need)
                need = (size_t)(M * P * 32 + M * 8 + kTagBytes);
        }
    }
    return need;
}

nt_status nt_layernorm_rows_ws(int64_t M, int64_t N, nt_dtype dt, float eps, const void *x, const void *gamma,
                               const void *beta, void *y, float *mean, float *rstd, void *workspace,
                               size_t workspace_bytes, void *stream) {
    return layernorm_impl(M, N, dt, eps, x, gamma, beta, y, mean, rstd, workspace, workspace_bytes, stream);
}

nt_status nt_rmsnorm_rows_ws(int64_t M, int64_t N, nt_dtype dt, float eps, const void *x, const void *weight,
                             void *y, void *workspace, size_t workspace_bytes, void *stream) {
    return rmsnorm_impl(M, N, dt, eps, x, weight, y, workspace, workspace_bytes, stream);
}

// Checks of the fused add + norm entry points beyond common_checks: the
// residual and h present, element-aligned and in x's 16-byte phase, y != h.
static nt_status residual_checks(int64_t M, int64_t N, nt_dtype dt, const void *x, const void *residual,
                                 const void *h, const void *y) {
    if (!residual || !h) return NT_ERR_NULL;
    const uintptr_t e = (uintptr_t)elem_bytes(dt);
    if (!aligned_to(residual, e) || !aligned_to(h, e)) return NT_ERR_ALIGN;
    if ((((uintptr_t)residual ^ (uintptr_t)x) & 15) || (((uintptr_t)h ^ (uintptr_t)x) & 15)) return NT_ERR_ALIGN;
    // h and y may each be x or the residual exactly; no other overlap
    const uint64_t b = matrix_bytes(M, N, dt);
    if (overlaps(h, b, y, b)) return NT_ERR_ALIAS;
    for (const void *in : {x, residual}) {
        if (h != in && overlaps(h, b, in, b)) return NT_ERR_ALIAS;
        if (y != in && overlaps(y, b, in, b)) return NT_ERR_ALIAS;
    }
    return NT_OK;
}

nt_status nt_add_layernorm_rows(int64_t M, int64_t N, nt_dtype dt, float eps, const void *x, const void *residual,
                                const void *gamma, const void *beta, void *h, void *y, float *mean, float *rstd,
                                void *stream) {
    if (!valid_dtype(dt)) return NT_ERR_DTYPE;
    if (!valid_shape(M, N)) return NT_ERR_SHAPE;
    if (!valid_eps(eps)) return NT_ERR_EPS;
    nt_status st = common_checks(M, N, dt, x, y);
    if (st != NT_OK || M == 0) return st;
    st = residual_checks(M, N, dt, x, residual, h, y);
    if (st != NT_OK) return st;
    const uintptr_t e = (uintptr_t)elem_bytes(dt);
    if ((gamma && !aligned_to(gamma, e)) || (beta && !aligned_to(beta, e)) || (mean && !aligned_to(mean, 4)) ||
        (rstd && !aligned_to(rstd, 4)))
        return NT_ERR_ALIGN;
    const bool al = all_aligned16(N, dt, x, y, gamma, beta) && aligned_to(residual, 16) && aligned_to(h, 16);
    nt_plan p;
    st = make_plan(NT_OP_LAYERNORM, M, N, dt, al, &p, gamma != nullptr && beta != nullptr, true);
    if (st != NT_OK) return st;
    ntk::RowArgs a{};
    a.x = static_cast<const char *>(x);
    a.y = static_cast<char *>(y);
    a.r = static_cast<const char *>(residual);
    a.h = static_cast<char *>(h);
    a.p0 = static_cast<const char *>(gamma);
    a.p1 = static_cast<const char *>(beta);
    a.mean = mean;
    a.rstd = rstd;
    a.M = M;
    a.N = (int32_t)N;
    a.inv_n = (float)(1.0 / (double)N);
    a.inv_nd = 1.0 / (double)N;
    a.eps = eps;
    return run(NT_OP_LAYERNORM, M, N, dt, p, a, stream);
}

nt_status nt_add_rmsnorm_rows(int64_t M, int64_t N, nt_dtype dt, float eps, const void *x, const void *residual,
                              const void *weight, void *h, void *y, void *stream) {
    if (!valid_dtype(dt)) return NT_ERR_DTYPE;
    if (!valid_shape(M, N)) return NT_ERR_SHAPE;
    if (!valid_eps(eps)) return NT_ERR_EPS;
    nt_status st = common_checks(M, N, dt, x, y);
    if (st != NT_OK || M == 0) return st;
    st = residual_checks(M, N, dt, x, residual, h, y);
    if (st != NT_OK) return st;
    if (weight && !aligned_to(weight, (uintptr_t)elem_bytes(dt))) return NT_ERR_ALIGN;
    const bool al = all_aligned16(N, dt, x, y, weight, nullptr) && aligned_to(residual, 16) && aligned_to(h, 16);
    nt_plan p;
    st = make_plan(NT_OP_RMSNORM, M, N, dt, al, &p, weight != nullptr, true);
    if (st != NT_OK) return st;
    ntk::RowArgs a{};
    a.x = static_cast<const char *>(x);
    a.y = static_cast<char *>(y);
    a.r = static_cast<const char *>(residual);
    a.h = static_cast<char *>(h);
    a.p0 = static_cast<const char *>(weight);
    a.M = M;
    a.N = (int32_t)N;
    a.inv_n = (float)(1.0 / (double)N);
    a.inv_nd = 1.0 / (double)N;
    a.eps = eps;
    return run(NT_OP_RMSNORM, M, N, dt, p, a, stream);
}

}  // extern "C"

extern "C" {

nt_status nt_attention_fwd(int64_t BH, int64_t Lq, int64_t Lk, int64_t D, nt_dtype dt, float scale, int causal,
                           int64_t offset, const void *q, const void *k, const void *v, void *o, void *stream) {
    if (dt != NT_F16 && dt != NT_BF16) return NT_ERR_DTYPE;
    if (BH < 0 || Lq < 0 || Lk < 1 || (D != 64 && D != 128) || offset < 0 || (causal != 0 && causal != 1))
        return NT_ERR_SHAPE;
    // element counts BH*Lq*D and BH*Lk*D, times 2 bytes, must fit int64; the
    // grid (one 256-thread workgroup per 128 queries of a head) the packet
    if ((BH > 0 && (Lq > INT64_MAX / 4 / D / BH || Lk > INT64_MAX / 4 / D / BH))) return NT_ERR_SHAPE;
    const int64_t nqb = (Lq + 127) / 128;
    if (BH > 0 && nqb > ((int64_t)1 << 31) / 256 / BH) return NT_ERR_SHAPE;
    if (!std::isfinite(scale) || !(scale > 0.0f)) return NT_ERR_SCALE;
    if (BH == 0 || Lq == 0) return NT_OK;
    if (!q || !k || !v || !o) return NT_ERR_NULL;
    for (const void *p : {q, k, v, (const void *)o})
        if (!aligned_to(p, 16)) return NT_ERR_ALIGN;
    const uint64_t qb = (uint64_t)BH * (uint64_t)Lq * (uint64_t)D * 2, kvb = (uint64_t)BH * (uint64_t)Lk * (uint64_t)D * 2;
    if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kvb) || overlaps(o, qb, v, kvb)) return NT_ERR_ALIAS;
    ntk::AttnArgs a{};
    a.q = static_cast<const char *>(q);
    a.k = static_cast<const char *>(k);
    a.v = static_cast<const char *>(v);
    a.o = static_cast<char *>(o);
    a.BH = BH;
    a.Lq = Lq;
    a.Lk = Lk;
    a.offset = offset;
    a.nqb = nqb;
    a.s2 = (float)((double)scale * 1.4426950408889634074);
    a.causal = causal;
    const hipError_t e = ntk::launch_attention(dt == NT_BF16 ? ntk::DT_BF16 : ntk::DT_F16, (int)D, a,
                                               reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        if (debug_on()) std::fprintf(stderr, "[nt] attention launch failed: %s\n", hipGetErrorString(e));
        return NT_ERR_HIP;
    }
    return NT_OK;
}

}  // extern "C"
