// sgemm.hip -- C ABI, argument validation and kernel dispatch of libsgemm.
//
// The operation, layout, ownership and error contract are documented in
// include/sgemm.h.  This file only validates, picks a kernel variant and
// launches it on the caller's stream; all arithmetic runs in the kernels of
// sgemm_kernels.hpp.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/sgemm.h"
#include "sgemm_kernels.hpp"

namespace libsgemm {
namespace {

using LaunchFn = hipError_t (*)(const GemmArgs&, hipStream_t);

enum Kind { kMfma = 0, kValu = 1 };

struct Variant {
    const char* name;
    int kind;
    int bm, bn, bk, wm, wn;  // wm/wn: MFMA wave tile, or VALU microtile tm/tn
    int threads;
    int vec;
    int lds_bytes;
    LaunchFn launch;
    int wide;  // 64-bit per-lane load offsets (no 4 GiB limit on one workgroup's operand span)
    int ks;    // k-groups sharing one tile inside a workgroup (split-K); 0 means 1
    int ta;    // op(A) = A^T: A stored K x M
    int tb;    // op(B) = B^T: B stored N x K
};

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Tile-rows per group of the workgroup -> tile map.  Measured on 4096^3 and 8192^3 with the
// 128x128 tile over groups of 4, 8, 16 and 32 rows, with and without the XCD renumbering:
// 4096^3 is insensitive (all within 0.3 %), 8192^3 is fastest with the renumbering and groups
// of 4 (151.6 TFLOP/s against 148.5-150.4 for 8 and 16).
int group_rows(int tiles_m, int tiles_n) {
    (void)tiles_n;
    return tiles_m < 4 ? tiles_m : 4;
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC, int OCC, bool WIDE, bool TA = false, bool TB = false>
hipError_t launch_mfma(const GemmArgs& g, hipStream_t stream) {
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN, VEC, TA, TB>;
    int tiles_m = ceil_div(g.M, BM), tiles_n = ceil_div(g.N, BN);
    int group_m = group_rows(tiles_m, tiles_n);
    GemmArgs a = g;
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(&sgemm_mfma_kernel<BM, BN, BK, WM, WN, VEC, OCC, WIDE, TA, TB>),
                           dim3(tiles_m * tiles_n), dim3(Cfg::NT), args, 0, stream);
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC, int OCC>
hipError_t launch_mfma_deep(const GemmArgs& g, hipStream_t stream) {
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN, VEC>;
    int tiles_m = ceil_div(g.M, BM), tiles_n = ceil_div(g.N, BN);
    int group_m = group_rows(tiles_m, tiles_n);
    GemmArgs a = g;
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(&sgemm_mfma_deep_kernel<BM, BN, BK, WM, WN, VEC, OCC>),
                           dim3(tiles_m * tiles_n), dim3(Cfg::NT), args, 0, stream);
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC, int OCC, bool WIDE>
hipError_t launch_mfma_pipe(const GemmArgs& g, hipStream_t stream) {
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN, VEC>;
    int tiles_m = ceil_div(g.M, BM), tiles_n = ceil_div(g.N, BN);
    int group_m = group_rows(tiles_m, tiles_n);
    GemmArgs a = g;
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(&sgemm_mfma_pipe_kernel<BM, BN, BK, WM, WN, VEC, OCC, WIDE>),
                           dim3(tiles_m * tiles_n), dim3(Cfg::NT), args, 0, stream);
}

template <int BM, int BN, int BK, int WM, int WN, int KS, bool VEC>
hipError_t launch_mfma_splitk(const GemmArgs& g, hipStream_t stream) {
    using Cfg = SplitKCfg<BM, BN, BK, WM, WN, KS, VEC>;
    int tiles_m = ceil_div(g.M, BM), tiles_n = ceil_div(g.N, BN);
    int group_m = group_rows(tiles_m, tiles_n);
    GemmArgs a = g;
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(&sgemm_mfma_splitk_kernel<BM, BN, BK, WM, WN, KS, VEC>),
                           dim3(tiles_m * tiles_n), dim3(Cfg::NT), args, 0, stream);
}

template <int BM, int BN, int BK, int TM, int TN, bool VEC, bool WIDE>
hipError_t launch_valu(const GemmArgs& g, hipStream_t stream) {
    using Cfg = ValuCfg<BM, BN, BK, TM, TN, VEC>;
    int tiles_m = ceil_div(g.M, BM), tiles_n = ceil_div(g.N, BN);
    int group_m = group_rows(tiles_m, tiles_n);
    GemmArgs a = g;
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(&sgemm_valu_kernel<BM, BN, BK, TM, TN, VEC, WIDE>),
                           dim3(tiles_m * tiles_n), dim3(Cfg::NT), args, 0, stream);
}

#define MFMA_VARIANT(BM, BN, BK, WM, WN, OCC, VEC, NAME)                                       \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES, &launch_mfma<BM, BN, BK, WM, WN, VEC, OCC, false>, 0}
#define WIDE_MFMA_VARIANT(BM, BN, BK, WM, WN, VEC, NAME)                                         \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES, &launch_mfma<BM, BN, BK, WM, WN, VEC, 0, true>, 1}
#define VALU_VARIANT(BM, BN, BK, TM, TN, VEC, SUFFIX)                                             \
    {"valu_" #BM "x" #BN "x" #BK "_t" #TM "x" #TN SUFFIX, kValu, BM, BN, BK, TM, TN,              \
     ValuCfg<BM, BN, BK, TM, TN, VEC>::NT, VEC, ValuCfg<BM, BN, BK, TM, TN, VEC>::LDS_BYTES,     \
     &launch_valu<BM, BN, BK, TM, TN, VEC, false>, 0}
#define MFMA_NAME(BM, BN, BK, WM, WN) "mfma32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN
#define BOTH_MFMA(BM, BN, BK, WM, WN)                                                       \
    MFMA_VARIANT(BM, BN, BK, WM, WN, 0, true, MFMA_NAME(BM, BN, BK, WM, WN) "_vec"),        \
        MFMA_VARIANT(BM, BN, BK, WM, WN, 0, false, MFMA_NAME(BM, BN, BK, WM, WN) "_scalar")
// vector-load form only, with an occupancy target of OCC waves per SIMD
#define VEC_MFMA_OCC(BM, BN, BK, WM, WN, OCC) \
    MFMA_VARIANT(BM, BN, BK, WM, WN, OCC, true, MFMA_NAME(BM, BN, BK, WM, WN) "_o" #OCC "_vec")
#define PIPE_VARIANT(BM, BN, BK, WM, WN, OCC, VEC, NAME)                                       \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES, &launch_mfma_pipe<BM, BN, BK, WM, WN, VEC, OCC, false>, 0}
#define PIPE_NAME(BM, BN, BK, WM, WN, OCC) "mfma32p_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_o" #OCC
#define BOTH_PIPE(BM, BN, BK, WM, WN, OCC)                                                      \
    PIPE_VARIANT(BM, BN, BK, WM, WN, OCC, true, PIPE_NAME(BM, BN, BK, WM, WN, OCC) "_vec"),     \
        PIPE_VARIANT(BM, BN, BK, WM, WN, OCC, false, PIPE_NAME(BM, BN, BK, WM, WN, OCC) "_scalar")
#define SPLITK_VARIANT(BM, BN, BK, WM, WN, KS, VEC, NAME)                                     \
    {NAME, kMfma, BM, BN, BK, WM, WN, SplitKCfg<BM, BN, BK, WM, WN, KS, VEC>::NT, VEC,            \
     SplitKCfg<BM, BN, BK, WM, WN, KS, VEC>::LDS_BYTES, &launch_mfma_splitk<BM, BN, BK, WM, WN, KS, VEC>, 0, KS}
#define SPLITK_NAME(BM, BN, BK, WM, WN, KS) "mfma32k" #KS "_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN
#define BOTH_SPLITK(BM, BN, BK, WM, WN, KS)                                                     \
    SPLITK_VARIANT(BM, BN, BK, WM, WN, KS, true, SPLITK_NAME(BM, BN, BK, WM, WN, KS) "_vec"),   \
        SPLITK_VARIANT(BM, BN, BK, WM, WN, KS, false, SPLITK_NAME(BM, BN, BK, WM, WN, KS) "_scalar")
#define TRANS_VARIANT(BM, BN, BK, WM, WN, VEC, WIDE, TA, TB, NAME)                              \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC, TA, TB>::NT, VEC,          \
     MfmaCfg<BM, BN, BK, WM, WN, VEC, TA, TB>::LDS_BYTES,                                         \
     &launch_mfma<BM, BN, BK, WM, WN, VEC, 0, WIDE, TA, TB>, WIDE, 0, TA, TB}
// the variants of one transposition (TAG: "nt", "tn" or "tt"; first letter op(A), second op(B))
#define TRANS_SET(TA, TB, TAG)                                                                     \
    TRANS_VARIANT(128, 128, 16, 64, 64, true, false, TA, TB, MFMA_NAME(128, 128, 16, 64, 64) "_" TAG "_vec"),     \
        TRANS_VARIANT(128, 128, 16, 64, 64, false, false, TA, TB, MFMA_NAME(128, 128, 16, 64, 64) "_" TAG "_scalar"), \
        TRANS_VARIANT(64, 64, 32, 32, 32, true, false, TA, TB, MFMA_NAME(64, 64, 32, 32, 32) "_" TAG "_vec"),         \
        TRANS_VARIANT(64, 64, 32, 32, 32, false, false, TA, TB, MFMA_NAME(64, 64, 32, 32, 32) "_" TAG "_scalar"),     \
        TRANS_VARIANT(128, 128, 16, 64, 64, true, true, TA, TB, MFMA_NAME(128, 128, 16, 64, 64) "_" TAG "_wide_vec"), \
        TRANS_VARIANT(128, 128, 16, 64, 64, false, true, TA, TB, MFMA_NAME(128, 128, 16, 64, 64) "_" TAG "_wide_scalar")
#define DEEP_VARIANT(BM, BN, BK, WM, WN, VEC, NAME)                                             \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES, &launch_mfma_deep<BM, BN, BK, WM, WN, VEC, 0>, 0}
#define DEEP_NAME(BM, BN, BK, WM, WN) "mfma32d_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN
#define BOTH_DEEP(BM, BN, BK, WM, WN)                                                        \
    DEEP_VARIANT(BM, BN, BK, WM, WN, true, DEEP_NAME(BM, BN, BK, WM, WN) "_vec"),            \
        DEEP_VARIANT(BM, BN, BK, WM, WN, false, DEEP_NAME(BM, BN, BK, WM, WN) "_scalar")
#define BOTH_VALU(BM, BN, BK, TM, TN) \
    VALU_VARIANT(BM, BN, BK, TM, TN, true, "_vec"), VALU_VARIANT(BM, BN, BK, TM, TN, false, "_scalar")

// The variant table.  Ids are positions in this table.
const Variant kVariants[] = {
    BOTH_MFMA(128, 128, 16, 64, 64),
    BOTH_MFMA(128, 128, 32, 64, 64),
    BOTH_MFMA(256, 128, 16, 128, 64),
    BOTH_MFMA(128, 256, 16, 64, 128),
    BOTH_MFMA(256, 64, 16, 64, 64),
    BOTH_MFMA(64, 64, 16, 32, 32),
    BOTH_MFMA(64, 64, 32, 32, 32),
    VEC_MFMA_OCC(128, 128, 16, 64, 64, 4),
    MFMA_VARIANT(128, 128, 16, 64, 64, 4, false, MFMA_NAME(128, 128, 16, 64, 64) "_o4_scalar"),
    VEC_MFMA_OCC(128, 128, 32, 64, 64, 2),
    PIPE_VARIANT(128, 128, 32, 64, 64, 2, true, PIPE_NAME(128, 128, 32, 64, 64, 2) "_vec"),
    BOTH_PIPE(256, 128, 16, 64, 64, 2),
    BOTH_PIPE(64, 64, 16, 32, 32, 4),
    BOTH_PIPE(256, 64, 16, 64, 64, 2),
    PIPE_VARIANT(128, 256, 16, 64, 128, 2, true, PIPE_NAME(128, 256, 16, 64, 128, 2) "_vec"),
    PIPE_VARIANT(256, 128, 16, 128, 64, 2, true, PIPE_NAME(256, 128, 16, 128, 64, 2) "_vec"),
    BOTH_SPLITK(64, 64, 32, 32, 32, 2),
    BOTH_SPLITK(64, 64, 32, 32, 32, 4),
    BOTH_MFMA(64, 64, 64, 32, 32),
    BOTH_MFMA(128, 64, 32, 64, 64),
    BOTH_MFMA(128, 64, 64, 64, 64),
    BOTH_MFMA(64, 64, 32, 64, 32),
    BOTH_VALU(128, 128, 8, 8, 8),
    BOTH_VALU(64, 64, 16, 4, 4),
    // 64-bit offsets: used whenever one workgroup's operand span does not fit 32-bit offsets
    WIDE_MFMA_VARIANT(128, 128, 16, 64, 64, true, MFMA_NAME(128, 128, 16, 64, 64) "_wide_vec"),
    WIDE_MFMA_VARIANT(128, 128, 16, 64, 64, false, MFMA_NAME(128, 128, 16, 64, 64) "_wide_scalar"),
    // deep prefetch (one wave per SIMD)
    BOTH_DEEP(64, 64, 32, 32, 32),
    BOTH_DEEP(64, 64, 64, 32, 32),
    // transposed operands (sgemm_op): op(A) x op(B) = N x T, T x N, T x T
    TRANS_SET(false, true, "nt"),
    TRANS_SET(true, false, "tn"),
    TRANS_SET(true, true, "tt"),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

// Shape classes of the dispatch table.
enum ShapeClass { kSkinny = 0, kSmall = 1, kLarge = 2, kHuge = 3, kShallow = 4, kNumClasses = 5 };

struct TableEntry {
    int shape_class;
    int vec;
    const char* variant;
};

// Default choice per (shape class, alignment class); regenerated by the autotuner.
#include "tuned_table.inc"

int find_variant(const char* name) {
    for (int i = 0; i < kNumVariants; ++i)
        if (std::strcmp(kVariants[i].name, name) == 0) return i;
    return -1;
}

struct DispatchTable {
    int id[kNumClasses][2];
    DispatchTable() {
        for (int c = 0; c < kNumClasses; ++c) {
            id[c][0] = find_variant("mfma32_128x128x16_w64x64_scalar");
            id[c][1] = find_variant("mfma32_128x128x16_w64x64_vec");
        }
        for (const TableEntry& e : kTunedTable) {
            int v = find_variant(e.variant);
            // a vector-load variant may only serve the vector-eligible class
            if (v >= 0 && e.shape_class >= 0 && e.shape_class < kNumClasses && (e.vec || !kVariants[v].vec))
                id[e.shape_class][e.vec ? 1 : 0] = v;
        }
    }
};

const DispatchTable& dispatch_table() {
    static const DispatchTable t;
    return t;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// One call's arguments.  op(A) is M x K and op(B) is K x N; the stored A is M x K (row length
// K) or, when ta, K x M (row length M); the stored B is K x N or, when tb, N x K.
struct Problem {
    bool ta, tb;
    int M, N, K;
    float alpha, beta;
    const float* A;
    int lda;
    const float* B;
    int ldb;
    float* C;
    int ldc;
    int a_rows() const { return ta ? K : M; }
    int a_cols() const { return ta ? M : K; }
    int b_rows() const { return tb ? N : K; }
    int b_cols() const { return tb ? K : N; }
};

// Arguments, for error reporting; each entry point maps them to its own 1-based positions.
enum Arg {
    kArgTransA = 1, kArgTransB, kArgM, kArgN, kArgK, kArgAlpha, kArgA, kArgLda, kArgB, kArgLdb, kArgBeta,
    kArgC, kArgLdc, kArgStream, kArgVariant, kNumArgs
};
// positions in sgemm / sgemm_ex (no transposition arguments) and in sgemm_op / sgemm_op_ex
const int kPosPlain[kNumArgs] = {0, 0, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13};
const int kPosOp[kNumArgs] = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15};

// Precondition of the 128-bit load/store variants: every operand row starts 16-byte aligned
// and has a multiple of 4 elements.
bool vec_ok(const Problem& p) {
    return aligned16(p.A) && aligned16(p.B) && aligned16(p.C) && (p.lda % 4 == 0) && (p.ldb % 4 == 0) &&
           (p.ldc % 4 == 0) && (p.a_cols() % 4 == 0) && (p.b_cols() % 4 == 0) && (p.N % 4 == 0);
}

// Do one workgroup's A and B panels fit 32-bit per-lane byte offsets? (narrow variants only)
bool offsets_fit(const Variant& v, const Problem& p) {
    if (v.wide) return true;
    const unsigned long long lim = 1ull << 32;
    const unsigned long long a_rows = v.ta ? v.bk : v.bm, a_cols = v.ta ? v.bm : v.bk;
    const unsigned long long b_rows = v.tb ? v.bn : v.bk, b_cols = v.tb ? v.bk : v.bn;
    const unsigned long long a = ((a_rows - 1) * (unsigned)p.lda + a_cols) * 4ull;
    const unsigned long long b = ((b_rows - 1) * (unsigned)p.ldb + b_cols) * 4ull;
    return a < lim && b < lim;
}

// skinny: N <= 64; small: fewer than 256 output tiles of 128x128 (under one per CU);
// large: up to 2048 such tiles; huge: more; shallow: a large tile count with K <= 1024 (each
// tile's K loop is short, so the last round of tiles weighs more: smaller tiles win there).
int shape_class(int M, int N, int K) {
    if (N <= 64) return kSkinny;
    long tiles128 = (long)ceil_div(M, 128) * ceil_div(N, 128);
    if (tiles128 < 256) return kSmall;
    if (tiles128 < 2048) return K <= 1024 ? kShallow : kLarge;
    return kHuge;
}

int wide_fallback(bool vec) {
    static const int ids[2] = {find_variant(MFMA_NAME(128, 128, 16, 64, 64) "_wide_scalar"),
                               find_variant(MFMA_NAME(128, 128, 16, 64, 64) "_wide_vec")};
    return ids[vec ? 1 : 0];
}

// Transposed-operand dispatch: [ta*2+tb-1][small/large][vec], and the wide forms [..][vec].
struct TransTable {
    int id[3][2][2];
    int wide[3][2];
    TransTable() {
        static const char* tags[3] = {"nt", "tn", "tt"};
        char name[96];
        for (int c = 0; c < 3; ++c) {
            for (int vec = 0; vec < 2; ++vec) {
                const char* suffix = vec ? "vec" : "scalar";
                std::snprintf(name, sizeof(name), MFMA_NAME(64, 64, 32, 32, 32) "_%s_%s", tags[c], suffix);
                id[c][0][vec] = find_variant(name);
                std::snprintf(name, sizeof(name), MFMA_NAME(128, 128, 16, 64, 64) "_%s_%s", tags[c], suffix);
                id[c][1][vec] = find_variant(name);
                std::snprintf(name, sizeof(name), MFMA_NAME(128, 128, 16, 64, 64) "_%s_wide_%s", tags[c], suffix);
                wide[c][vec] = find_variant(name);
            }
        }
    }
};

const TransTable& trans_table() {
    static const TransTable t;
    return t;
}

int select_variant(const Problem& p) {
    const bool v = vec_ok(p);
    const int cls = shape_class(p.M, p.N, p.K);
    if (!p.ta && !p.tb) {
        const int id = dispatch_table().id[cls][v ? 1 : 0];
        return offsets_fit(kVariants[id], p) ? id : wide_fallback(v);
    }
    const int combo = (p.ta ? 2 : 0) + (p.tb ? 1 : 0) - 1;
    const bool big = cls == kLarge || cls == kHuge || cls == kShallow;
    const int id = trans_table().id[combo][big ? 1 : 0][v ? 1 : 0];
    return offsets_fit(kVariants[id], p) ? id : trans_table().wide[combo][v ? 1 : 0];
}

// Argument checks shared by every computing entry point.  Returns 0 or -Arg.
int validate(const Problem& p) {
    if (p.M < 0) return -kArgM;
    if (p.N < 0) return -kArgN;
    if (p.K < 0) return -kArgK;
    if (p.lda < (p.a_cols() > 1 ? p.a_cols() : 1)) return -kArgLda;
    if (p.ldb < (p.b_cols() > 1 ? p.b_cols() : 1)) return -kArgLdb;
    if (p.ldc < (p.N > 1 ? p.N : 1)) return -kArgLdc;
    if (p.M == 0 || p.N == 0) return 0;
    if (p.C == nullptr) return -kArgC;
    const bool reads_ab = p.alpha != 0.f && p.K > 0;
    if (reads_ab && p.A == nullptr) return -kArgA;
    if (reads_ab && p.B == nullptr) return -kArgB;
    // C must not overlap A or B (byte ranges of the addressed elements).
    const uintptr_t c0 = reinterpret_cast<uintptr_t>(p.C);
    const uintptr_t c1 = c0 + ((uintptr_t)(p.M - 1) * (uintptr_t)p.ldc + (uintptr_t)p.N) * sizeof(float);
    if (reads_ab) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(p.A);
        const uintptr_t a1 =
            a0 + ((uintptr_t)(p.a_rows() - 1) * (uintptr_t)p.lda + (uintptr_t)p.a_cols()) * sizeof(float);
        if (a0 < c1 && c0 < a1) return -kArgC;
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(p.B);
        const uintptr_t b1 =
            b0 + ((uintptr_t)(p.b_rows() - 1) * (uintptr_t)p.ldb + (uintptr_t)p.b_cols()) * sizeof(float);
        if (b0 < c1 && c0 < b1) return -kArgC;
    }
    return 0;
}

hipError_t launch_scale(int M, int N, float beta, float* C, int ldc, hipStream_t stream) {
    if (beta == 1.f) return hipSuccess;  // C := 1 * C is the identity
    long total = (long)M * N;
    long blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    long ldcl = ldc;
    void* args[] = {&M, &N, &beta, &C, &ldcl};
    return hipLaunchKernel(reinterpret_cast<const void*>(&sgemm_scale_kernel), dim3((unsigned)blocks), dim3(256),
                           args, 0, stream);
}

// Returns 0, a positive hipError_t, or -Arg.
int run(const Problem& p, hipStream_t stream, int variant) {
    int rc = validate(p);
    if (rc != 0) return rc;
    if (variant >= kNumVariants) return -kArgVariant;
    if (p.M == 0 || p.N == 0) return 0;
    if (p.alpha == 0.f || p.K == 0) return (int)launch_scale(p.M, p.N, p.beta, p.C, p.ldc, stream);
    if (variant < 0) {
        variant = select_variant(p);
        if (variant < 0) return -kArgVariant;
    }
    const Variant& v = kVariants[variant];
    if ((v.ta != 0) != p.ta || (v.tb != 0) != p.tb) return -kArgVariant;
    if (v.vec && !vec_ok(p)) return -kArgVariant;
    if (!offsets_fit(v, p)) return -kArgVariant;
    const long tiles = (long)ceil_div(p.M, v.bm) * (long)ceil_div(p.N, v.bn);
    if (tiles > INT_MAX) return -kArgM;
    GemmArgs g{p.M, p.N, p.K, p.alpha, p.beta, p.A, (long)p.lda, p.B, (long)p.ldb, p.C, (long)p.ldc};
    return (int)v.launch(g, stream);
}

// 'N'/'n': as stored; 'T'/'t' or 'C'/'c' (real data: the conjugate transpose is the transpose).
int parse_trans(char c) {
    if (c == 'N' || c == 'n') return 0;
    if (c == 'T' || c == 't' || c == 'C' || c == 'c') return 1;
    return -1;
}

int run_entry(const Problem& p, hipStream_t stream, int variant, const int* pos) {
    const int rc = run(p, stream, variant);
    return rc < 0 ? -pos[-rc] : rc;
}

int run_op(char transa, char transb, int M, int N, int K, float alpha, const float* A, int lda, const float* B,
           int ldb, float beta, float* C, int ldc, hipStream_t stream, int variant) {
    const int ta = parse_trans(transa), tb = parse_trans(transb);
    if (ta < 0) return -kPosOp[kArgTransA];
    if (tb < 0) return -kPosOp[kArgTransB];
    const Problem p{ta != 0, tb != 0, M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
    return run_entry(p, stream, variant, kPosOp);
}

}  // namespace
}  // namespace libsgemm

extern "C" {

int sgemm(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb, float beta, float* C,
          int ldc, hipStream_t stream) {
    const libsgemm::Problem p{false, false, M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
    return libsgemm::run_entry(p, stream, -1, libsgemm::kPosPlain);
}

int sgemm_ex(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
             float* C, int ldc, hipStream_t stream, int variant) {
    const libsgemm::Problem p{false, false, M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
    return libsgemm::run_entry(p, stream, variant, libsgemm::kPosPlain);
}

int sgemm_op(char transa, char transb, int M, int N, int K, float alpha, const float* A, int lda, const float* B,
             int ldb, float beta, float* C, int ldc, hipStream_t stream) {
    return libsgemm::run_op(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, -1);
}

int sgemm_op_ex(char transa, char transb, int M, int N, int K, float alpha, const float* A, int lda,
                const float* B, int ldb, float beta, float* C, int ldc, hipStream_t stream, int variant) {
    return libsgemm::run_op(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant);
}

int sgemm_num_variants(void) { return libsgemm::kNumVariants; }

const char* sgemm_variant_name(int variant) {
    if (variant < 0 || variant >= libsgemm::kNumVariants) return nullptr;
    return libsgemm::kVariants[variant].name;
}

int sgemm_variant_info(int variant, int* info, int n) {
    if (variant < 0 || variant >= libsgemm::kNumVariants || info == nullptr || n < 9) return -1;
    const libsgemm::Variant& v = libsgemm::kVariants[variant];
    info[0] = v.kind;
    info[1] = v.bm;
    info[2] = v.bn;
    info[3] = v.bk;
    info[4] = v.wm;
    info[5] = v.wn;
    info[6] = v.threads;
    info[7] = v.vec;
    info[8] = v.lds_bytes;
    if (n >= 10) info[9] = v.wide;
    if (n >= 11) info[10] = v.ks > 1 ? v.ks : 1;
    if (n >= 13) {
        info[11] = v.ta;
        info[12] = v.tb;
    }
    return 0;
}

int sgemm_select_variant(int M, int N, int K, const float* A, int lda, const float* B, int ldb, const float* C,
                         int ldc) {
    return sgemm_op_select_variant('N', 'N', M, N, K, A, lda, B, ldb, C, ldc);
}

int sgemm_op_select_variant(char transa, char transb, int M, int N, int K, const float* A, int lda,
                            const float* B, int ldb, const float* C, int ldc) {
    const int ta = libsgemm::parse_trans(transa), tb = libsgemm::parse_trans(transb);
    if (ta < 0 || tb < 0 || M <= 0 || N <= 0 || K <= 0) return -1;
    const libsgemm::Problem p{ta != 0, tb != 0, M, N, K, 1.f, 0.f, A, lda, B, ldb, const_cast<float*>(C), ldc};
    if (lda < p.a_cols() || ldb < p.b_cols() || ldc < N) return -1;
    return libsgemm::select_variant(p);
}

int sgemm_tile_order(int tiles_m, int tiles_n, int group_m, int* tile_m, int* tile_n) {
    if (tiles_m <= 0 || tiles_n <= 0 || group_m <= 0 || tile_m == nullptr || tile_n == nullptr) return -1;
    const long total = (long)tiles_m * tiles_n;
    if (total > INT_MAX) return -1;
    for (int w = 0; w < (int)total; ++w) libsgemm::tile_of(w, (int)total, tiles_m, tiles_n, group_m, tile_m[w], tile_n[w]);
    return 0;
}

const char* sgemm_version(void) { return "libsgemm 0.1.0 (gfx950)"; }

}  // extern "C"
