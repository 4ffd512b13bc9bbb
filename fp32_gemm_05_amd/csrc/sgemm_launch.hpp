// sgemm_launch.hpp -- the kernel variants of libsgemm: how each is launched (grid, block,
// workgroup-to-tile grouping) and the table of all variants with their tile parameters.
// Included by sgemm.hip only, inside its anonymous namespace; the kernels themselves are in
// sgemm_kernels.hpp (one header per kernel family).  Together they fix what runs on the GPU for a given variant;
// which variant runs for a given call is decided in sgemm.hip and tuned_table.inc.
#pragma once

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
    int bq;    // B loaded in k-quads and staged n-major in LDS (KQuadLoader; 32-bit loads only)
    int dl;    // operands loaded straight into LDS (global_load_lds), a ring of `dl` LDS stages
    int ps;    // persistent: one workgroup per resident slot, looping over tiles
    int mb;    // MFMA block edge: 0 for 32x32 blocks (or a VALU kernel), 16 for 16x16 blocks
};

// 64-bit sum: a + b - 1 would overflow int for a near INT_MAX.
inline int ceil_div(int a, int b) { return (int)(((long)a + b - 1) / b); }

// Tile-rows per group of the workgroup -> tile map.  Measured on 4096^3 and 8192^3 with the
// 128x128 tile over groups of 4, 8, 16 and 32 rows, with and without the XCD renumbering:
// 4096^3 is insensitive (all within 0.3 %), 8192^3 is fastest with the renumbering and groups
// of 4 (151.6 TFLOP/s against 148.5-150.4 for 8 and 16).
int group_rows(int tiles_m, int tiles_n) {
    (void)tiles_n;
    return tiles_m < 4 ? tiles_m : 4;
}

// Compute units of the current device (cached per device id).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// First workgroup of the last round of an nwg-workgroup grid of `kernel`: the workgroups from
// there on start in slots that no later workgroup refills.  resident_per_cu is the kernel's
// occupancy (workgroups per CU); 0 when unknown, which puts the whole grid in the last round.
// INT_MAX (ordering off) when the grid has no more workgroups than the device has CUs.
int drain_from(int nwg, int resident_per_cu) {
    const int cus = device_cus();
    if (cus > 0 && nwg <= cus) return INT_MAX;
    const long resident = (long)resident_per_cu * cus;
    return resident <= 0 || resident >= nwg ? 0 : (int)(nwg - resident);
}

template <typename Kernel>
int occupancy(Kernel kernel, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) n = 0;
    return n;
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC, int OCC, bool WIDE, bool TA = false, bool TB = false,
          int FAIR = 0, bool NTA = false, bool BQ = false>
hipError_t launch_mfma(const GemmArgs& g, hipStream_t stream) {
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN, VEC, TA, TB, BQ>;
    auto kernel = &sgemm_mfma_kernel<BM, BN, BK, WM, WN, VEC, OCC, WIDE, TA, TB, FAIR, NTA, BQ>;
    int tiles_m = ceil_div(g.M, BM), tiles_n = ceil_div(g.N, BN);
    int group_m = group_rows(tiles_m, tiles_n);
    GemmArgs a = g;
    if (FAIR > 0) {
        static const int per_cu = occupancy(kernel, Cfg::NT);
        a.drain_from = drain_from(tiles_m * tiles_n, per_cu);
    }
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(tiles_m * tiles_n), dim3(Cfg::NT), args, 0,
                           stream);
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC, int OCC, int FAIR = 0, bool NTA = false,
          bool CPRE = false, bool ACC2 = false>
hipError_t launch_mfma_deep(const GemmArgs& g, hipStream_t stream) {
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN, VEC>;
    auto kernel = &sgemm_mfma_deep_kernel<BM, BN, BK, WM, WN, VEC, OCC, FAIR, NTA, CPRE, ACC2>;
    int tiles_m = ceil_div(g.M, BM), tiles_n = ceil_div(g.N, BN);
    int group_m = group_rows(tiles_m, tiles_n);
    GemmArgs a = g;
    if (FAIR > 0) {
        static const int per_cu = occupancy(kernel, Cfg::NT);
        a.drain_from = drain_from(tiles_m * tiles_n, per_cu);
    }
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(tiles_m * tiles_n), dim3(Cfg::NT), args, 0,
                           stream);
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int W, int OCC, int FAIR = 0, bool CPRE = false,
          bool SPREAD = false, int MB = 32, int EB = 0, bool NTA = false>
hipError_t launch_mfma_dl(const GemmArgs& g, hipStream_t stream) {
    using Cfg = DlCfg<BM, BN, BK, WM, WN, STAGES, W, MB>;
    auto kernel = &sgemm_mfma_dl_kernel<BM, BN, BK, WM, WN, STAGES, W, OCC, FAIR, CPRE, SPREAD, MB, EB, NTA>;
    int tiles_m = ceil_div(g.M, BM), tiles_n = ceil_div(g.N, BN);
    int group_m = group_rows(tiles_m, tiles_n);
    GemmArgs a = g;
    if (FAIR > 0) {
        static const int per_cu = occupancy(kernel, Cfg::NT);
        a.drain_from = drain_from(tiles_m * tiles_n, per_cu);
    }
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(tiles_m * tiles_n), dim3(Cfg::NT), args, 0,
                           stream);
}

// Persistent form: one workgroup per resident slot (occupancy x CUs, at most one per tile).
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int W, int OCC, bool SPREAD = false>
hipError_t launch_mfma_dlp(const GemmArgs& g, hipStream_t stream) {
    using Cfg = DlCfg<BM, BN, BK, WM, WN, STAGES, W>;
    auto kernel = &sgemm_mfma_dlp_kernel<BM, BN, BK, WM, WN, STAGES, W, OCC, SPREAD>;
    int tiles_m = ceil_div(g.M, BM), tiles_n = ceil_div(g.N, BN);
    int group_m = group_rows(tiles_m, tiles_n);
    static const int per_cu = occupancy(kernel, Cfg::NT);
    const long slots = (long)(per_cu > 0 ? per_cu : 1) * (device_cus() > 0 ? device_cus() : 1);
    const long tiles = (long)tiles_m * tiles_n;
    const int grid = (int)(tiles < slots ? tiles : slots);
    GemmArgs a = g;
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(Cfg::NT), args, 0, stream);
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC, int OCC, bool WIDE, int FAIR = 0>
hipError_t launch_mfma_pipe(const GemmArgs& g, hipStream_t stream) {
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN, VEC>;
    auto kernel = &sgemm_mfma_pipe_kernel<BM, BN, BK, WM, WN, VEC, OCC, WIDE, FAIR>;
    int tiles_m = ceil_div(g.M, BM), tiles_n = ceil_div(g.N, BN);
    int group_m = group_rows(tiles_m, tiles_n);
    GemmArgs a = g;
    if (FAIR > 0) {
        static const int per_cu = occupancy(kernel, Cfg::NT);
        a.drain_from = drain_from(tiles_m * tiles_n, per_cu);
    }
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(tiles_m * tiles_n), dim3(Cfg::NT), args, 0,
                           stream);
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

template <bool VEC, int D, bool TA = false, bool TB = false, bool CPRE = false>
hipError_t launch_mfma_direct(const GemmArgs& g, hipStream_t stream) {
    int tiles_m = ceil_div(g.M, 32), tiles_n = ceil_div(g.N, 32);
    int group_m = group_rows(tiles_m, tiles_n);
    GemmArgs a = g;
    void* args[] = {&a, &tiles_m, &tiles_n, &group_m};
    return hipLaunchKernel(reinterpret_cast<const void*>(&sgemm_mfma_direct_kernel<VEC, D, TA, TB, CPRE>),
                           dim3(tiles_m * tiles_n), dim3(64), args, 0, stream);
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

// ---- The variant table: the macros that spell out its rows, then the rows.  A row's name
// encodes its template configuration (tile, wave tile, loads, schedule, flags). ----
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
#define TRANS_VARIANT(BM, BN, BK, WM, WN, VEC, WIDE, TA, TB, FAIR, NAME)                        \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC, TA, TB>::NT, VEC,          \
     MfmaCfg<BM, BN, BK, WM, WN, VEC, TA, TB>::LDS_BYTES,                                         \
     &launch_mfma<BM, BN, BK, WM, WN, VEC, 0, WIDE, TA, TB, FAIR>, WIDE, 0, TA, TB}
// streamed A with B transposed (op(B) = B^T): the skinny and narrow workgroups, nontemporal A loads
#define NT_STREAM_VARIANT(BM, BN, BK, WM, WN, VEC, FAIR, NAME)                                    \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC, false, true>::NT, VEC,       \
     MfmaCfg<BM, BN, BK, WM, WN, VEC, false, true>::LDS_BYTES,                                      \
     &launch_mfma<BM, BN, BK, WM, WN, VEC, 0, false, false, true, FAIR, true>, 0, 0, false, true}
#define DIRECT_TRANS(D, BK, VEC, TA, TB, NAME) \
    {NAME, kMfma, 32, 32, BK, 32, 32, 64, VEC, 0, &launch_mfma_direct<VEC, D, TA, TB>, 0, 0, TA, TB}
// the variants of one transposition (TAG: "nt", "tn" or "tt"; first letter op(A), second op(B));
// the 128x128 ones with drain ordering (schedule 4); the LDS-free ones (BK = 16 D)
#define TRANS_SET(TA, TB, TAG)                                                                     \
    TRANS_VARIANT(128, 128, 16, 64, 64, true, false, TA, TB, 4, MFMA_NAME(128, 128, 16, 64, 64) "_" TAG "_vec"),     \
        TRANS_VARIANT(128, 128, 16, 64, 64, false, false, TA, TB, 4, MFMA_NAME(128, 128, 16, 64, 64) "_" TAG "_scalar"), \
        TRANS_VARIANT(64, 64, 32, 32, 32, true, false, TA, TB, 0, MFMA_NAME(64, 64, 32, 32, 32) "_" TAG "_vec"),         \
        TRANS_VARIANT(64, 64, 32, 32, 32, false, false, TA, TB, 0, MFMA_NAME(64, 64, 32, 32, 32) "_" TAG "_scalar"),     \
        TRANS_VARIANT(128, 128, 16, 64, 64, true, true, TA, TB, 4, MFMA_NAME(128, 128, 16, 64, 64) "_" TAG "_wide_vec"), \
        TRANS_VARIANT(128, 128, 16, 64, 64, false, true, TA, TB, 4, MFMA_NAME(128, 128, 16, 64, 64) "_" TAG "_wide_scalar"), \
        DIRECT_TRANS(8, 128, true, TA, TB, "mfma32r_32x32x128_w32x32_g8_" TAG "_vec"),                                 \
        DIRECT_TRANS(6, 96, false, TA, TB, "mfma32r_32x32x96_w32x32_g6_" TAG "_scalar")
#define FAIR_VARIANT(BM, BN, BK, WM, WN, OCC, VEC, P, NAME)                                    \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES,                                              \
     &launch_mfma<BM, BN, BK, WM, WN, VEC, OCC, false, false, false, P>, 0}
#define DEEP_VARIANT(BM, BN, BK, WM, WN, VEC, NAME)                                             \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES, &launch_mfma_deep<BM, BN, BK, WM, WN, VEC, 0>, 0}
#define PIPE_FAIR_VARIANT(BM, BN, BK, WM, WN, OCC, VEC, P, NAME)                                 \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES, &launch_mfma_pipe<BM, BN, BK, WM, WN, VEC, OCC, false, P>, 0}
#define DEEP_FAIR_VARIANT(BM, BN, BK, WM, WN, VEC, P, NAME)                                      \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES, &launch_mfma_deep<BM, BN, BK, WM, WN, VEC, 0, P>, 0}
// nontemporal loads of A (the skinny class: with one tile column, no two workgroups read the
// same rows of A)
#define NTA_FAIR_VARIANT(BM, BN, BK, WM, WN, VEC, P, NAME)                                      \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES,                                              \
     &launch_mfma<BM, BN, BK, WM, WN, VEC, 0, false, false, false, P, true>, 0}
#define NTA_DEEP_VARIANT(BM, BN, BK, WM, WN, VEC, P, NAME)                                      \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES, &launch_mfma_deep<BM, BN, BK, WM, WN, VEC, 0, P, true>, 0}
#define CP_DEEP_VARIANT(BM, BN, BK, WM, WN, VEC, P, NAME)                                       \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT, VEC,                  \
     MfmaCfg<BM, BN, BK, WM, WN, VEC>::LDS_BYTES, &launch_mfma_deep<BM, BN, BK, WM, WN, VEC, 0, P, false, true>, 0}
// B in k-quads, staged n-major ("_bq"; 32-bit loads only)
#define BQ_VARIANT(BM, BN, BK, WM, WN, OCC, FAIR, NTA, NAME)                                       \
    {NAME, kMfma, BM, BN, BK, WM, WN, MfmaCfg<BM, BN, BK, WM, WN, false>::NT, 0,                    \
     MfmaCfg<BM, BN, BK, WM, WN, false, false, false, true>::LDS_BYTES,                            \
     &launch_mfma<BM, BN, BK, WM, WN, false, OCC, false, false, false, FAIR, NTA, true>, 0, 0, 0, 0, 1}
#define DEEP_NAME(BM, BN, BK, WM, WN) "mfma32d_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN
// operands loaded straight into a ring of STAGES LDS buffers ("mfma32l_"): 128-bit loads ("_vec")
// or 32-bit loads ("_scalar")
#define DL_ROW(BM, BN, BK, WM, WN, STAGES, W, OCC, FAIR, CPRE, SP, NAME)                                 \
    {NAME, kMfma, BM, BN, BK, WM, WN, DlCfg<BM, BN, BK, WM, WN, STAGES, W>::NT, W == 16,                  \
     DlCfg<BM, BN, BK, WM, WN, STAGES, W>::LDS_BYTES,                                                     \
     &launch_mfma_dl<BM, BN, BK, WM, WN, STAGES, W, OCC, FAIR, CPRE, SP>, 0, 0, 0, 0, 0, STAGES}
#define DL_NAME(BM, BN, BK, WM, WN, STAGES) "mfma32l_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #STAGES
#define DL_VARIANT(BM, BN, BK, WM, WN, STAGES, OCC, FAIR, CPRE, SUFFIX) \
    DL_ROW(BM, BN, BK, WM, WN, STAGES, 16, OCC, FAIR, CPRE, false, DL_NAME(BM, BN, BK, WM, WN, STAGES) SUFFIX "_vec")
#define DL_SCALAR(BM, BN, BK, WM, WN, STAGES, OCC, FAIR, CPRE, SUFFIX) \
    DL_ROW(BM, BN, BK, WM, WN, STAGES, 4, OCC, FAIR, CPRE, false, DL_NAME(BM, BN, BK, WM, WN, STAGES) SUFFIX "_scalar")
// 16x16x4 MFMA blocks ("mfma16l_"): the same kernel with smaller wave tiles, so that a one-tile
// workgroup holds 8 or 16 waves
#define DL16_ROW(BM, BN, BK, WM, WN, STAGES, W, OCC, CPRE, SP, NAME)                                      \
    {NAME, kMfma, BM, BN, BK, WM, WN, DlCfg<BM, BN, BK, WM, WN, STAGES, W, 16>::NT, W == 16,              \
     DlCfg<BM, BN, BK, WM, WN, STAGES, W, 16>::LDS_BYTES,                                                 \
     &launch_mfma_dl<BM, BN, BK, WM, WN, STAGES, W, OCC, 0, CPRE, SP, 16>, 0, 0, 0, 0, 0, STAGES, 0, 16}
#define DL16_NAME(BM, BN, BK, WM, WN, STAGES) "mfma16l_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_s" #STAGES
// A loaded without allocating in the caches ("_nta": the streamed panels of the skinny and narrow shapes)
#define DLNT_ROW(BM, BN, BK, WM, WN, STAGES, W, FAIR, SP, NAME)                                          \
    {NAME, kMfma, BM, BN, BK, WM, WN, DlCfg<BM, BN, BK, WM, WN, STAGES, W>::NT, W == 16,                  \
     DlCfg<BM, BN, BK, WM, WN, STAGES, W>::LDS_BYTES,                                                     \
     &launch_mfma_dl<BM, BN, BK, WM, WN, STAGES, W, 0, FAIR, false, SP, 32, 0, true>, 0, 0, 0, 0, 0, STAGES}
// the barrier that opens each slab EB fragment groups early ("_ebN"; 32x32 or 16x16 blocks)
#define DLEB_ROW(BM, BN, BK, WM, WN, STAGES, W, CPRE, SP, MB, EB, NAME)                                   \
    {NAME, kMfma, BM, BN, BK, WM, WN, DlCfg<BM, BN, BK, WM, WN, STAGES, W, MB>::NT, W == 16,              \
     DlCfg<BM, BN, BK, WM, WN, STAGES, W, MB>::LDS_BYTES,                                                 \
     &launch_mfma_dl<BM, BN, BK, WM, WN, STAGES, W, 0, 0, CPRE, SP, MB, EB>, 0, 0, 0, 0, 0, STAGES, 0, MB}
#define DL16_VARIANT(BM, BN, BK, WM, WN, STAGES, OCC, CPRE, SP, SUFFIX) \
    DL16_ROW(BM, BN, BK, WM, WN, STAGES, 16, OCC, CPRE, SP, DL16_NAME(BM, BN, BK, WM, WN, STAGES) SUFFIX "_vec")
#define DL16_SCALAR(BM, BN, BK, WM, WN, STAGES, OCC, CPRE, SP, SUFFIX) \
    DL16_ROW(BM, BN, BK, WM, WN, STAGES, 4, OCC, CPRE, SP, DL16_NAME(BM, BN, BK, WM, WN, STAGES) SUFFIX "_scalar")
// persistent grid-stride form ("_ps"): one workgroup per resident slot, tiles in a loop
#define DLP_ROW(BM, BN, BK, WM, WN, STAGES, W, OCC, SP, NAME)                                            \
    {NAME, kMfma, BM, BN, BK, WM, WN, DlCfg<BM, BN, BK, WM, WN, STAGES, W>::NT, W == 16,                  \
     DlCfg<BM, BN, BK, WM, WN, STAGES, W>::LDS_BYTES, &launch_mfma_dlp<BM, BN, BK, WM, WN, STAGES, W, OCC, SP>, \
     0, 0, 0, 0, 0, STAGES, 1}
// the same with the next slab's requests spread over the slab's 8-deep groups ("_sp")
#define DL_SP_VARIANT(BM, BN, BK, WM, WN, STAGES, OCC, FAIR, CPRE, SUFFIX) \
    DL_ROW(BM, BN, BK, WM, WN, STAGES, 16, OCC, FAIR, CPRE, true, DL_NAME(BM, BN, BK, WM, WN, STAGES) SUFFIX "_sp_vec")
#define DL_SP_SCALAR(BM, BN, BK, WM, WN, STAGES, OCC, FAIR, CPRE, SUFFIX) \
    DL_ROW(BM, BN, BK, WM, WN, STAGES, 4, OCC, FAIR, CPRE, true, DL_NAME(BM, BN, BK, WM, WN, STAGES) SUFFIX "_sp_scalar")
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
    // drain ordering in the last round (schedules 3 and 4)
    FAIR_VARIANT(128, 128, 16, 64, 64, 0, true, 3, MFMA_NAME(128, 128, 16, 64, 64) "_d3_vec"),
    FAIR_VARIANT(128, 128, 16, 64, 64, 0, true, 4, MFMA_NAME(128, 128, 16, 64, 64) "_d4_vec"),
    FAIR_VARIANT(128, 128, 16, 64, 64, 4, true, 3, MFMA_NAME(128, 128, 16, 64, 64) "_o4_d3_vec"),
    FAIR_VARIANT(128, 128, 16, 64, 64, 4, false, 3, MFMA_NAME(128, 128, 16, 64, 64) "_o4_d3_scalar"),
    FAIR_VARIANT(128, 128, 16, 64, 64, 4, false, 4, MFMA_NAME(128, 128, 16, 64, 64) "_o4_d4_scalar"),
    FAIR_VARIANT(64, 64, 16, 32, 32, 0, true, 3, MFMA_NAME(64, 64, 16, 32, 32) "_d3_vec"),
    FAIR_VARIANT(64, 64, 16, 32, 32, 0, false, 3, MFMA_NAME(64, 64, 16, 32, 32) "_d3_scalar"),
    FAIR_VARIANT(64, 64, 32, 32, 32, 0, true, 3, MFMA_NAME(64, 64, 32, 32, 32) "_d3_vec"),
    FAIR_VARIANT(64, 64, 32, 32, 32, 0, false, 3, MFMA_NAME(64, 64, 32, 32, 32) "_d3_scalar"),
    PIPE_FAIR_VARIANT(64, 64, 16, 32, 32, 4, true, 3, PIPE_NAME(64, 64, 16, 32, 32, 4) "_d3_vec"),
    PIPE_FAIR_VARIANT(64, 64, 16, 32, 32, 4, false, 3, PIPE_NAME(64, 64, 16, 32, 32, 4) "_d3_scalar"),
    DEEP_FAIR_VARIANT(64, 64, 32, 32, 32, true, 3, DEEP_NAME(64, 64, 32, 32, 32) "_d3_vec"),
    DEEP_FAIR_VARIANT(64, 64, 32, 32, 32, false, 3, DEEP_NAME(64, 64, 32, 32, 32) "_d3_scalar"),
    // deep prefetch (one wave per SIMD)
    BOTH_DEEP(64, 64, 32, 32, 32),
    BOTH_DEEP(64, 64, 64, 32, 32),
    // nontemporal A (skinny class)
    NTA_FAIR_VARIANT(64, 64, 32, 32, 32, true, 3, MFMA_NAME(64, 64, 32, 32, 32) "_d3_nta_vec"),
    NTA_FAIR_VARIANT(64, 64, 32, 32, 32, false, 3, MFMA_NAME(64, 64, 32, 32, 32) "_d3_nta_scalar"),
    NTA_DEEP_VARIANT(64, 64, 32, 32, 32, true, 0, DEEP_NAME(64, 64, 32, 32, 32) "_nta_vec"),
    NTA_DEEP_VARIANT(64, 64, 32, 32, 32, false, 0, DEEP_NAME(64, 64, 32, 32, 32) "_nta_scalar"),
    NTA_DEEP_VARIANT(64, 64, 32, 32, 32, true, 3, DEEP_NAME(64, 64, 32, 32, 32) "_d3_nta_vec"),
    NTA_DEEP_VARIANT(64, 64, 32, 32, 32, false, 3, DEEP_NAME(64, 64, 32, 32, 32) "_d3_nta_scalar"),
    NTA_FAIR_VARIANT(128, 64, 32, 64, 64, true, 0, MFMA_NAME(128, 64, 32, 64, 64) "_nta_vec"),
    // transposed operands (sgemm_op): op(A) x op(B) = N x T, T x N, T x T
    TRANS_SET(false, true, "nt"),
    TRANS_SET(true, false, "tn"),
    TRANS_SET(true, true, "tt"),
    // LDS-free: one wave per 32x32 tile, operands loaded straight into registers D groups ahead
    // (BK = 16 D: the K span of the loads in flight, which bounds the 32-bit per-lane offsets)
    {"mfma32r_32x32x128_w32x32_g8_vec", kMfma, 32, 32, 128, 32, 32, 64, 1, 0, &launch_mfma_direct<true, 8>, 0},
    {"mfma32r_32x32x128_w32x32_g8_scalar", kMfma, 32, 32, 128, 32, 32, 64, 0, 0, &launch_mfma_direct<false, 8>, 0},
    {"mfma32r_32x32x96_w32x32_g6_vec", kMfma, 32, 32, 96, 32, 32, 64, 1, 0, &launch_mfma_direct<true, 6>, 0},
    {"mfma32r_32x32x96_w32x32_g6_scalar", kMfma, 32, 32, 96, 32, 32, 64, 0, 0, &launch_mfma_direct<false, 6>, 0},
    // skinny streams: four 64x32 wave tiles per 128x64 workgroup (the B panel stays in L2)
    NTA_FAIR_VARIANT(128, 64, 32, 64, 32, true, 3, MFMA_NAME(128, 64, 32, 64, 32) "_d3_nta_vec"),
    // N <= 32 streams: 32-wide workgroups (64-wide ones would compute half padding)
    NTA_FAIR_VARIANT(128, 32, 32, 32, 32, true, 3, MFMA_NAME(128, 32, 32, 32, 32) "_d3_nta_vec"),
    NTA_FAIR_VARIANT(128, 32, 32, 32, 32, false, 3, MFMA_NAME(128, 32, 32, 32, 32) "_d3_nta_scalar"),
    NTA_FAIR_VARIANT(256, 32, 32, 64, 32, true, 0, MFMA_NAME(256, 32, 32, 64, 32) "_nta_vec"),
    NTA_DEEP_VARIANT(128, 64, 32, 64, 32, true, 3, DEEP_NAME(128, 64, 32, 64, 32) "_d3_nta_vec"),
    NTA_DEEP_VARIANT(128, 32, 32, 32, 32, true, 3, DEEP_NAME(128, 32, 32, 32, 32) "_d3_nta_vec"),
    NTA_DEEP_VARIANT(128, 32, 32, 32, 32, false, 3, DEEP_NAME(128, 32, 32, 32, 32) "_d3_nta_scalar"),
    // C for the beta term read at the start of the tile ("_cp"): one-round grids
    CP_DEEP_VARIANT(64, 64, 32, 32, 32, true, 0, DEEP_NAME(64, 64, 32, 32, 32) "_cp_vec"),
    CP_DEEP_VARIANT(64, 64, 32, 32, 32, false, 0, DEEP_NAME(64, 64, 32, 32, 32) "_cp_scalar"),
    CP_DEEP_VARIANT(64, 64, 32, 32, 32, true, 3, DEEP_NAME(64, 64, 32, 32, 32) "_d3_cp_vec"),
    CP_DEEP_VARIANT(64, 64, 32, 32, 32, false, 3, DEEP_NAME(64, 64, 32, 32, 32) "_d3_cp_scalar"),
    {"mfma32r_32x32x128_w32x32_g8_cp_vec", kMfma, 32, 32, 128, 32, 32, 64, 1, 0,
     &launch_mfma_direct<true, 8, false, false, true>, 0},
    {"mfma32r_32x32x96_w32x32_g6_cp_scalar", kMfma, 32, 32, 96, 32, 32, 64, 0, 0,
     &launch_mfma_direct<false, 6, false, false, true>, 0},
    {"mfma32r_32x32x96_w32x32_g6_cp_vec", kMfma, 32, 32, 96, 32, 32, 64, 1, 0,
     &launch_mfma_direct<true, 6, false, false, true>, 0},
    // two accumulator sets per block ("_a2"): independent consecutive MFMAs at one wave per SIMD
    {DEEP_NAME(64, 64, 32, 32, 32) "_cp_a2_vec", kMfma, 64, 64, 32, 32, 32, MfmaCfg<64, 64, 32, 32, 32, true>::NT, 1,
     MfmaCfg<64, 64, 32, 32, 32, true>::LDS_BYTES, &launch_mfma_deep<64, 64, 32, 32, 32, true, 0, 0, false, true, true>, 0},
    {DEEP_NAME(64, 64, 32, 32, 32) "_d3_a2_scalar", kMfma, 64, 64, 32, 32, 32, MfmaCfg<64, 64, 32, 32, 32, false>::NT, 0,
     MfmaCfg<64, 64, 32, 32, 32, false>::LDS_BYTES, &launch_mfma_deep<64, 64, 32, 32, 32, false, 0, 3, false, false, true>, 0},
    NT_STREAM_VARIANT(128, 64, 32, 64, 32, true, 3, MFMA_NAME(128, 64, 32, 64, 32) "_d3_nta_nt_vec"),
    NT_STREAM_VARIANT(128, 64, 32, 64, 32, false, 3, MFMA_NAME(128, 64, 32, 64, 32) "_d3_nta_nt_scalar"),
    NT_STREAM_VARIANT(128, 32, 32, 32, 32, true, 3, MFMA_NAME(128, 32, 32, 32, 32) "_d3_nta_nt_vec"),
    NT_STREAM_VARIANT(128, 32, 32, 32, 32, false, 3, MFMA_NAME(128, 32, 32, 32, 32) "_d3_nta_nt_scalar"),
    // unaligned operands with B in k-quads (one 128-bit LDS store and one 128-bit fragment read per
    // four k of a column, instead of four 32-bit ones each)
    BQ_VARIANT(64, 64, 16, 32, 32, 0, 0, false, MFMA_NAME(64, 64, 16, 32, 32) "_bq_scalar"),
    BQ_VARIANT(64, 64, 32, 32, 32, 0, 3, false, MFMA_NAME(64, 64, 32, 32, 32) "_d3_bq_scalar"),
    BQ_VARIANT(128, 128, 16, 64, 64, 4, 4, false, MFMA_NAME(128, 128, 16, 64, 64) "_o4_d4_bq_scalar"),
    // direct global -> LDS loads into a ring of two or three LDS stages
    DL_VARIANT(64, 64, 32, 32, 32, 3, 0, 0, true, "_cp"),
    DL_VARIANT(64, 64, 32, 32, 32, 3, 0, 0, false, ""),
    DL_VARIANT(64, 64, 32, 32, 32, 2, 0, 0, true, "_cp"),
    DL_VARIANT(64, 64, 32, 32, 32, 3, 0, 3, false, "_d3"),
    DL_VARIANT(128, 128, 16, 64, 64, 3, 0, 4, false, "_d4"),
    DL_VARIANT(128, 128, 16, 64, 64, 3, 0, 3, false, "_d3"),
    DL_VARIANT(128, 128, 16, 64, 64, 2, 4, 4, false, "_o4_d4"),
    DL_VARIANT(128, 64, 32, 64, 32, 3, 0, 3, false, "_d3"),
    DL_VARIANT(64, 64, 64, 32, 32, 3, 0, 0, true, "_cp"),
    DL_VARIANT(64, 64, 64, 32, 32, 2, 0, 0, true, "_cp"),
    DL_VARIANT(64, 64, 32, 32, 32, 4, 0, 0, true, "_cp"),
    DL_VARIANT(128, 128, 16, 64, 64, 4, 0, 3, false, "_d3"),
    // 32-bit direct loads (unaligned operands)
    DL_SCALAR(64, 64, 16, 32, 32, 3, 0, 0, false, ""),
    DL_SCALAR(64, 64, 32, 32, 32, 3, 0, 0, true, "_cp"),
    DL_SCALAR(64, 64, 32, 32, 32, 3, 0, 3, false, "_d3"),
    DL_SCALAR(64, 64, 16, 32, 32, 2, 0, 0, false, ""),
    DL_SCALAR(128, 128, 16, 64, 64, 3, 0, 4, false, "_d4"),
    DL_SP_VARIANT(64, 64, 32, 32, 32, 3, 0, 0, true, "_cp"),
    DL_SP_VARIANT(64, 64, 32, 32, 32, 3, 0, 0, false, ""),
    DL_SP_VARIANT(64, 64, 32, 32, 32, 4, 0, 0, true, "_cp"),
    DL_SP_VARIANT(64, 64, 32, 32, 32, 3, 0, 3, false, "_d3"),
    DL_SP_VARIANT(128, 128, 16, 64, 64, 4, 0, 3, false, "_d3"),
    DL_SP_VARIANT(128, 64, 32, 64, 32, 3, 0, 3, false, "_d3"),
    DL_SP_SCALAR(64, 64, 16, 32, 32, 3, 0, 0, false, ""),
    DL_SP_SCALAR(64, 64, 32, 32, 32, 3, 0, 3, false, "_d3"),
    DLP_ROW(64, 64, 32, 32, 32, 3, 16, 0, true, DL_NAME(64, 64, 32, 32, 32, 3) "_ps_sp_vec"),
    DLP_ROW(128, 128, 16, 64, 64, 4, 16, 0, true, DL_NAME(128, 128, 16, 64, 64, 4) "_ps_sp_vec"),
    DLP_ROW(128, 128, 16, 64, 64, 4, 16, 0, false, DL_NAME(128, 128, 16, 64, 64, 4) "_ps_vec"),
    DLP_ROW(128, 64, 32, 64, 32, 3, 16, 0, true, DL_NAME(128, 64, 32, 64, 32, 3) "_ps_sp_vec"),
    DLP_ROW(64, 64, 16, 32, 32, 3, 4, 0, true, DL_NAME(64, 64, 16, 32, 32, 3) "_ps_sp_scalar"),
    DLP_ROW(64, 64, 32, 32, 32, 3, 4, 0, true, DL_NAME(64, 64, 32, 32, 32, 3) "_ps_sp_scalar"),
    // 16x16x4 blocks: 64x64 tiles of 8 waves (two per SIMD) or 16 waves, and 128-wide tiles of 8 or
    // 16 waves of 32x32
    DL16_VARIANT(64, 64, 32, 32, 16, 3, 0, true, false, "_cp"),
    DL16_VARIANT(64, 64, 32, 16, 32, 3, 0, true, false, "_cp"),
    DL16_VARIANT(64, 64, 32, 32, 16, 3, 0, true, true, "_cp_sp"),
    DL16_VARIANT(64, 64, 32, 32, 16, 2, 0, true, false, "_cp"),
    DL16_VARIANT(64, 64, 64, 16, 16, 3, 0, true, false, "_cp"),
    DL16_VARIANT(64, 64, 32, 32, 32, 3, 0, true, false, "_cp"),
    DL16_VARIANT(128, 64, 32, 32, 32, 3, 0, false, false, ""),
    DL16_VARIANT(128, 128, 32, 32, 32, 3, 0, false, false, ""),
    DL16_SCALAR(64, 64, 32, 32, 16, 3, 0, false, false, ""),
    DL16_SCALAR(64, 64, 32, 32, 16, 3, 0, false, true, "_sp"),
    // 32x64 tiles of four 32x16 waves: a 1024^2 grid has 512 of them, two workgroups per CU, so a
    // SIMD's two waves belong to different workgroups and wait at different barriers
    DL16_VARIANT(32, 64, 32, 32, 16, 3, 0, true, true, "_cp_sp"),
    DL16_VARIANT(32, 64, 32, 32, 16, 3, 0, true, false, "_cp"),
    DL16_VARIANT(32, 64, 32, 16, 32, 3, 0, true, false, "_cp"),
    DL16_VARIANT(32, 64, 32, 32, 16, 4, 0, true, false, "_cp"),
    DL16_SCALAR(32, 64, 32, 32, 16, 3, 0, false, false, ""),
    // early barrier: at one wave per SIMD the K loop runs 2-4 % faster, a launch at most ~1 %
    DLEB_ROW(64, 64, 32, 32, 32, 3, 16, true, true, 32, 2, DL_NAME(64, 64, 32, 32, 32, 3) "_cp_sp_eb2_vec"),
    DLEB_ROW(64, 64, 32, 32, 32, 3, 16, true, true, 32, 3, DL_NAME(64, 64, 32, 32, 32, 3) "_cp_sp_eb3_vec"),
    DLEB_ROW(64, 64, 16, 32, 32, 3, 4, false, true, 32, 1, DL_NAME(64, 64, 16, 32, 32, 3) "_sp_eb1_scalar"),
    DLEB_ROW(64, 64, 32, 32, 16, 3, 16, true, true, 16, 1, DL16_NAME(64, 64, 32, 32, 16, 3) "_cp_sp_eb1_vec"),
    DLEB_ROW(32, 64, 32, 32, 16, 3, 16, true, true, 16, 1, DL16_NAME(32, 64, 32, 32, 16, 3) "_cp_sp_eb1_vec"),
    // 32x32 tiles of one wave: a workgroup's barrier waits for its own wave only (B rows of 32
    // floats, row-permuted); slower than the 64x64 and 32x64 tiles at 256^3 and 1024^3
    DL_ROW(32, 32, 32, 32, 32, 3, 16, 0, 0, true, true, DL_NAME(32, 32, 32, 32, 32, 3) "_cp_sp_vec"),
    // the narrow stream's 128x32 tiles, nontemporal A: within a few per cent of the dispatched
    // kernels, never ahead
    DLNT_ROW(128, 32, 32, 32, 32, 3, 16, 3, false, DL_NAME(128, 32, 32, 32, 32, 3) "_d3_nta_vec"),
    DLNT_ROW(128, 32, 32, 32, 32, 3, 4, 3, false, DL_NAME(128, 32, 32, 32, 32, 3) "_d3_nta_scalar"),
    // nontemporal A: the skinny stream
    DLNT_ROW(128, 64, 32, 64, 32, 3, 16, 3, false, DL_NAME(128, 64, 32, 64, 32, 3) "_d3_nta_vec"),
    DLNT_ROW(128, 64, 32, 64, 32, 3, 16, 3, true, DL_NAME(128, 64, 32, 64, 32, 3) "_d3_sp_nta_vec"),
    DLNT_ROW(128, 64, 32, 64, 32, 3, 4, 3, false, DL_NAME(128, 64, 32, 64, 32, 3) "_d3_nta_scalar"),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);
