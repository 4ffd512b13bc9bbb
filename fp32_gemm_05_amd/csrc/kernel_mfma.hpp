// kernel_mfma.hpp -- the plain MFMA kernel: two LDS stages, register prefetch of the next slab (every tile shape, transposed operands, drain ordering).
#pragma once

#include "kernel_common.hpp"

namespace libsgemm {

template <int BM, int BN, int BK, int WM, int WN, bool VEC, int OCC, bool WIDE, bool TA = false, bool TB = false,
          int FAIR = 0, bool NTA = false, bool BQ = false>
__global__ void __launch_bounds__((MfmaCfg<BM, BN, BK, WM, WN, VEC, TA, TB, BQ>::NT))
__attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1, 8)))
sgemm_mfma_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    SGEMM_PHASE_STAMP(0);
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN, VEC, TA, TB, BQ>;
    constexpr int NT = Cfg::NT, FM = Cfg::FM, FN = Cfg::FN;
    constexpr int AP = Cfg::A_PITCH, BP = Cfg::B_PITCH;
    __shared__ __attribute__((aligned(16))) float lds_a[2 * Cfg::A_STAGE];
    __shared__ __attribute__((aligned(16))) float lds_b[2 * Cfg::B_STAGE];

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / Cfg::WAVES_N) * WM;
    const int wn0 = (wave % Cfg::WAVES_N) * WN;
    const int li = lane & 31, lh = lane >> 5;

    const int K = g.K;
    // A slab: BM rows x BK columns of A, or (TA) BK rows x BM columns of the stored A^T.
    // B slab: BK rows x BN columns of B, or (TB) BN rows x BK columns of the stored B^T.
    using LoaderA = typename std::conditional<TA, PanelLoader<BK, BM, NT, VEC, true, WIDE, 1, NTA>,
                                              PanelLoader<BM, BK, NT, VEC, false, WIDE, 1, NTA>>::type;
    using LoaderB = typename std::conditional<
        TB, PanelLoader<BN, BK, NT, VEC, false, WIDE>,
        typename std::conditional<BQ, KQuadLoader<BK, BN, NT, WIDE>, PanelLoader<BK, BN, NT, VEC, true, WIDE>>::type>::type;
    LoaderA la;
    LoaderB lb;
    if (TA)
        la.init(tid, g.A, g.lda, 0, m0, K, g.M, BK);
    else
        la.init(tid, g.A, g.lda, m0, 0, g.M, K, BK);
    if (TB)
        lb.init(tid, g.B, g.ldb, n0, 0, g.N, K, BK);
    else
        lb.init(tid, g.B, g.ldb, 0, n0, K, g.N, BK);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nslab = (K + BK - 1) / BK;
    const int nfull = K / BK;  // slabs with no element past K

    la.fetch_slab(0, BK, K);
    lb.fetch_slab(0, BK, K);
    la.template store<AP>(lds_a);
    lb.template store<BP>(lds_b);
    __syncthreads();

    // One slab: prefetch slab s+1 (PREFETCH 1: a full slab, 2: the partial last slab,
    // 0: none), multiply slab s out of LDS, store the prefetched slab to the other stage.
    // STAGE is s & 1 when known at compile time (the unrolled main loop), -1 otherwise.
    auto slab = [&](int s, auto prefetch, auto stage) {
        constexpr int PREFETCH = decltype(prefetch)::value;
        constexpr int STAGE = decltype(stage)::value;
        const int cur = STAGE >= 0 ? STAGE : (s & 1);
        if (PREFETCH != 0) {
            la.advance();
            lb.advance();
            la.template fetch<PREFETCH == 2>((s + 1) * BK, K);
            lb.template fetch<PREFETCH == 2>((s + 1) * BK, K);
            // keep the prefetch at the top of the slab: its latency hides under the MFMAs below
            __builtin_amdgcn_sched_barrier(0);
        }
        const float* sa = lds_a + cur * Cfg::A_STAGE;
        const float* sb = lds_b + cur * Cfg::B_STAGE;
#pragma unroll
        for (int kk = 0; kk < BK / 8; ++kk) {
            f32x4 a[FM];
            float b[FN][4];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                if (TA) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) a[i][t] = sa[(kk * 8 + lh * 4 + t) * AP + wm0 + i * 32 + li];
                } else {
                    a[i] = *reinterpret_cast<const f32x4*>(sa + (wm0 + i * 32 + li) * AP + kk * 8 + lh * 4);
                }
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if (TB || BQ) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(sb + (wn0 + j * 32 + li) * BP + kk * 8 + lh * 4);
                    b[j][0] = v.x;
                    b[j][1] = v.y;
                    b[j][2] = v.z;
                    b[j][3] = v.w;
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) b[j][t] = sb[(kk * 8 + lh * 4 + t) * BP + wn0 + j * 32 + li];
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = mfma_step<VEC>(a[i][t], b[j][t], acc[i][j]);
        }
        if (PREFETCH != 0) {
            la.template store<AP>(lds_a + (cur ^ 1) * Cfg::A_STAGE);
            lb.template store<BP>(lds_b + (cur ^ 1) * Cfg::B_STAGE);
        }
        __syncthreads();
    };
    using Full = std::integral_constant<int, 1>;
    using Dyn = std::integral_constant<int, -1>;
    DrainPhases drain;
    if (FAIR > 0) drain.init(FAIR, nslab, g.drain_from);
    SGEMM_PHASE_STAMP(1);
    int s = 0;
    // main loop, two slabs per trip so that both LDS stage offsets are constants
    for (; s + 2 < nfull; s += 2) {
        if (FAIR > 0) drain.step(s);
        slab(s, Full{}, std::integral_constant<int, 0>{});
        slab(s + 1, Full{}, std::integral_constant<int, 1>{});
    }
    for (; s + 1 < nfull; ++s) slab(s, Full{}, Dyn{});
    for (; s + 1 < nslab; ++s) slab(s, std::integral_constant<int, 2>{}, Dyn{});
    slab(s, std::integral_constant<int, 0>{}, Dyn{});
    SGEMM_PHASE_STAMP(2);

    mfma_epilogue<FM, FN, VEC>(g.M, g.N, g.alpha, g.beta, g.C, g.ldc, acc, m0 + wm0, n0 + wn0, li, lh);
    SGEMM_PHASE_STAMP(3);
}

}  // namespace libsgemm
