// kernel_splitk.hpp -- the in-workgroup split-K MFMA kernel (k-groups of waves reduce through LDS).
#pragma once

#include "kernel_common.hpp"

namespace libsgemm {

// ---------------------------------------------------------------------------------
// Split-K MFMA kernel for shapes with few output tiles: KS groups of waves share one
// workgroup and one BM x BN tile.  Group g multiplies slabs g, g + KS, g + 2 KS, ...
// (each group with its own two LDS stages, loaders and accumulators, same K loop as
// sgemm_mfma_kernel), so a CU gets KS times the waves and each wave a K loop KS times
// shorter.  At the end groups 1..KS-1 leave their accumulators in LDS and group 0 adds
// them in group order (a fixed order: results are deterministic) and writes C.
// ---------------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN, int KS, bool VEC>
struct SplitKCfg {
    using Base = MfmaCfg<BM, BN, BK, WM, WN, VEC>;
    static constexpr int GT = Base::NT;  // threads per k-group
    static constexpr int NT = GT * KS;
    static constexpr int GROUP_FLOATS = 2 * (Base::A_STAGE + Base::B_STAGE);
    static constexpr int RED_FLOATS = (KS - 1) * BM * BN;
    static constexpr int LDS_FLOATS = KS * GROUP_FLOATS > RED_FLOATS ? KS * GROUP_FLOATS : RED_FLOATS;
    static constexpr int LDS_BYTES = LDS_FLOATS * 4;
    static_assert(KS >= 2 && NT <= 1024, "2..(1024 / group threads) k-groups");
};

template <int BM, int BN, int BK, int WM, int WN, int KS, bool VEC>
__global__ void __launch_bounds__((SplitKCfg<BM, BN, BK, WM, WN, KS, VEC>::NT))
sgemm_mfma_splitk_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    using Base = MfmaCfg<BM, BN, BK, WM, WN, VEC>;
    using Cfg = SplitKCfg<BM, BN, BK, WM, WN, KS, VEC>;
    constexpr int GT = Cfg::GT, FM = Base::FM, FN = Base::FN;
    constexpr int AP = Base::A_PITCH, BP = Base::B_PITCH;
    __shared__ __attribute__((aligned(16))) float lds[Cfg::LDS_FLOATS];

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int grp = tid / GT;           // k-group: whole waves, so wave-uniform
    const int gtid = tid - grp * GT;    // thread index within the group
    const int lane = gtid & 63, wave = gtid >> 6;
    const int wm0 = (wave / Base::WAVES_N) * WM;
    const int wn0 = (wave % Base::WAVES_N) * WN;
    const int li = lane & 31, lh = lane >> 5;
    float* lds_a = lds + grp * Cfg::GROUP_FLOATS;  // [2][A_STAGE] of this group
    float* lds_b = lds_a + 2 * Base::A_STAGE;      // [2][B_STAGE] of this group

    const int K = g.K;
    PanelLoader<BM, BK, GT, VEC, false, false> la;
    PanelLoader<BK, BN, GT, VEC, true, false> lb;
    la.init(gtid, g.A, g.lda, m0, grp * BK, g.M, K, KS * BK);
    lb.init(gtid, g.B, g.ldb, grp * BK, n0, K, g.N, KS * BK);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nslab = (K + BK - 1) / BK;
    const int nfull = K / BK;
    const int niter = (nslab + KS - 1) / KS;  // every group runs this many slab steps

    la.fetch_slab(grp * BK, BK, K);  // a group whose first slab lies past K loads zeros
    lb.fetch_slab(grp * BK, BK, K);
    la.template store<AP>(lds_a);
    lb.template store<BP>(lds_b);
    __syncthreads();

    // Step i: group grp multiplies slab i*KS + grp.  PREFETCH 1: the next step's slabs are
    // full for every group; 2: some are partial or past K (checked loads); 0: no next step.
    auto step = [&](int i, auto prefetch) {
        constexpr int PREFETCH = decltype(prefetch)::value;
        const int cur = i & 1;
        if (PREFETCH != 0) {
            la.advance();
            lb.advance();
            const int kb = ((i + 1) * KS + grp) * BK;
            la.template fetch<PREFETCH == 2>(kb, K);
            lb.template fetch<PREFETCH == 2>(kb, K);
            __builtin_amdgcn_sched_barrier(0);
        }
        const float* sa = lds_a + cur * Base::A_STAGE;
        const float* sb = lds_b + cur * Base::B_STAGE;
#pragma unroll
        for (int kk = 0; kk < BK / 8; ++kk) {
            f32x4 a[FM];
            float b[FN][4];
#pragma unroll
            for (int i2 = 0; i2 < FM; ++i2)
                a[i2] = *reinterpret_cast<const f32x4*>(sa + (wm0 + i2 * 32 + li) * AP + kk * 8 + lh * 4);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int t = 0; t < 4; ++t) b[j][t] = sb[(kk * 8 + lh * 4 + t) * BP + wn0 + j * 32 + li];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i2 = 0; i2 < FM; ++i2)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i2][j] = mfma_step<VEC>(a[i2][t], b[j][t], acc[i2][j]);
        }
        if (PREFETCH != 0) {
            la.template store<AP>(lds_a + (cur ^ 1) * Base::A_STAGE);
            lb.template store<BP>(lds_b + (cur ^ 1) * Base::B_STAGE);
        }
        __syncthreads();
    };
    int i = 0;
    for (; i + 1 < niter && (i + 2) * KS <= nfull; ++i) step(i, std::integral_constant<int, 1>{});
    for (; i + 1 < niter; ++i) step(i, std::integral_constant<int, 2>{});
    step(i, std::integral_constant<int, 0>{});  // ends with a barrier: every LDS stage is free

    // Reduction through LDS: group g >= 1 writes its partial tile, group 0 adds them in order.
    constexpr int WAVE_FLOATS = FM * FN * 16 * 64;
    if (grp > 0) {
        float* red = lds + (grp - 1) * BM * BN + wave * WAVE_FLOATS;
#pragma unroll
        for (int i2 = 0; i2 < FM; ++i2)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4 v = {acc[i2][j][4 * q + 0], acc[i2][j][4 * q + 1], acc[i2][j][4 * q + 2],
                               acc[i2][j][4 * q + 3]};
                    *reinterpret_cast<f32x4*>(red + (((i2 * FN + j) * 4 + q) * 64 + lane) * 4) = v;
                }
    }
    __syncthreads();
    if (grp == 0) {
        for (int g2 = 1; g2 < KS; ++g2) {
            const float* red = lds + (g2 - 1) * BM * BN + wave * WAVE_FLOATS;
#pragma unroll
            for (int i2 = 0; i2 < FM; ++i2)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 v = *reinterpret_cast<const f32x4*>(red + (((i2 * FN + j) * 4 + q) * 64 + lane) * 4);
                        acc[i2][j][4 * q + 0] += v.x;
                        acc[i2][j][4 * q + 1] += v.y;
                        acc[i2][j][4 * q + 2] += v.z;
                        acc[i2][j][4 * q + 3] += v.w;
                    }
        }
        mfma_epilogue<FM, FN, VEC>(g.M, g.N, g.alpha, g.beta, g.C, g.ldc, acc, m0 + wm0, n0 + wn0, li, lh);
    }
}

}  // namespace libsgemm
