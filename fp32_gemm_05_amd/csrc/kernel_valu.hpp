// kernel_valu.hpp -- the vector-FMA register-microtile kernel.
#pragma once

#include "kernel_common.hpp"

namespace libsgemm {

// ---------------------------------------------------------------------------------
// VALU kernel: TM x TN register microtile per lane, A stored k-major in LDS.
// A lane's TM rows are TM/4 groups of 4 consecutive rows spaced BM/(TM/4)
// apart (likewise for columns), so the 128-bit LDS reads of a wave touch
// consecutive addresses (B) or broadcast (A).
// ---------------------------------------------------------------------------------
template <int BM, int BN, int BK, int TM, int TN, bool VEC>
struct ValuCfg {
    static constexpr int TX = BN / TN, TY = BM / TM, NT = TX * TY;
    static constexpr int GM = TM / 4, GN = TN / 4;
    static constexpr int SM = BM / GM, SN = BN / GN;
    static constexpr int PA = 4, PB = 4;
    static constexpr int A_PITCH = BM + PA, B_PITCH = BN + PB;
    static constexpr int A_STAGE = BK * A_PITCH, B_STAGE = BK * B_PITCH;
    static constexpr int LDS_BYTES = 2 * (A_STAGE + B_STAGE) * 4;
    static_assert(TM % 4 == 0 && TN % 4 == 0, "microtile in groups of 4");
    static_assert(BM % TM == 0 && BN % TN == 0, "tiling");
};

template <int BM, int BN, int BK, int TM, int TN, bool VEC, bool WIDE>
__global__ void __launch_bounds__((ValuCfg<BM, BN, BK, TM, TN, VEC>::NT))
sgemm_valu_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    using Cfg = ValuCfg<BM, BN, BK, TM, TN, VEC>;
    constexpr int NT = Cfg::NT, GM = Cfg::GM, GN = Cfg::GN, SM = Cfg::SM, SN = Cfg::SN;
    constexpr int AP = Cfg::A_PITCH, BP = Cfg::B_PITCH;
    __shared__ __attribute__((aligned(16))) float lds_a[2 * Cfg::A_STAGE];
    __shared__ __attribute__((aligned(16))) float lds_b[2 * Cfg::B_STAGE];

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int tx = tid % Cfg::TX, ty = tid / Cfg::TX;

    const int K = g.K;
    PanelLoader<BM, BK, NT, VEC, false, WIDE> la;
    PanelLoader<BK, BN, NT, VEC, true, WIDE> lb;
    la.init(tid, g.A, g.lda, m0, 0, g.M, K, BK);
    lb.init(tid, g.B, g.ldb, 0, n0, K, g.N, BK);

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

    const int nslab = (K + BK - 1) / BK;
    const int nfull = K / BK;
    la.fetch_slab(0, BK, K);
    lb.fetch_slab(0, BK, K);
    la.template store_transposed<AP>(lds_a);
    lb.template store<BP>(lds_b);
    __syncthreads();

    auto slab = [&](int s, auto prefetch) {
        constexpr int PREFETCH = decltype(prefetch)::value;
        const int cur = s & 1;
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
        for (int k = 0; k < BK; ++k) {
            float a[TM], b[TN];
#pragma unroll
            for (int gi = 0; gi < GM; ++gi) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(sa + k * AP + gi * SM + ty * 4);
                a[gi * 4 + 0] = v.x; a[gi * 4 + 1] = v.y; a[gi * 4 + 2] = v.z; a[gi * 4 + 3] = v.w;
            }
#pragma unroll
            for (int gj = 0; gj < GN; ++gj) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(sb + k * BP + gj * SN + tx * 4);
                b[gj * 4 + 0] = v.x; b[gj * 4 + 1] = v.y; b[gj * 4 + 2] = v.z; b[gj * 4 + 3] = v.w;
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        if (PREFETCH != 0) {
            la.template store_transposed<AP>(lds_a + (cur ^ 1) * Cfg::A_STAGE);
            lb.template store<BP>(lds_b + (cur ^ 1) * Cfg::B_STAGE);
        }
        __syncthreads();
    };
    int s = 0;
    for (; s + 1 < nfull; ++s) slab(s, std::integral_constant<int, 1>{});
    for (; s + 1 < nslab; ++s) slab(s, std::integral_constant<int, 2>{});
    slab(s, std::integral_constant<int, 0>{});

    const float alpha = g.alpha, beta = g.beta;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = m0 + (i / 4) * SM + ty * 4 + (i % 4);
        if (row >= g.M) continue;
        float* prow = g.C + (long)row * g.ldc;
#pragma unroll
        for (int gj = 0; gj < GN; ++gj) {
            const int col = n0 + gj * SN + tx * 4;
            if (VEC) {
                // N % 4 == 0: a 4-column group is entirely inside or outside.
                if (col < g.N) {
                    f32x4* pc = reinterpret_cast<f32x4*>(prow + col);
                    f32x4 v = {alpha * acc[i][gj * 4 + 0], alpha * acc[i][gj * 4 + 1],
                               alpha * acc[i][gj * 4 + 2], alpha * acc[i][gj * 4 + 3]};
                    if (beta != 0.f) v += beta * *pc;
                    *pc = v;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (col + e < g.N) {
                        float v = alpha * acc[i][gj * 4 + e];
                        if (beta != 0.f) v += beta * prow[col + e];
                        prow[col + e] = v;
                    }
                }
            }
        }
    }
}

}  // namespace libsgemm
