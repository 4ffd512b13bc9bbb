// kernel_pipe.hpp -- the MFMA kernel with LDS -> register fragments double-buffered.
#pragma once

#include "kernel_common.hpp"

namespace libsgemm {

// ---------------------------------------------------------------------------------
// Pipelined MFMA kernel: same tiling, operand mapping and LDS layout as
// sgemm_mfma_kernel, with the LDS -> register fragments double-buffered:
// while the MFMAs of one 8-deep group run, the fragments of the next group are
// read; the next slab's first fragments are read right after the slab's barrier,
// under the MFMAs of the current slab's last group.  One barrier per slab:
//   store slab s+1 (registers -> LDS stage (s+1)&1); barrier; fetch slab s+2
//   (global -> registers); read group 0 of slab s+1; MFMAs of slab s's last group.
// Stage (s+1)&1 was last read during slab s-1, whose reads all completed before
// the barrier of iteration s-1 (the barrier waits for outstanding LDS accesses).
// ---------------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN, bool VEC, int OCC, bool WIDE, int FAIR = 0>
__global__ void __launch_bounds__((MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT))
__attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1, 8)))
sgemm_mfma_pipe_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN, VEC>;
    constexpr int NT = Cfg::NT, FM = Cfg::FM, FN = Cfg::FN;
    constexpr int AP = Cfg::A_PITCH, BP = Cfg::B_PITCH;
    constexpr int KK = BK / 8;
    static_assert(KK % 2 == 0, "the fragment double buffer alternates per 8-deep group: BK must be 16 or 32");
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
    PanelLoader<BM, BK, NT, VEC, false, WIDE> la;
    PanelLoader<BK, BN, NT, VEC, true, WIDE> lb;
    la.init(tid, g.A, g.lda, m0, 0, g.M, K, BK);
    lb.init(tid, g.B, g.ldb, 0, n0, K, g.N, BK);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // per-lane offsets of the fragment reads inside one LDS stage
    const int a_off = (wm0 + li) * AP + lh * 4;
    const int b_off = (lh * 4) * BP + wn0 + li;

    auto read_frag = [&](MfmaFrag<FM, FN>& f, const float* sa, const float* sb, int kk) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            f.a[i] = *reinterpret_cast<const f32x4*>(sa + a_off + i * 32 * AP + kk * 8);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) f.b[j][t] = sb[b_off + (kk * 8 + t) * BP + j * 32];
    };
    auto mfma_frag = [&](const MfmaFrag<FM, FN>& f) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = mfma_step<VEC>(f.a[i][t], f.b[j][t], acc[i][j]);
    };

    const int nslab = (K + BK - 1) / BK;
    const int nfull = K / BK;

    la.fetch_slab(0, BK, K);
    lb.fetch_slab(0, BK, K);
    la.template store<AP>(lds_a);
    lb.template store<BP>(lds_b);
    __syncthreads();
    if (nslab > 1) {
        la.advance();
        lb.advance();
        la.fetch_slab(BK, BK, K);
        lb.fetch_slab(BK, BK, K);
    }
    MfmaFrag<FM, FN> F[2];
    read_frag(F[0], lds_a, lds_b, 0);

    // One slab.  MODE 0: s is the last slab; 1: slab s+1 exists and a full slab s+2 is
    // prefetched; 2: the partial slab s+2 is prefetched; 3: slab s+1 exists, no s+2.
    auto slab = [&](int s, auto mode, auto stage) {
        constexpr int MODE = decltype(mode)::value;
        constexpr int STAGE = decltype(stage)::value;  // s & 1 when known at compile time, else -1
        const int cur = STAGE >= 0 ? STAGE : (s & 1);
        const float* sa = lds_a + cur * Cfg::A_STAGE;
        const float* sb = lds_b + cur * Cfg::B_STAGE;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            if (kk + 1 < KK) {
                read_frag(F[(kk + 1) & 1], sa, sb, kk + 1);
            } else if (MODE != 0) {
                float* na = lds_a + (cur ^ 1) * Cfg::A_STAGE;
                float* nb = lds_b + (cur ^ 1) * Cfg::B_STAGE;
                la.template store<AP>(na);
                lb.template store<BP>(nb);
                __syncthreads();
                if (MODE == 1 || MODE == 2) {
                    la.advance();
                    lb.advance();
                    la.template fetch<MODE == 2>((s + 2) * BK, K);
                    lb.template fetch<MODE == 2>((s + 2) * BK, K);
                    __builtin_amdgcn_sched_barrier(0);
                }
                read_frag(F[0], na, nb, 0);
            }
            mfma_frag(F[kk & 1]);
        }
    };
    using Dyn = std::integral_constant<int, -1>;
    DrainPhases drain;
    if (FAIR > 0) drain.init(FAIR, nslab, g.drain_from);
    int s = 0;
    for (; s + 3 < nfull; s += 2) {  // two slabs per trip: constant LDS stage offsets
        if (FAIR > 0) drain.step(s);
        slab(s, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
        slab(s + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
    }
    for (; s + 2 < nfull; ++s) slab(s, std::integral_constant<int, 1>{}, Dyn{});
    for (; s + 2 < nslab; ++s) slab(s, std::integral_constant<int, 2>{}, Dyn{});
    for (; s + 1 < nslab; ++s) slab(s, std::integral_constant<int, 3>{}, Dyn{});
    slab(s, std::integral_constant<int, 0>{}, Dyn{});

    mfma_epilogue<FM, FN, VEC>(g.M, g.N, g.alpha, g.beta, g.C, g.ldc, acc, m0 + wm0, n0 + wn0, li, lh);
}

}  // namespace libsgemm
