// kernel_deep.hpp -- the deep-prefetch MFMA kernel for grids of about one workgroup per CU.
#pragma once

#include "kernel_common.hpp"

namespace libsgemm {

// ---------------------------------------------------------------------------------
// Deep-prefetch MFMA kernel, for grids of about one workgroup per compute unit: there a
// SIMD runs a single wave, and no other wave covers its stalls.  Same tiling, operand
// mapping, LDS layout (two stages) and epilogue as sgemm_mfma_kernel, with
//   - global loads two slabs ahead, into two register buffers (slab s+2 is fetched at the
//     top of slab s; slab s+1, fetched one slab earlier, is stored to LDS at its end), so a
//     load has two slabs of MFMAs to arrive instead of one;
//   - LDS -> register fragments read one 8-deep group ahead of the MFMAs that use them (the
//     order is pinned with scheduling barriers; left alone, the compiler reads each
//     fragment just before its use and the wave waits on every read);
//   - the next slab's first fragments read right after the slab's barrier, under the MFMAs
//     of the slab's last group.
// LDS safety with two stages and one barrier per slab: stage (s+1)&1 is written in slab s
// after the barrier of slab s-1, and every wave finished its reads of that stage (slab s-1)
// before reaching that barrier (the barrier waits for outstanding LDS accesses).
// ---------------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN, bool VEC, int OCC, int FAIR = 0, bool NTA = false,
          bool CPRE = false, bool ACC2 = false>
__global__ void __launch_bounds__((MfmaCfg<BM, BN, BK, WM, WN, VEC>::NT))
__attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1, 8)))
sgemm_mfma_deep_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    SGEMM_PHASE_STAMP(0);
    using Cfg = MfmaCfg<BM, BN, BK, WM, WN, VEC>;
    constexpr int NT = Cfg::NT, FM = Cfg::FM, FN = Cfg::FN;
    constexpr int AP = Cfg::A_PITCH, BP = Cfg::B_PITCH;
    constexpr int KK = BK / 8;
    static_assert(KK % 2 == 0, "fragment buffers alternate per 8-deep group: BK must be a multiple of 16");
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
    PanelLoader<BM, BK, NT, VEC, false, false, 2, NTA> la;
    PanelLoader<BK, BN, NT, VEC, true, false, 2> lb;
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
    // ACC2: odd k-steps accumulate into a second set of registers, so that consecutive MFMAs of a
    // wave that owns a single block do not depend on each other; the two sums are added at the end
    f32x16 acc2[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc2[i][j][r] = 0.f;
    auto mfma_frag = [&](const MfmaFrag<FM, FN>& f) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if (ACC2 && (t & 1))
                        acc2[i][j] = mfma_step<VEC>(f.a[i][t], f.b[j][t], acc2[i][j]);
                    else
                        acc[i][j] = mfma_step<VEC>(f.a[i][t], f.b[j][t], acc[i][j]);
                }
    };

    const int nslab = (K + BK - 1) / BK;
    const int nfull = K / BK;  // slabs with no element past K

    // prologue: slab 0 to LDS stage 0, slab 1 into register buffer 1
    la.template fetch_slab<0>(0, BK, K);
    lb.template fetch_slab<0>(0, BK, K);
    la.template store<AP, 0>(lds_a);
    lb.template store<BP, 0>(lds_b);
    if (nslab > 1) {
        la.advance();
        lb.advance();
        la.template fetch_slab<1>(BK, BK, K);
        lb.template fetch_slab<1>(BK, BK, K);
    }
    f32x16 cv[FM][FN];  // CPRE: C for the beta term, read after the first operand loads
    if (CPRE && g.beta != 0.f) mfma_load_c<FM, FN, VEC>(g.M, g.N, g.C, g.ldc, cv, m0 + wm0, n0 + wn0, li, lh);
    __syncthreads();
    MfmaFrag<FM, FN> F[2];
    read_frag(F[0], lds_a, lds_b, 0);

    // Slab s, with P = s & 1: LDS stage P holds slab s, register buffer P is free (slab s went
    // to LDS during slab s-1) and buffer P^1 holds slab s+1.  FULL: slab s+2 is a whole slab
    // (no K checks) and slab s+1 exists; otherwise both are decided at run time.
    auto slab = [&](int s, auto parity, auto full) {
        constexpr int P = decltype(parity)::value;
        constexpr bool FULL = decltype(full)::value;
        const float* sa = lds_a + P * Cfg::A_STAGE;
        const float* sb = lds_b + P * Cfg::B_STAGE;
        if (FULL) {
            la.advance();
            lb.advance();
            la.template fetch<false, P>((s + 2) * BK, K);
            lb.template fetch<false, P>((s + 2) * BK, K);
        } else if (s + 2 < nslab) {
            la.advance();
            lb.advance();
            la.template fetch<true, P>((s + 2) * BK, K);
            lb.template fetch<true, P>((s + 2) * BK, K);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
            read_frag(F[(kk + 1) & 1], sa, sb, kk + 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frag(F[kk & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (FULL || s + 1 < nslab) {
            float* na = lds_a + (P ^ 1) * Cfg::A_STAGE;
            float* nb = lds_b + (P ^ 1) * Cfg::B_STAGE;
            la.template store<AP, P ^ 1>(na);
            lb.template store<BP, P ^ 1>(nb);
            __syncthreads();
            read_frag(F[0], na, nb, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        mfma_frag(F[(KK - 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
    };
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    using Full = std::integral_constant<bool, true>;
    using Checked = std::integral_constant<bool, false>;
    DrainPhases drain;
    if (FAIR > 0) drain.init(FAIR, nslab, g.drain_from);
    SGEMM_PHASE_STAMP(1);
    int s = 0;
    for (; s + 3 < nfull; s += 2) {  // two slabs per trip: the buffer and stage of each are constants
        if (FAIR > 0) drain.step(s);
        slab(s, Even{}, Full{});
        slab(s + 1, Odd{}, Full{});
    }
    while (s < nslab) {  // s is even here
        slab(s, Even{}, Checked{});
        if (++s >= nslab) break;
        slab(s, Odd{}, Checked{});
        ++s;
    }
    SGEMM_PHASE_STAMP(2);

    if (ACC2) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] += acc2[i][j];
    }
    mfma_epilogue<FM, FN, VEC, CPRE>(g.M, g.N, g.alpha, g.beta, g.C, g.ldc, acc, m0 + wm0, n0 + wn0, li, lh, cv);
    SGEMM_PHASE_STAMP(3);
}

}  // namespace libsgemm
