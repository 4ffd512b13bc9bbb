// kernel_direct.hpp -- the LDS-free MFMA kernel of small grids (operands straight into registers).
#pragma once

#include "kernel_common.hpp"

namespace libsgemm {

// ---------------------------------------------------------------------------------
// LDS-free MFMA kernel for small grids.  One wave per workgroup owns a 32x32 tile of C and loads
// its MFMA operands from global memory straight into registers, in the layout the 32x32x2
// instruction takes: for each 8-deep group of K, lane (i, h) needs A(m0+i, k) and B(k, n0+i) for
// k = 4h + t, t = 0..3.  There is no LDS and no barrier; the loads run D groups ahead of the
// MFMAs in a ring of registers.  Rows past M and columns past N are clamped (they feed outputs
// that are never stored); k past K is zero.
// ---------------------------------------------------------------------------------

// One operand of the LDS-free kernel, X(r, k) with r = r0 + i along the tile (m for A, n for B).
// KC: k runs along the stored rows (A, or B^T): a lane's four k values are contiguous, one
// 128-bit load (VEC) or four 32-bit loads from row min(r0+i, R-1).  Otherwise (B, or A^T) each k
// is a stored row and the lane reads column min(r0+i, R-1) of it: four 32-bit loads whose 32
// lanes read 128 contiguous bytes.  Addressing of the full groups of the main loop: the tile's
// origin plus a workgroup-uniform byte position that moves D groups per trip, plus
// loop-invariant 32-bit per-lane byte offsets (KC: one, the group's step being an immediate;
// otherwise one per (slot, t)), so each load is a scalar base plus a vector offset.  The
// prologue's and the last trips' groups, which may reach past K, are addressed from the origin
// with k clamped to K - 1, so no address outside the operand is ever formed.  The caller
// guarantees the offsets fit 32 bits: KC: (31 * ld + 16 D) * 4 < 2^32, otherwise
// ((16 D - 1) * ld + 32) * 4 < 2^32.
template <bool KC, bool VEC, int D>
struct DirectOperand {
    static constexpr int NO = KC ? 1 : 4 * D;
    const char* origin;  // X(r0, 0)
    long pos;            // byte position of the current trip's first group from the origin
    long step;           // bytes per trip
    long ld;
    int r;               // this lane's clamped row (KC) or column, relative to r0
    uint32_t off[NO];

    __device__ inline void init(const float* X, long ld_, int r0, int R, int li, int lh) {
        ld = ld_;
        r = imin(r0 + li, R - 1) - r0;
        pos = 0;
        if (KC) {
            origin = reinterpret_cast<const char*>(X + (long)r0 * ld);
            step = (long)D * 32;
            off[0] = (uint32_t)(((long)r * ld + lh * 4) * 4);
        } else {
            origin = reinterpret_cast<const char*>(X + r0);
            step = (long)D * 8 * ld * 4;
            const long o = ((long)(lh * 4) * ld + r) * 4;
#pragma unroll
            for (int d = 0; d < D; ++d)
#pragma unroll
                for (int t = 0; t < 4; ++t) off[d * 4 + t] = (uint32_t)(o + ((long)(D + d) * 8 + t) * ld * 4);
        }
    }

    __device__ inline void advance() { pos += step; }

    // Slot d's values for k = kb + t, kb = 8 g + 4h.  Without TAIL, group g is the trip's
    // (D + d)-th group from its position and lies wholly below K.  With TAIL (any group), the
    // elements with k >= K are read at k = K - 1 (K - 4 for the 128-bit load), so that no load is
    // conditional and no address outside the operand is formed; the caller zeroes them when it
    // multiplies the slot (zero_past_k), one trip later.  Zeroing them here, right after the load,
    // made the compiler wait for each load in turn (vmcnt(0) after every tail load); a branch
    // around a load would make it wait for all loads in flight at the top of every trip.
    template <bool TAIL>
    __device__ inline void load(f32x4& v, int d, int kb, int K) {
        if (KC) {
            if (!TAIL) {
                asm volatile("" : "+v"(off[0]));
                const char* q = origin + pos + off[0] + (D + d) * 32;
                if (VEC)
                    v = *reinterpret_cast<const f32x4*>(q);
                else
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = reinterpret_cast<const float*>(q)[t];
            } else if (VEC) {  // K % 4 == 0: the four k are all below K or all at or past it
                v = *reinterpret_cast<const f32x4*>(origin + ((long)r * ld + imin(kb, K - 4)) * 4);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    v[t] = *reinterpret_cast<const float*>(origin + ((long)r * ld + imin(kb + t, K - 1)) * 4);
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (!TAIL) {
                    asm volatile("" : "+v"(off[d * 4 + t]));
                    v[t] = *reinterpret_cast<const float*>(origin + pos + off[d * 4 + t]);
                } else {
                    v[t] = *reinterpret_cast<const float*>(origin + ((long)imin(kb + t, K - 1) * ld + r) * 4);
                }
            }
        }
    }
};

// The values a TAIL load read for k >= K (k = kb + t) replaced by zeros, in both operands, so
// that the padded steps add exact zeros (0 * x with x finite, and never 0 * inf).
__device__ inline f32x4 zero_past_k(f32x4 v, int kb, int K) {
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = kb + t < K ? v[t] : 0.f;
    return v;
}

template <bool VEC, int D, bool TA = false, bool TB = false, bool CPRE = false>
__global__ void __launch_bounds__(64) sgemm_mfma_direct_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * 32, n0 = tn * 32;
    const int lane = threadIdx.x, li = lane & 31, lh = lane >> 5;
    const int K = g.K;
    DirectOperand<!TA, VEC, D> oa;  // A (M x K): k along its rows; A^T (K x M): k down its rows
    DirectOperand<TB, VEC, D> ob;   // B (K x N): k down its rows; B^T (N x K): k along its rows
    oa.init(g.A, g.lda, m0, g.M, li, lh);
    ob.init(g.B, g.ldb, n0, g.N, li, lh);

    f32x4 ra[D], rb[D];
    auto load = [&](int d, int grp, auto tail) {  // group grp into slot d
        constexpr bool TAIL = decltype(tail)::value;
        const int kb = 8 * grp + 4 * lh;
        oa.template load<TAIL>(ra[d], d, kb, K);
        ob.template load<TAIL>(rb[d], d, kb, K);
    };
    f32x16 acc[1][1];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][0][r] = 0.f;
    auto mfma = [&](int d) {
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[0][0] = mfma_step<VEC>(ra[d][t], rb[d][t], acc[0][0]);
    };
    auto mfma_tail = [&](int d, int grp) {  // slot d holds group grp, which may reach past K
        const int kb = 8 * grp + 4 * lh;
        const f32x4 a = zero_past_k(ra[d], kb, K), b = zero_past_k(rb[d], kb, K);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[0][0] = mfma_step<VEC>(a[t], b[t], acc[0][0]);
    };
    auto advance = [&]() {
        oa.advance();
        ob.advance();
    };
    using Tail = std::integral_constant<bool, true>;
    using Full = std::integral_constant<bool, false>;

    const int ngroups = (K + 7) / 8, nfull = K / 8;
    // at the top of the trip at group q, slot d holds group q + d (zeros for groups past K)
#pragma unroll
    for (int d = 0; d < D; ++d) load(d, d, Tail{});
    f32x16 cv[1][1];  // CPRE: C for the beta term, read after the ring's first loads
    if (CPRE && g.beta != 0.f) mfma_load_c<1, 1, VEC>(g.M, g.N, g.C, g.ldc, cv, m0, n0, li, lh);
    int q = 0;
    // main trips: slots q .. q + D - 1 hold groups below nfull, read exactly
    for (; q + 2 * D <= nfull; q += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            mfma(d);
            load(d, q + D + d, Full{});
        }
        advance();
    }
    for (; q + D < ngroups; q += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            mfma_tail(d, q + d);
            load(d, q + D + d, Tail{});
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) mfma_tail(d, q + d);

    mfma_epilogue<1, 1, VEC, CPRE>(g.M, g.N, g.alpha, g.beta, g.C, g.ldc, acc, m0, n0, li, lh, cv);
}

}  // namespace libsgemm
