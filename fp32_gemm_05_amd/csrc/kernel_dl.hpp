// kernel_dl.hpp -- the direct-to-LDS MFMA kernel (global_load_lds into a ring of LDS stages).
#pragma once

#include "kernel_common.hpp"

namespace libsgemm {

// ---------------------------------------------------------------------------------
// Direct-to-LDS MFMA kernel: the operand slabs go from global memory straight into LDS with
// gfx950's global_load_lds (each lane's W bytes land at the wave's LDS base + W x lane; W = 16
// with global_load_lds_dwordx4 for 16-byte aligned rows, W = 4 with global_load_lds_dword
// otherwise), so no register holds a prefetched slab and no LDS store instruction runs in the K
// loop -- the stores that, at one wave per SIMD, take issue cycles and VGPR read bandwidth from
// the matrix pipe.  STAGES LDS buffers form a ring: slab s + STAGES - 1 is requested right after
// the barrier that opens slab s, into the buffer every wave finished reading before that
// barrier, so a slab has STAGES - 1 slabs of MFMAs to arrive.  One barrier per slab; before it,
// each wave waits (s_waitcnt vmcnt) only for its own loads of the next slab, leaving later slabs
// in flight.
//
// Layout: a wave's load fills 64 W bytes of LDS contiguously, so the slabs are unpadded -- A as
// [BM][BK] (k contiguous), B as [BK][BN] (n contiguous) -- and bank conflicts of the fragment
// reads are avoided by choosing WHICH 16-byte quad of its row a lane (W = 16) or a group of four
// lanes (W = 4) fetches: the quad at LDS position u of row r holds global quad u ^ swz(r) (an XOR
// swizzle, a permutation within the row, so the loads of a row still cover the same cache lines).
// The swizzles make the 128-bit A reads (16 consecutive rows at one quad) and the 32-bit B reads
// (rows k and k + 4 at 32 consecutive columns) free of conflicts both with 64 banks and 16 lanes
// per pass and with 32 banks and 8 lanes per pass.
//
// Edges: rows of A past M and columns of B past N are clamped (they feed C elements that are never
// stored).  The slab that crosses K is loaded with k clamped into range, so every address lies
// inside the operand, and each wave then overwrites what it loaded past K with zeros, after its
// loads have landed and before the barrier.  W = 16 needs the 128-bit variants' precondition
// (16-byte aligned rows; K and N multiples of 4).
// ---------------------------------------------------------------------------------
// The LDS serves a 128-bit access of 64 lanes in four passes of 16 lanes: lanes of one half-wave
// (lane / 32) whose bits 2-4 have the same parity (lanes 0-3, 12-15, 20-23, 24-27 and lanes 4-11,
// 16-19, 28-31, then the same in the upper half) -- measured lane pair by lane pair with the
// SQ_LDS_BANK_CONFLICT counter.  A pass is conflict-free when its 16 accesses cover the 64 banks.
// 32x32 blocks: a pass holds 16 rows of one quad; 16x16 blocks: 8 rows of one lane group's quad and
// the complementary 8 rows of the next group's, which these swizzles keep apart.
template <int QPR, int MB = 32>
__device__ __host__ inline int dl_swz_a(int r) {  // swizzle of A row r (QPR quads per row)
    static_assert(QPR == 4 || QPR == 8 || QPR == 16, "A rows of 16, 32 or 64 floats");
    if (MB == 16) return QPR == 16 ? r & 15 : QPR == 8 ? (r >> 1) & 7 : ((r >> 3) & 1) * 2;
    return QPR == 16 ? r & 15 : QPR == 8 ? ((r & 15) + ((r >> 3) & 1)) & 7 : (((r >> 1) & 7) + ((r >> 3) & 1)) & 3;
}
// Swizzle of B row k, in quads, for MFMA blocks of MB columns: a B fragment read (32-bit, one pass
// of 64 lanes) takes row 4 h + t (t fixed) of each of the 64 / MB lane groups h at MB consecutive
// columns, and the swizzle flips the column by MB h on those rows (quad bit 3 for 32x32 blocks;
// quad bits 2-3 for 16x16 blocks), putting the groups on distinct banks.
template <int MB = 32>
__device__ __host__ inline int dl_swz_b(int k) {
    static_assert(MB == 32 || MB == 16, "32x32 or 16x16 MFMA blocks");
    return ((k >> 2) & (64 / MB - 1)) * (MB / 4);
}
// B rows of 32 floats (one 32x32 block wide) span only half the banks, so the column flip above has
// no room: instead row k is stored at row k ^ ((k >> 2) & 1) (rows 4-7 of every 8 trade places in
// pairs), which gives the rows 4 h + t of the two lane groups opposite parities, i.e. opposite
// halves of the 64 banks.  The map is its own inverse.  Rows of 64 floats or more keep k.
template <int BN>
__device__ __host__ inline int dl_brow(int k) {
    return BN == 32 ? k ^ ((k >> 2) & 1) : k;
}

// MB: edge of the MFMA blocks (32: v_mfma_f32_32x32x2_f32; 16: v_mfma_f32_16x16x4_f32, whose
// smaller wave tiles let a workgroup of one tile hold more waves).  A fragment group spans
// KG = 4 (64 / MB) k: each of the 64 / MB lane groups of a wave brings one k-quad.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int W = 16, int MB = 32>
struct DlCfg {
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
    static constexpr int FM = WM / MB, FN = WN / MB;
    static constexpr int KG = 4 * (64 / MB);                      // k of one fragment group
    static constexpr int QPR_A = BK / 4, QPR_B = BN / 4;           // 16-byte quads per row
    static constexpr int A_STAGE = BM * BK, B_STAGE = BK * BN;     // floats
    static constexpr int CH = 16 * W;                              // floats one wave's load fills
    static constexpr int LA = A_STAGE / CH / NW, LB = B_STAGE / CH / NW;  // loads per wave and slab
    static constexpr int LPW = LA + LB;
    static constexpr int D = STAGES - 1;                           // slabs in flight ahead
    static constexpr int LDS_BYTES = STAGES * (A_STAGE + B_STAGE) * 4;
    static_assert(W == 4 || W == 16, "32-bit or 128-bit loads");
    static_assert(STAGES >= 2 && STAGES <= 4, "two to four LDS stages");
    static_assert(A_STAGE % (CH * NW) == 0 && B_STAGE % (CH * NW) == 0, "whole loads per wave");
    static_assert(BN % 64 == 0 || (BN == 32 && WN == 32 && MB == 32),
                  "B rows of 16 quads or more, or one 32x32 block wide (the row-permuted layout)");
    static_assert(MB == 32 || MB == 16, "32x32 or 16x16 MFMA blocks");
    static_assert(BK % KG == 0 && BM % WM == 0 && BN % WN == 0 && WM % MB == 0 && WN % MB == 0, "tiling");
    static_assert(NT <= 1024, "workgroup size");
    static_assert(LPW * D < 64, "vmcnt counts at most 63 loads in flight");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// The direct loads, their waits and the barrier are inline asm.  Issued through the compiler
// builtin, a load into LDS makes the compiler wait for it (s_waitcnt vmcnt(0)) before every later
// LDS read it cannot tell apart from the loaded stage -- here every fragment read -- which would
// expose the full load latency in every slab.  As asm with a memory clobber, the compiler neither
// waits for these loads nor moves LDS accesses across them, the barrier or the waits; the kernel
// waits for them itself.  Its own waits for other loads stay correct: counting fewer loads in
// flight than there are only makes a vmcnt wait stricter.  The loads have no register results.
// M0 holds the LDS address (M0 is reserved to the compiler, so the asm restores it); the s_nop
// covers the wait state between an SALU write of M0 and the load that reads it.
// NT: the load does not allocate in the caches (operand panels that no other workgroup reads).
template <int W, bool NT = false>
__device__ __attribute__((always_inline)) inline void dl_load(const void* base, uint32_t off, uint32_t lds) {
    uint32_t keep;
    if (W == 16 && NT)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3 nt\n\ts_mov_b32 m0, %0"
            : "=&s"(keep)
            : "s"(lds), "v"(off), "s"(base)
            : "memory");
    else if (W == 16)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
            : "=&s"(keep)
            : "s"(lds), "v"(off), "s"(base)
            : "memory");
    else if (NT)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, %3 nt\n\ts_mov_b32 m0, %0"
            : "=&s"(keep)
            : "s"(lds), "v"(off), "s"(base)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
            : "=&s"(keep)
            : "s"(lds), "v"(off), "s"(base)
            : "memory");
}
template <int W, bool NT = false>
__device__ __attribute__((always_inline)) inline void dl_load_at(const void* p, uint32_t lds) {
    uint32_t keep;
    if (W == 16 && NT)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off nt\n\ts_mov_b32 m0, %0"
            : "=&s"(keep)
            : "s"(lds), "v"(p)
            : "memory");
    else if (W == 16)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
            : "=&s"(keep)
            : "s"(lds), "v"(p)
            : "memory");
    else if (NT)
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off nt\n\ts_mov_b32 m0, %0"
            : "=&s"(keep)
            : "s"(lds), "v"(p)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
            : "=&s"(keep)
            : "s"(lds), "v"(p)
            : "memory");
}
// Wait until at most N of this wave's vector-memory loads are in flight and all its LDS accesses
// are done.
template <int N>
__device__ __attribute__((always_inline)) inline void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"i"(N) : "memory");
}
// The same with N = n * PER chosen at run time (n = 0 .. 3 slabs of PER loads each).
template <int PER>
__device__ __attribute__((always_inline)) inline void wait_slabs(int n) {
    if (n <= 0)
        wait_vm_lgkm0<0>();
    else if (n == 1)
        wait_vm_lgkm0<PER>();
    else if (n == 2)
        wait_vm_lgkm0<(2 * PER < 64 ? 2 * PER : 63)>();
    else
        wait_vm_lgkm0<(3 * PER < 64 ? 3 * PER : 63)>();
}
__device__ __attribute__((always_inline)) inline void dl_barrier() { asm volatile("s_barrier" ::: "memory"); }
// The LDS address of a pointer into a __shared__ array.
__device__ __attribute__((always_inline)) inline uint32_t lds_addr(const float* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float*)(p);
}
// Wave-uniform values the compiler cannot prove uniform (the persistent kernel's, which change
// from tile to tile), moved into scalar registers for the loads' M0 and scalar base operands.
// The builtin returns a signed int: each 32-bit half goes through uint32_t before it is widened,
// or a low word with bit 31 set would fill the high word with ones.
__device__ __attribute__((always_inline)) inline uint32_t uniform_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __attribute__((always_inline)) inline const float* uniform_ptr(const float* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = uniform_u32((uint32_t)v);
    const uint64_t hi = uniform_u32((uint32_t)(v >> 32));
    return reinterpret_cast<const float*>(lo | (hi << 32));
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int W, int OCC, int FAIR = 0, bool CPRE = false,
          bool SPREAD = false, int MB = 32, int EB = 0, bool NTA = false>
__global__ void __launch_bounds__((DlCfg<BM, BN, BK, WM, WN, STAGES, W, MB>::NT))
__attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1, 8)))
sgemm_mfma_dl_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    SGEMM_PHASE_STAMP(0);
    using Cfg = DlCfg<BM, BN, BK, WM, WN, STAGES, W, MB>;
    using Acc = typename MfmaBlock<MB>::acc_t;
    constexpr int FM = Cfg::FM, FN = Cfg::FN, KK = BK / Cfg::KG, LA = Cfg::LA, LB = Cfg::LB, D = Cfg::D;
    constexpr int QA = Cfg::QPR_A, QB = Cfg::QPR_B, CH = Cfg::CH, E = W / 4;  // E: floats per lane load
    constexpr int G = 64 / MB;                                                // lane groups of a wave
    constexpr bool VEC = W == 16;
    static_assert(KK % 2 == 0 || KK == 1, "fragment buffers alternate per fragment group");
    __shared__ __attribute__((aligned(1024))) float lds_a[STAGES * Cfg::A_STAGE];
    __shared__ __attribute__((aligned(1024))) float lds_b[STAGES * Cfg::B_STAGE];

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / Cfg::WAVES_N) * WM;
    const int wn0 = (wave % Cfg::WAVES_N) * WN;
    const int li = lane % MB, lh = lane / MB;  // lane within its group, lane group
    const int M = g.M, N = g.N, K = g.K;
    const long lda = g.lda, ldb = g.ldb;

    // This lane's loads: load j of the wave fills floats [c CH, (c + 1) CH) of the slab,
    // c = wave * L + j; the lane's E floats start at float f = c CH + E lane, i.e. row f / (row
    // length), LDS quad u = (f % row length) / 4, element f % 4 of it, which holds global quad
    // u ^ swz(row).
    // The k of a lane's load j inside the slab (recomputed where needed: only the slab that
    // crosses K uses it, and keeping it live would cost registers throughout the loop).
    auto a_kin = [&](int j) {
        const int f = (wave * LA + j) * CH + E * lane;
        return 4 * (((f % BK) / 4) ^ dl_swz_a<QA, MB>(f / BK)) + f % 4;
    };
    // the k of a lane's B load: the row it fills, through the row permutation of 32-float rows
    auto b_kin = [&](int j) { return dl_brow<BN>(((wave * LB + j) * CH + E * lane) / BN); };
    uint32_t a_off[LA], b_off[LB];  // byte offsets from the slab's first element
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int f = (wave * LA + j) * CH + E * lane;
        const int row = imin(m0 + f / BK, M - 1) - m0;
        a_off[j] = (uint32_t)(((long)row * lda + a_kin(j)) * 4);
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        const int f = (wave * LB + j) * CH + E * lane;
        const int kr = f / BN, u = (f % BN) / 4;
        const int k = dl_brow<BN>(kr);
        const int n = imin(n0 + 4 * (BN == 32 ? u : u ^ dl_swz_b<MB>(kr)) + f % 4, N - E) - n0;
        b_off[j] = (uint32_t)(((long)k * ldb + n) * 4);
    }
    const float* a_tile = g.A + (long)m0 * lda;  // A(m0, 0)
    const float* b_tile = g.B + n0;              // B(0, n0)

    // Request slab s into its stage.  TAIL: the slab crosses K; k is clamped into range here (the
    // address moves from k0 + k to min(k0 + k, K - E) for A, to row min(k0 + k, K - 1) for B) and
    // what lies past K is zeroed by fix_tail once the loads have landed.
    auto issue = [&](int s, auto tail) {
        constexpr bool TAIL = decltype(tail)::value;
        const int st = s % STAGES, k0 = s * BK;
        float* sa = lds_a + st * Cfg::A_STAGE + wave * LA * CH;
        float* sb = lds_b + st * Cfg::B_STAGE + wave * LB * CH;
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            if (!TAIL) {
                dl_load<W, NTA>(a_tile + k0, a_off[j], lds_addr(sa + j * CH));
            } else {
                const int k = a_kin(j);
                dl_load_at<W, NTA>(reinterpret_cast<const char*>(a_tile) + a_off[j] + 4L * (imin(k0 + k, K - E) - k),
                              lds_addr(sa + j * CH));
            }
        }
#pragma unroll
        for (int j = 0; j < LB; ++j) {
            if (!TAIL) {
                dl_load<W>(b_tile + (long)k0 * ldb, b_off[j], lds_addr(sb + j * CH));
            } else {
                const int k = b_kin(j);
                dl_load_at<W>(reinterpret_cast<const char*>(b_tile) + b_off[j] + 4L * (imin(k0 + k, K - 1) - k) * ldb,
                              lds_addr(sb + j * CH));
            }
        }
    };
    // Load q (0 .. LPW - 1) of whole slab s: the A loads, then the B loads.
    auto issue_one = [&](int s, int q) {
        const int st = s % STAGES, k0 = s * BK;
        if (q < LA)
            dl_load<W, NTA>(a_tile + k0, a_off[q], lds_addr(lds_a + st * Cfg::A_STAGE + (wave * LA + q) * CH));
        else
            dl_load<W>(b_tile + (long)k0 * ldb, b_off[q - LA],
                       lds_addr(lds_b + st * Cfg::B_STAGE + (wave * LB + q - LA) * CH));
    };
    // After the loads of the slab that crosses K have landed: zero what lies past K (each wave
    // the elements its own loads wrote; with W = 16, K % 4 == 0 makes a quad wholly in or out).
    auto fix_tail = [&](int s) {
        const int st = s % STAGES, k0 = s * BK;
        float* sa = lds_a + st * Cfg::A_STAGE + wave * LA * CH;
        float* sb = lds_b + st * Cfg::B_STAGE + wave * LB * CH;
#pragma unroll
        for (int j = 0; j < LA; ++j)
            if (k0 + a_kin(j) >= K) {
                if (VEC)
                    *reinterpret_cast<f32x4*>(sa + j * CH + E * lane) = f32x4{0.f, 0.f, 0.f, 0.f};
                else
                    sa[j * CH + lane] = 0.f;
            }
#pragma unroll
        for (int j = 0; j < LB; ++j)
            if (k0 + b_kin(j) >= K) {
                if (VEC)
                    *reinterpret_cast<f32x4*>(sb + j * CH + E * lane) = f32x4{0.f, 0.f, 0.f, 0.f};
                else
                    sb[j * CH + lane] = 0.f;
            }
    };

    // Fragment reads (fragment group kk: k = KG kk + 4 h + t for lane group h and step t): A's
    // quad G kk + h of row wm0 + MB fi + li sits at quad ((G kk + h) ^ swz) of that row (the
    // swizzle depends on the row's low four bits only, so not on fi); B's element (k, n) sits at
    // column n ^ MB h of row k (the B swizzle of row k is MB ((k >> 2) % G) columns).
    int a_frag[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        a_frag[kk] = (wm0 + li) * BK + 4 * ((G * kk + lh) ^ dl_swz_a<QA, MB>(wm0 + li));
    int b_frag[FN];
#pragma unroll
    for (int fj = 0; fj < FN; ++fj) b_frag[fj] = 4 * lh * BN + ((wn0 + fj * MB + li) ^ (MB * lh));
    // 32-float B rows: row 4 h + t of a fragment group sits at row dl_brow(4 h + t) (KG kk is a
    // multiple of 8, which the permutation leaves alone)
    int b_row32[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) b_row32[t] = dl_brow<BN>(4 * lh + t) * BN + li;
    auto read_frag = [&](MfmaFrag<FM, FN>& f, int st, int kk) {
        const float* sa = lds_a + st * Cfg::A_STAGE;
        const float* sb = lds_b + st * Cfg::B_STAGE;
#pragma unroll
        for (int fi = 0; fi < FM; ++fi)
            f.a[fi] = *reinterpret_cast<const f32x4*>(sa + a_frag[kk] + fi * MB * BK);
#pragma unroll
        for (int fj = 0; fj < FN; ++fj)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                f.b[fj][t] = BN == 32 ? sb[b_row32[t] + Cfg::KG * kk * BN] : sb[b_frag[fj] + (Cfg::KG * kk + t) * BN];
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < MfmaBlock<MB>::NR; ++r) acc[i][j][r] = 0.f;
    auto mfma_frag = [&](const MfmaFrag<FM, FN>& f) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_block_step<MB, VEC>(f.a[i][t], f.b[j][t], acc[i][j]);
    };

    const int nslab = (K + BK - 1) / BK;
    const int nfull = K / BK;
    using Tail = std::integral_constant<bool, true>;
    using Whole = std::integral_constant<bool, false>;
    // the C values of the beta term first: the oldest loads, consumed only by the epilogue
    Acc cv[FM][FN];
    if (CPRE && g.beta != 0.f) mfma_block_load_c<MB, FM, FN, VEC>(M, N, g.C, g.ldc, cv, m0 + wm0, n0 + wn0, li, lh);
    if constexpr (EB > 0) {
        // Early barrier (EB = P): the barrier that opens slab s + 1 sits P fragment groups before
        // the end of slab s.  Fragment reads run P groups ahead of the MFMAs (P + 1 register
        // buffers, buffer (s KK + kk) % (P + 1) for group kk of slab s), so every read of slab s has
        // been issued, and is waited for, before that barrier; the stage of slab s is free right
        // after it, and slab s + STAGES is requested there.  The barrier's wait for the slowest wave
        // then overlaps the P groups of MFMAs still to issue, and each slab's loads are requested
        // P groups earlier than in the form above.
        constexpr int P = EB, NB = EB + 1;
        static_assert(P < KK, "the barrier sits inside the slab");
        static_assert((STAGES * KK) % NB == 0, "the fragment buffers follow the ring's stages");
        static_assert(FAIR == 0, "no drain ordering with the early barrier");
        static_assert(Cfg::LPW * STAGES < 64, "vmcnt counts at most 63 loads in flight");
        using IC0 = std::integral_constant<int, 0>;
        using IC1 = std::integral_constant<int, 1 % STAGES>;
        using IC2 = std::integral_constant<int, 2 % STAGES>;
        using IC3 = std::integral_constant<int, 3 % STAGES>;
        // prologue: the whole ring requested (every stage is free); wait for slab 0
#pragma unroll
        for (int t = 0; t < STAGES; ++t) {
            if (t < nfull)
                issue(t, Whole{});
            else if (t < nslab)
                issue(t, Tail{});
        }
        wait_slabs<Cfg::LPW>(imin(STAGES, nslab) - 1);
        if (nfull == 0) {
            fix_tail(0);
            wait_vm_lgkm0<0>();
        }
        dl_barrier();
        MfmaFrag<FM, FN> F[NB];
#pragma unroll
        for (int q = 0; q < P; ++q) read_frag(F[q], 0, q);
        constexpr int LPG = (Cfg::LPW + P - 1) / P;  // spread requests per fragment group after the barrier
        // Slab s, stage STC = s % STAGES.  FULL: slabs s + 1 .. s + STAGES exist and are whole.
        auto slab_eb = [&](int s, auto stage, auto full) {
            constexpr int STC = decltype(stage)::value;
            constexpr bool FULL = decltype(full)::value;
            constexpr bool SP = SPREAD && FULL;
            const bool next = FULL || s + 1 < nslab;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                if (kk == KK - P && next) {
                    // slabs requested after slab s + 1: s + 2 .. min(s + STAGES - 1, nslab - 1)
                    if (FULL) {
                        wait_vm_lgkm0<Cfg::LPW * (STAGES - 2)>();
                    } else {
                        wait_slabs<Cfg::LPW>(imin(s + STAGES - 1, nslab - 1) - (s + 1));
                        if (s + 1 >= nfull) {
                            fix_tail(s + 1);
                            wait_vm_lgkm0<0>();
                        }
                    }
                    dl_barrier();
                    if (!SP) {
                        if (FULL || s + STAGES < nfull)
                            issue(s + STAGES, Whole{});
                        else if (s + STAGES < nslab)
                            issue(s + STAGES, Tail{});
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int gn = kk + P;  // the group read now, counted from slab s's first
                if (gn < KK)
                    read_frag(F[(STC * KK + gn) % NB], STC, gn);
                else if (next)
                    read_frag(F[(STC * KK + gn) % NB], (STC + 1) % STAGES, gn - KK);
                __builtin_amdgcn_sched_barrier(0);
                mfma_frag(F[(STC * KK + kk) % NB]);
                if (SP && kk >= KK - P) {
#pragma unroll
                    for (int q = (kk - (KK - P)) * LPG; q < (kk - (KK - P) + 1) * LPG && q < Cfg::LPW; ++q)
                        issue_one(s + STAGES, q);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        using Full = std::integral_constant<bool, true>;
        using Checked = std::integral_constant<bool, false>;
        SGEMM_PHASE_STAMP(1);
        int s = 0;
        for (; s + 2 * STAGES - 1 < nfull; s += STAGES) {
            slab_eb(s, IC0{}, Full{});
            slab_eb(s + 1, IC1{}, Full{});
            if (STAGES > 2) slab_eb(s + 2, IC2{}, Full{});
            if (STAGES > 3) slab_eb(s + 3, IC3{}, Full{});
        }
        // the last slabs, still STAGES to a trip so that every stage is known (s % STAGES == 0 here)
        for (; s < nslab; s += STAGES) {
            slab_eb(s, IC0{}, Checked{});
            if (s + 1 < nslab) slab_eb(s + 1, IC1{}, Checked{});
            if (STAGES > 2 && s + 2 < nslab) slab_eb(s + 2, IC2{}, Checked{});
            if (STAGES > 3 && s + 3 < nslab) slab_eb(s + 3, IC3{}, Checked{});
        }
        SGEMM_PHASE_STAMP(2);
        mfma_block_epilogue<MB, FM, FN, VEC, CPRE>(M, N, g.alpha, g.beta, g.C, g.ldc, acc, m0 + wm0, n0 + wn0, li,
                                                  lh, cv);
        SGEMM_PHASE_STAMP(3);
        return;
    }
    // prologue: slabs 0 .. D-1 requested; wait for slab 0 (the later ones may stay in flight)
#pragma unroll
    for (int s = 0; s < D; ++s) {
        if (s < nfull)
            issue(s, Whole{});
        else if (s < nslab)
            issue(s, Tail{});
    }
    wait_slabs<Cfg::LPW>(imin(D, nslab) - 1);
    if (nfull == 0) {
        fix_tail(0);
        wait_vm_lgkm0<0>();
    }
    dl_barrier();
    MfmaFrag<FM, FN> F[2];
    read_frag(F[0], 0, 0);

    // Slab s (stage ST = s % STAGES when known at compile time, else -1).  FULL: slab s + D exists
    // and is whole, so the wait before the next barrier leaves exactly D - 1 slabs in flight.
    // SPREAD (whole slabs, rings of three or more stages): the requests for slab s + D are issued
    // LPG at a time after each fragment group's MFMAs instead of all at the top of the slab, so that
    // they issue in the matrix pipe's shadow.  It pays at one wave per SIMD on L2-resident operands
    // (per-wave timestamps at 1024^3: 1103 against 1169 cycles per 16-MFMA slab), and costs where
    // the last requests, issued at the end of the slab, then have one slab instead of two to land
    // (three-stage 128x128 tiles at 4096^3: 1120 against 922 us), so it is a variant of its own.
    constexpr bool SP_ON = SPREAD && D >= 2 && KK > 1;
    constexpr int LPG = (Cfg::LPW + KK - 1) / KK;
    auto slab = [&](int s, auto stage, auto full) {
        constexpr int STC = decltype(stage)::value;
        constexpr bool FULL = decltype(full)::value;
        constexpr bool SP = SP_ON && FULL;
        const int st = STC >= 0 ? STC : s % STAGES;
        if (!SP) {
            if (FULL || s + D < nfull)
                issue(s + D, Whole{});
            else if (s + D < nslab)
                issue(s + D, Tail{});
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
            read_frag(F[(kk + 1) & 1], st, kk + 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frag(F[kk & 1]);
            if (SP) {
#pragma unroll
                for (int q = kk * LPG; q < (kk + 1) * LPG && q < Cfg::LPW; ++q) issue_one(s + D, q);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (SP) {
#pragma unroll
            for (int q = (KK - 1) * LPG; q < Cfg::LPW; ++q) issue_one(s + D, q);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (FULL || s + 1 < nslab) {
            // slabs requested after slab s + 1: s + 2 .. min(s + D, nslab - 1)
            if (FULL) {
                wait_vm_lgkm0<Cfg::LPW * (D - 1)>();
            } else {
                wait_slabs<Cfg::LPW>(imin(s + D, nslab - 1) - (s + 1));
                if (s + 1 >= nfull) {
                    fix_tail(s + 1);
                    wait_vm_lgkm0<0>();
                }
            }
            dl_barrier();
            read_frag(F[0], STC >= 0 ? (STC + 1) % STAGES : (s + 1) % STAGES, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        mfma_frag(F[(KK - 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
    };
    using Full = std::integral_constant<bool, true>;
    using Checked = std::integral_constant<bool, false>;
    DrainPhases drain;
    if (FAIR > 0) drain.init(FAIR, nslab, g.drain_from);
    SGEMM_PHASE_STAMP(1);
    int s = 0;
    // STAGES slabs per trip, so that every stage offset is a constant
    for (; s + STAGES - 1 + D < nfull; s += STAGES) {
        if (FAIR > 0) drain.step(s);
        slab(s, std::integral_constant<int, 0>{}, Full{});
        slab(s + 1, std::integral_constant<int, 1>{}, Full{});
        if (STAGES > 2) slab(s + 2, std::integral_constant<int, 2 % STAGES>{}, Full{});
        if (STAGES > 3) slab(s + 3, std::integral_constant<int, 3 % STAGES>{}, Full{});
    }
    for (; s < nslab; ++s) slab(s, std::integral_constant<int, -1>{}, Checked{});
    SGEMM_PHASE_STAMP(2);

    mfma_block_epilogue<MB, FM, FN, VEC, CPRE>(M, N, g.alpha, g.beta, g.C, g.ldc, acc, m0 + wm0, n0 + wn0, li, lh,
                                              cv);
    SGEMM_PHASE_STAMP(3);
}

// ---------------------------------------------------------------------------------
// Persistent direct-to-LDS kernel: a grid-stride tile loop (the block loops of the handbook's
// sgemm_tiled / sgemm_regblock, "Shared Memory and Register Blocking"), one workgroup per
// resident slot.  Workgroup w runs tiles w, w + G, w + 2 G, ... (G = grid size, tile t placed by
// tile_of exactly where the one-tile-per-workgroup kernels place workgroup t), and its slabs form
// ONE sequence through the LDS ring across tiles: slab gs of the workgroup is slab gs % nslab of
// its tile gs / nslab.  So the first slabs of the next tile are requested while the current tile
// finishes, and the next tile's prologue hides under the current tile's last slabs and epilogue
// instead of stalling a newly started workgroup.  Same loads, layout, waits and edge handling as
// sgemm_mfma_dl_kernel; the per-lane load offsets (which depend on the tile through the M and N
// clamps) are recomputed when the requests move to the next tile.  Every vmcnt wait also covers
// the epilogue's C accesses issued before it, which only makes it stricter.
// ---------------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int W, int OCC, bool SPREAD = false>
__global__ void __launch_bounds__((DlCfg<BM, BN, BK, WM, WN, STAGES, W>::NT))
__attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1, 8)))
sgemm_mfma_dlp_kernel(GemmArgs g, int tiles_m, int tiles_n, int group_m) {
    static_assert(BN % 64 == 0, "the persistent form keeps the column-flipped B layout");
    using Cfg = DlCfg<BM, BN, BK, WM, WN, STAGES, W>;
    constexpr int FM = Cfg::FM, FN = Cfg::FN, KK = BK / 8, LA = Cfg::LA, LB = Cfg::LB, D = Cfg::D;
    constexpr int QA = Cfg::QPR_A, CH = Cfg::CH, E = W / 4;
    constexpr bool VEC = W == 16;
    static_assert(KK % 2 == 0 || KK == 1, "fragment buffers alternate per 8-deep group");
    __shared__ __attribute__((aligned(1024))) float lds_a[STAGES * Cfg::A_STAGE];
    __shared__ __attribute__((aligned(1024))) float lds_b[STAGES * Cfg::B_STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / Cfg::WAVES_N) * WM;
    const int wn0 = (wave % Cfg::WAVES_N) * WN;
    const int li = lane & 31, lh = lane >> 5;
    // the arguments as local scalars: lambdas that capture the argument block itself make the
    // compiler keep an addressable copy of it in private memory
    const int M = g.M, N = g.N, K = g.K;
    const long lda = g.lda, ldb = g.ldb, ldc = g.ldc;
    const float alpha = g.alpha, beta = g.beta;
    const float* const Ag = g.A;
    const float* const Bg = g.B;
    float* const Cg = g.C;
    const int nt = tiles_m * tiles_n;
    const int mine = (nt - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;  // tiles of this workgroup
    const int nslab = (K + BK - 1) / BK;
    const int nfull = K / BK;
    const int total = mine * nslab;  // slabs of this workgroup

    auto origin = [&](int i, int& m0, int& n0) {
        int tm, tn;
        tile_of((int)blockIdx.x + i * (int)gridDim.x, nt, tiles_m, tiles_n, group_m, tm, tn);
        m0 = tm * BM;
        n0 = tn * BN;
    };
    auto a_kin = [&](int j) {
        const int f = (wave * LA + j) * CH + E * lane;
        return 4 * (((f % BK) / 4) ^ dl_swz_a<QA>(f / BK)) + f % 4;
    };
    auto b_kin = [&](int j) { return ((wave * LB + j) * CH + E * lane) / BN; };
    // Per lane and load: the in-tile row (A) or column (B) and the byte offset before the M / N
    // clamp, fixed for the whole kernel; a request applies the clamp of its tile to them.
    int a_row[LA], b_col[LB];
    uint32_t a_off0[LA], b_off0[LB];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int f = (wave * LA + j) * CH + E * lane;
        a_row[j] = f / BK;
        a_off0[j] = (uint32_t)(((long)a_row[j] * lda + a_kin(j)) * 4);
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        const int f = (wave * LB + j) * CH + E * lane;
        const int k = f / BN, u = (f % BN) / 4;
        b_col[j] = 4 * (u ^ dl_swz_b(k)) + f % 4;
        b_off0[j] = (uint32_t)(((long)k * ldb + b_col[j]) * 4);
    }
    // the tile whose slabs are being requested (uniform values only)
    int req = -1, req_m0 = 0, req_n0 = 0;
    const float* a_tile = Ag;
    const float* b_tile = Bg;
    auto request_tile = [&](int i) {
        if (i == req) return;
        req = i;
        origin(i, req_m0, req_n0);
        a_tile = uniform_ptr(Ag + (long)req_m0 * lda);
        b_tile = uniform_ptr(Bg + req_n0);
    };
    // clamped offsets: rows past M to M - 1, columns past N to the last E-wide group
    auto a_off = [&](int j) {
        const int over = req_m0 + a_row[j] - (M - 1);
        return a_off0[j] - (over > 0 ? (uint32_t)(over * lda * 4) : 0u);
    };
    auto b_off = [&](int j) {
        const int over = req_n0 + b_col[j] - (N - E);
        return b_off0[j] - (over > 0 ? (uint32_t)(over * 4) : 0u);
    };
    // request the whole slab at k0 of the request tile into ring stage st
    auto issue_full = [&](int k0, int st) {
        float* sa = lds_a + st * Cfg::A_STAGE + wave * LA * CH;
        float* sb = lds_b + st * Cfg::B_STAGE + wave * LB * CH;
#pragma unroll
        for (int q = 0; q < LA; ++q)
            dl_load<W>(uniform_ptr(a_tile + k0), a_off(q), uniform_u32(lds_addr(sa + q * CH)));
#pragma unroll
        for (int q = 0; q < LB; ++q)
            dl_load<W>(uniform_ptr(b_tile + (long)k0 * ldb), b_off(q), uniform_u32(lds_addr(sb + q * CH)));
    };
    // request slab j of tile i into ring stage st
    auto issue = [&](int i, int j, int st) {
        request_tile(i);
        const int k0 = j * BK;
        float* sa = lds_a + st * Cfg::A_STAGE + wave * LA * CH;
        float* sb = lds_b + st * Cfg::B_STAGE + wave * LB * CH;
        if (j < nfull) {
            issue_full(k0, st);
        } else {
#pragma unroll
            for (int q = 0; q < LA; ++q) {
                const int k = a_kin(q);
                dl_load_at<W>(reinterpret_cast<const char*>(a_tile) + a_off(q) + 4L * (imin(k0 + k, K - E) - k),
                              uniform_u32(lds_addr(sa + q * CH)));
            }
#pragma unroll
            for (int q = 0; q < LB; ++q) {
                const int k = b_kin(q);
                dl_load_at<W>(reinterpret_cast<const char*>(b_tile) + b_off(q) + 4L * (imin(k0 + k, K - 1) - k) * ldb,
                              uniform_u32(lds_addr(sb + q * CH)));
            }
        }
    };
    // load q of the whole slab at k0 into stage st (request_tile must already hold the slab's tile)
    auto issue_one = [&](int k0, int st, int q) {
        if (q < LA)
            dl_load<W>(uniform_ptr(a_tile + k0), a_off(q),
                       uniform_u32(lds_addr(lds_a + st * Cfg::A_STAGE + (wave * LA + q) * CH)));
        else
            dl_load<W>(uniform_ptr(b_tile + (long)k0 * ldb), b_off(q - LA),
                       uniform_u32(lds_addr(lds_b + st * Cfg::B_STAGE + (wave * LB + q - LA) * CH)));
    };
    // zero the entries of tail slab j (in stage st) whose k is past K
    auto fix_tail = [&](int j, int st) {
        const int k0 = j * BK;
        float* sa = lds_a + st * Cfg::A_STAGE + wave * LA * CH;
        float* sb = lds_b + st * Cfg::B_STAGE + wave * LB * CH;
#pragma unroll
        for (int q = 0; q < LA; ++q)
            if (k0 + a_kin(q) >= K) {
                if (VEC)
                    *reinterpret_cast<f32x4*>(sa + q * CH + E * lane) = f32x4{0.f, 0.f, 0.f, 0.f};
                else
                    sa[q * CH + lane] = 0.f;
            }
#pragma unroll
        for (int q = 0; q < LB; ++q)
            if (k0 + b_kin(q) >= K) {
                if (VEC)
                    *reinterpret_cast<f32x4*>(sb + q * CH + E * lane) = f32x4{0.f, 0.f, 0.f, 0.f};
                else
                    sb[q * CH + lane] = 0.f;
            }
    };
    // The request cursor: the next slab to request is slab rj of tile ri, into stage rst;
    // `requested` slabs of the workgroup have been requested so far.
    int ri = 0, rj = 0, rst = 0, requested = 0;
    auto advance_request = [&]() {
        ++requested;
        rst = rst + 1 == STAGES ? 0 : rst + 1;
        if (++rj == nslab) {
            rj = 0;
            ++ri;
        }
    };

    int a_frag[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        a_frag[kk] = (wm0 + li) * BK + 4 * ((2 * kk + lh) ^ dl_swz_a<QA>(wm0 + li));
    int b_frag[FN];
#pragma unroll
    for (int fj = 0; fj < FN; ++fj) b_frag[fj] = 4 * lh * BN + ((wn0 + fj * 32 + li) ^ (32 * lh));
    auto read_frag = [&](MfmaFrag<FM, FN>& f, int st, int kk) {
        const float* sa = lds_a + st * Cfg::A_STAGE;
        const float* sb = lds_b + st * Cfg::B_STAGE;
#pragma unroll
        for (int fi = 0; fi < FM; ++fi)
            f.a[fi] = *reinterpret_cast<const f32x4*>(sa + a_frag[kk] + fi * 32 * BK);
#pragma unroll
        for (int fj = 0; fj < FN; ++fj)
#pragma unroll
            for (int t = 0; t < 4; ++t) f.b[fj][t] = sb[b_frag[fj] + (8 * kk + t) * BN];
    };

    f32x16 acc[FM][FN];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    };
    zero_acc();
    auto mfma_frag = [&](const MfmaFrag<FM, FN>& f) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma_step<VEC>(f.a[i][t], f.b[j][t], acc[i][j]);
    };

    // prologue: the first D slabs requested; wait for slab 0
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (requested < total) {
            issue(ri, rj, rst);
            advance_request();
        }
    wait_slabs<Cfg::LPW>(imin(D, total) - 1);
    if (nfull == 0) {
        fix_tail(0, 0);
        wait_vm_lgkm0<0>();
    }
    dl_barrier();
    MfmaFrag<FM, FN> F[2];
    read_frag(F[0], 0, 0);

    constexpr bool SP_ON = SPREAD && D >= 2 && KK > 1;
    constexpr int LPG = (Cfg::LPW + KK - 1) / KK;
    // Tiles outside, slabs inside: the accumulators are one loop-carried set and the epilogue
    // has one copy.  The ring stage runs on as a counter across tiles.
    int st = 0;  // stage of the current slab
    // The MFMAs of the slab in stage st, with the loads of the slab at rk0 into stage rs spread
    // over its 8-deep groups (spread = true) or issued before it.
    auto slab_mfma = [&](bool spread, int rk0, int rs) {
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
            read_frag(F[(kk + 1) & 1], st, kk + 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frag(F[kk & 1]);
            if (SP_ON && spread) {
#pragma unroll
                for (int q = kk * LPG; q < (kk + 1) * LPG && q < Cfg::LPW; ++q) issue_one(rk0, rs, q);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (SP_ON && spread) {
#pragma unroll
            for (int q = (KK - 1) * LPG; q < Cfg::LPW; ++q) issue_one(rk0, rs, q);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int i = 0; i < mine; ++i) {
        // Steady slabs j < nfull - D: slab gs + D is a whole slab of this tile (so the request tile
        // is this tile and the cursor needs no checks), slab gs + 1 is a whole slab, and D - 1 slabs
        // stay in flight at the wait -- a body with no branches.  At j = 0 the cursor is at slab
        // D of this tile; the steady slabs move it on by jfast.
        const int jfast = imax(nfull - D, 0);
        for (int j = 0; j < jfast; ++j) {
            const int rs = st == 0 ? STAGES - 1 : st - 1;  // stage of slab gs + D (read by slab gs - 1)
            const int rk0 = (j + D) * BK;
            if (!SP_ON) issue_full(rk0, rs);
            __builtin_amdgcn_sched_barrier(0);
            slab_mfma(true, rk0, rs);
            const int nst = st + 1 == STAGES ? 0 : st + 1;
            wait_vm_lgkm0<Cfg::LPW * (D - 1)>();
            dl_barrier();
            read_frag(F[0], nst, 0);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frag(F[(KK - 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            st = nst;
        }
        if (jfast > 0) {
            requested += jfast;
            rst = (rst + jfast) % STAGES;
            rj += jfast;
            if (rj == nslab) {
                rj = 0;
                ++ri;
            }
        }
        // the last slabs of the tile: requests move on to the next tile, tails, the end of the work
        for (int j = jfast; j < nslab; ++j) {
            const int gs = i * nslab + j;
            // slab gs + D, the cursor's slab, if there is one: whole slabs may be spread
            const int sk0 = rj * BK, sst = rst;
            const bool more = requested < total;
            const bool sp = SP_ON && more && rj < nfull;
            if (sp) {
                request_tile(ri);
                advance_request();
            } else if (more) {
                issue(ri, rj, rst);
                advance_request();
            }
            __builtin_amdgcn_sched_barrier(0);
            slab_mfma(sp, sk0, sst);
            const int nst = st + 1 == STAGES ? 0 : st + 1;
            if (gs + 1 < total) {
                // slabs requested after slab gs + 1 may stay in flight
                wait_slabs<Cfg::LPW>(requested - (gs + 2));
                const int nj = j + 1 == nslab ? 0 : j + 1;
                if (nj >= nfull) {
                    fix_tail(nj, nst);
                    wait_vm_lgkm0<0>();
                }
                dl_barrier();
                read_frag(F[0], nst, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            mfma_frag(F[(KK - 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            st = nst;
        }
        int m0, n0;
        origin(i, m0, n0);
        mfma_epilogue<FM, FN, VEC>(M, N, alpha, beta, Cg, ldc, acc, m0 + wm0, n0 + wn0, li, lh);
        zero_acc();
    }
}

}  // namespace libsgemm
