// kernel_common.hpp -- what the HIP kernels of libsgemm share (gfx950, CDNA4, wave64).
//
// Every kernel computes C := alpha*A*B + beta*C on row-major fp32 matrices with
// leading dimensions (the operation of "SGEMM CUDA kernel (First Half)",
// introduction).  One workgroup owns one BM x BN tile of C and walks K in
// BK-deep slabs, staging a BM x BK slab of A and a BK x BN slab of B in LDS
// (the shared-memory tiling of "Shared Memory and Register Blocking", CUDA
// Handbook ch. 17).  What is MI355X-specific:
//
//   * two LDS stages: slab s+1 is fetched from global memory into registers
//     while slab s is multiplied out of LDS, then written to the other stage,
//     so each slab costs one workgroup barrier instead of two;
//   * the MFMA family multiplies with v_mfma_f32_32x32x2_f32: a wave owns a
//     WM x WN sub-tile made of 32x32 blocks (the warp tiling of "Optimizing
//     Matrix Multiplication in CUDA", section "Warp Tiling", re-cut for 64-lane
//     waves and matrix cores);
//   * the VALU family keeps a TM x TN register microtile per lane (the outer
//     product of "SGEMM CUDA kernel (First Half)", "Part 4", and Figure 17-3 of
//     the handbook) with A stored k-major in LDS (the transposed slab of "Part
//     5: Reduced bank conflict (v3)");
//   * global loads are 128-bit (the float4 loads of "Part 6: Vectorized load
//     (v4)") when every row is 16-byte aligned, otherwise 32-bit; in both the
//     lane-fastest index walks contiguous memory (the coalescing of "Global
//     Memory Coalescing");
//   * the workgroup -> tile map is XCD-aware: consecutive workgroup ids are
//     spread round-robin over the 8 XCDs, so each XCD is handed a contiguous
//     range of tiles, ordered in groups of rows so that tiles running at the
//     same time share A rows and B columns in that XCD's L2.
//
// Edge handling (out-of-range slab elements are zero, stores are guarded, as
// in the pages' bounds-checked kernels): A rows past M and B columns past N
// are clamped to the last valid row/column -- they only feed accumulators of C
// elements that are never stored -- while slab elements past K are zero, so
// that they add nothing (and no NaN) to valid outputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace libsgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct GemmArgs {
    int M, N, K;
    float alpha, beta;
    const float* A;
    long lda;
    const float* B;
    long ldb;
    float* C;
    long ldc;
    int drain_from;  // first workgroup of the grid's last round (no workgroup starts after it)
};

constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// Workgroup id -> (tile_m, tile_n).  A bijection of [0, tiles_m*tiles_n).
__host__ __device__ inline void tile_of(int wg, int nwg, int tiles_m, int tiles_n, int group_m,
                                        int& tm, int& tn) {
    // (1) the hardware hands workgroup w to XCD w % 8; renumber so that XCD x
    //     gets the contiguous range [start_x, start_x + count_x).
    const int q = nwg / kNumXcd, r = nwg % kNumXcd;
    const int x = wg % kNumXcd, p = wg / kNumXcd;
    const int t = x * q + (x < r ? x : r) + p;
    // (2) grouped order: blocks of group_m tile-rows, swept column by column.
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int rows_left = tiles_m - first_m;
    const int gsz = rows_left < group_m ? rows_left : group_m;
    const int local = t - g * per_group;
    tm = first_m + local % gsz;
    tn = local / gsz;
}

__device__ inline int imin(int a, int b) { return a < b ? a : b; }

// Phase stamps, compiled only into the profiling build (SGEMM_PHASE_STAMPS: libsgemm_stamps.so,
// read by `python -m fp32_gemm_05_amd.profiling phases`).  Lane 0 of every wave writes the shader
// clock (s_memtime) and the constant-rate real-time clock (s_memrealtime) at the kernel's phase
// boundaries -- slot 0 the kernel starts, 1 the first slab has landed and the K loop begins, 2 the
// K loop has ended, 3 the epilogue's stores are issued -- and, with slot 0, the wave's HW_ID
// register (its SIMD, CU, shader array and engine) in slot 4: g_phase_stamps[(w * 5 + slot) * 2]
// and [... + 1] for the grid's wave w = blockIdx.x * (waves per workgroup) + wave,
// w < g_phase_stamp_waves.  In every other build the hook is empty.
#ifdef SGEMM_PHASE_STAMPS
__device__ unsigned long long* g_phase_stamps;
__device__ unsigned g_phase_stamp_waves;
__device__ __attribute__((always_inline)) inline void phase_stamp(int slot) {
    __builtin_amdgcn_sched_barrier(0);
    const unsigned long long c = clock64(), r = wall_clock64();
    unsigned long long* buf = g_phase_stamps;
    const unsigned w = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if ((threadIdx.x & 63) == 0 && buf != nullptr && w < g_phase_stamp_waves) {
        buf[(w * 5 + slot) * 2] = c;
        buf[(w * 5 + slot) * 2 + 1] = r;
        if (slot == 0) buf[(w * 5 + 4) * 2] = (unsigned)__builtin_amdgcn_s_getreg((31 << 11) | 4);  // HW_ID
    }
    __builtin_amdgcn_sched_barrier(0);
}
#define SGEMM_PHASE_STAMP(slot) phase_stamp(slot)
#else
#define SGEMM_PHASE_STAMP(slot) ((void)0)
#endif
__device__ inline int imax(int a, int b) { return a > b ? a : b; }

// ---------------------------------------------------------------------------------
// Slab loaders (global -> registers -> LDS).  LDS slabs are row-major with a
// padded pitch: A as [BM][BK + PA] (k contiguous) for the MFMA kernel.
// ---------------------------------------------------------------------------------

// Loader of one operand's slab: a ROWS x COLS row-major panel, moved one slab
// along K per call of advance().  KROWS selects which panel dimension runs
// along K: false for A (the slab is BM rows x BK columns, K along columns),
// true for B (BK rows x BN columns, K along rows).  The other dimension is
// clamped once, at init, to the operand's last valid row/column (those lanes
// feed only C elements that are never stored); elements past K are zero and
// are checked only in the last, partial slab.  Vector form: one 16-byte load
// covers 4 consecutive columns (needs ld % 4 == 0, ncols % 4 == 0 and a
// 16-byte aligned base, which also make every 4-column group wholly inside or
// outside K).  Per-lane offsets are 32-bit unless WIDE (64-bit, for leading
// dimensions so large that one workgroup's panel spans 4 GiB or more).  NTL marks
// the loads nontemporal (streamed: no other workgroup reads this operand's panel).
template <int ROWS, int COLS, int NT, bool VEC, bool KROWS, bool WIDE, int NBUF = 1, bool NTL = false>
struct PanelLoader {
    using OffT = typename std::conditional<WIDE, uint64_t, uint32_t>::type;
    static constexpr int W = VEC ? 4 : 1;             // floats per load
    static constexpr int CPR = COLS / W;              // loads per panel row
    static constexpr int L = ROWS * CPR / NT;         // loads per thread
    static_assert(COLS % W == 0, "panel width");
    static_assert((ROWS * CPR) % NT == 0, "panel must split evenly over the workgroup");
    static_assert(NT % CPR == 0, "a load pass must cover whole panel rows");
    static constexpr int ROWS_PER_PASS = NT / CPR;

    f32x4 v[NBUF][L];      // NBUF register buffers of one slab each; only .x used when !VEC
    const float* base;     // workgroup-uniform address of the current slab's first row/column
    OffT off[L];           // this thread's BYTE offsets from base (same for every slab)
    int row0, col;         // this thread's first panel row and its column (panel coordinates)
    long step;             // address step from one slab to the next

    // The panel's top-left element is (r0, c0) of an nrows x ncols operand with leading
    // dimension ld.  Unless WIDE, byte offsets are 32-bit (the load then takes the uniform
    // base from scalar registers and only the offset from a vector register): the caller
    // guarantees ((ROWS - 1) * ld + COLS) * 4 < 2^32.
    __device__ inline void init(int tid, const float* __restrict__ op, long ld, int r0, int c0, int nrows,
                                int ncols, int bk) {
        row0 = tid / CPR;
        col = (tid % CPR) * W;
        step = KROWS ? (long)bk * ld : (long)bk;
        base = op + (long)r0 * ld + c0;
        int c = col;
        if (KROWS) c = imin(c0 + col, ncols - W) - c0;  // B: clamp columns past N
#pragma unroll
        for (int l = 0; l < L; ++l) {
            int r = row0 + l * ROWS_PER_PASS;
            if (!KROWS) r = imin(r0 + r, nrows - 1) - r0;  // A: clamp rows past M
            off[l] = (OffT)(((long)r * ld + c) * 4);
        }
    }

    __device__ inline void advance() { base += step; }

    // Position along K of the l-th element, relative to the slab start.
    __device__ inline int kpos(int l) const { return KROWS ? row0 + l * ROWS_PER_PASS : col; }

    // Fetch the current slab; with TAIL, elements whose K index (kbase + kpos) is >= K become zero.
    template <bool TAIL, int BUF = 0>
    __device__ inline void fetch(int kbase, int K) {
#pragma unroll
        for (int l = 0; l < L; ++l) {
            const bool ok = !TAIL || kbase + kpos(l) < K;
            // An empty asm statement that "redefines" the 32-bit offset keeps its zero extension
            // inside the loop, where it folds into the load's scalar-base + 32-bit-offset form
            // instead of becoming a 64-bit vector add per load and slab.
            if (!WIDE) asm volatile("" : "+v"(off[l]));
            const float* p = reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + off[l]);
            if (VEC) {
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f32x4* p4 = reinterpret_cast<const f32x4*>(p);
                v[BUF][l] = ok ? (NTL ? __builtin_nontemporal_load(p4) : *p4) : z;
            } else {
                v[BUF][l].x = ok ? (NTL ? __builtin_nontemporal_load(p) : *p) : 0.f;
            }
        }
    }

    // Fetch the slab starting at K index kbase (the pointers must already point at it).
    template <int BUF = 0>
    __device__ inline void fetch_slab(int kbase, int bk, int K) {
        if (kbase + bk <= K)
            fetch<false, BUF>(kbase, K);
        else
            fetch<true, BUF>(kbase, K);
    }

    // Store into an LDS panel [ROWS][PITCH].
    template <int PITCH, int BUF = 0>
    __device__ inline void store(float* __restrict__ lds) const {
#pragma unroll
        for (int l = 0; l < L; ++l) {
            float* q = lds + (row0 + l * ROWS_PER_PASS) * PITCH + col;
            if (VEC)
                *reinterpret_cast<f32x4*>(q) = v[BUF][l];
            else
                *q = v[BUF][l].x;
        }
    }

    // Store transposed into an LDS panel [COLS][PITCH] (element (r, c) -> lds[c][r]).
    template <int PITCH>
    __device__ inline void store_transposed(float* __restrict__ lds) const {
#pragma unroll
        for (int l = 0; l < L; ++l) {
            const int r = row0 + l * ROWS_PER_PASS;
            if (VEC) {
                lds[(col + 0) * PITCH + r] = v[0][l].x;
                lds[(col + 1) * PITCH + r] = v[0][l].y;
                lds[(col + 2) * PITCH + r] = v[0][l].z;
                lds[(col + 3) * PITCH + r] = v[0][l].w;
            } else {
                lds[col * PITCH + r] = v[0][l].x;
            }
        }
    }
};

// Loader of a B slab (BK rows along K x BN columns of a row-major B) for the 32-bit-load
// variants that stage B n-major in LDS, [BN][BK + 4]: each thread loads four consecutive k of one
// column -- four 32-bit loads, each coalesced along N across the wave, since the lane-fastest
// index is the column -- and writes them with ONE 128-bit LDS store, so that a lane's MFMA
// fragment, four consecutive k of one column, is one 128-bit LDS read (the staging transpose of
// "SGEMM CUDA kernel (First Half)", "Part 5: Reduced bank conflict (v3)", applied to B).  Against
// PanelLoader's one LDS store per element and four 32-bit fragment reads, a quarter of the LDS
// instructions for B.  Columns past N are clamped (they feed only C elements that are never
// stored); k past K is zero (checked in the last slab only).  The four rows of a quad are
// addressed from workgroup-uniform bases (scalar registers) plus one 32-bit per-lane byte offset
// per quad (64-bit when WIDE).  Same interface as PanelLoader.
template <int BK, int BN, int NT, bool WIDE, int NBUF = 1>
struct KQuadLoader {
    using OffT = typename std::conditional<WIDE, uint64_t, uint32_t>::type;
    static constexpr int QROWS = BK / 4;          // k-quads per column per slab
    static constexpr int QPP = NT / BN;           // k-quads of one column per pass of the workgroup
    static constexpr int L = QROWS * BN / NT;     // quads per thread
    static_assert(BK % 4 == 0 && NT % BN == 0 && QROWS % QPP == 0, "k-quads must split evenly");

    f32x4 v[NBUF][L];
    const float* base;  // workgroup-uniform address of the current slab's first row, first column
    long ld_bytes;      // bytes from one row of B to the next
    OffT off[L];        // byte offset of quad l's first element from base
    int q0, col;        // this thread's first quad row and its column (panel coordinates)
    long step;

    __device__ inline void init(int tid, const float* __restrict__ op, long ld, int r0, int c0, int nrows,
                                int ncols, int bk) {
        (void)nrows;
        col = tid % BN;
        q0 = tid / BN;
        step = (long)bk * ld;
        ld_bytes = ld * 4;
        base = op + (long)r0 * ld + c0;
        const int c = imin(c0 + col, ncols - 1) - c0;  // clamp columns past N
#pragma unroll
        for (int l = 0; l < L; ++l) off[l] = (OffT)(((long)(q0 + l * QPP) * 4 * ld + c) * 4);
    }

    __device__ inline void advance() { base += step; }

    template <bool TAIL, int BUF = 0>
    __device__ inline void fetch(int kbase, int K) {
#pragma unroll
        for (int l = 0; l < L; ++l) {
            if (!WIDE) asm volatile("" : "+v"(off[l]));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool ok = !TAIL || kbase + (q0 + l * QPP) * 4 + t < K;
                const float* p = reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) +
                                                                t * ld_bytes + off[l]);
                v[BUF][l][t] = ok ? *p : 0.f;
            }
        }
    }

    template <int BUF = 0>
    __device__ inline void fetch_slab(int kbase, int bk, int K) {
        if (kbase + bk <= K)
            fetch<false, BUF>(kbase, K);
        else
            fetch<true, BUF>(kbase, K);
    }

    // Store into an LDS panel [BN][PITCH] (column-major slab: element (k, n) at lds[n][k]).
    template <int PITCH, int BUF = 0>
    __device__ inline void store(float* __restrict__ lds) const {
#pragma unroll
        for (int l = 0; l < L; ++l) *reinterpret_cast<f32x4*>(lds + col * PITCH + (q0 + l * QPP) * 4) = v[BUF][l];
    }
};

// ---------------------------------------------------------------------------------
// MFMA kernel: v_mfma_f32_32x32x2_f32, wave tile WM x WN of 32x32 blocks.
//
// One 32x32x2 step computes D += X * Y where lane l (h = l / 32, i = l % 32)
// supplies X(i, h) and Y(h, i), and accumulator register r of lane l holds
// D(8*(r/4) + 4*h + r%4, i).  In the 128-bit variants each 32x32 block of C is
// accumulated transposed: X is fed from B (X(i, h) = B(k(h), n0 + i)) and Y from A
// (Y(h, i) = A(m0 + i, k(h))), so D = (A B)^T and register r of lane l holds
// C(m0 + i, n0 + 8*(r/4) + 4*h + r%4): every group of four registers is four
// consecutive columns of one row of C, written back with a single 128-bit store.
// Within one 8-deep group of a slab, step s in 0..3 takes k = 4*h + s for half h,
// so a lane's four A values are contiguous in the k-major LDS slab (one 128-bit
// LDS read) and the 8 k's of the group are each used exactly once.
// ---------------------------------------------------------------------------------
// TA / TB: op(A) = A^T (A stored K x M) / op(B) = B^T (B stored N x K).  The LDS slab of an
// operand keeps the layout of its global rows: k-contiguous [rows][BK + 4] when K runs along
// the stored rows (A, or B^T), and [BK][cols + 8] when it runs down the stored columns (B, or A^T).
// BQ: B (not transposed) is loaded in k-quads by KQuadLoader and staged n-major like B^T.
template <int BM, int BN, int BK, int WM, int WN, bool VEC, bool TA = false, bool TB = false, bool BQ = false>
struct MfmaCfg {
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr bool B_NMAJOR = TB || BQ;  // B slab stored [BN][BK + 4], k contiguous
    // k-contiguous slabs: pitch BK+4, so the 128-bit reads of 16 consecutive rows hit distinct
    // banks; k-strided slabs: pitch (width)+8, so the two half-waves (k and k+4) land on
    // opposite bank halves.
    static constexpr int A_PITCH = TA ? BM + 8 : BK + 4, B_PITCH = B_NMAJOR ? BK + 4 : BN + 8;
    static constexpr int A_STAGE = (TA ? BK : BM) * A_PITCH, B_STAGE = (B_NMAJOR ? BN : BK) * B_PITCH;
    static constexpr int LDS_BYTES = 2 * (A_STAGE + B_STAGE) * 4;
    static_assert(BM % WM == 0 && BN % WN == 0, "wave tiling");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
    static_assert(BK % 8 == 0, "BK must be a multiple of 8");
    static_assert(!(BQ && (TB || VEC)), "k-quad staging serves the 32-bit loads of an untransposed B");
};

// OCC > 0 asks the compiler for at least OCC waves per SIMD (registers capped at 512 / OCC),
// so that OCC workgroups of 4 waves fit on one CU.
// One 32x32x2 step on a block.  TRANS (used by the 128-bit variants) accumulates the block
// transposed, as described above; otherwise X comes from A and Y from B, D = A B, and register
// r of lane l holds C(m0 + 8*(r/4) + 4*h + r%4, n0 + i): lanes run along a row of C, which
// keeps the 32-bit stores of the unaligned variants coalesced.
template <bool TRANS>
__device__ __attribute__((always_inline)) inline f32x16 mfma_step(float a, float b, const f32x16& c) {
    return TRANS ? __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, c, 0, 0, 0)
                 : __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Epilogue of the MFMA kernels: C = alpha*acc + beta*C (C not read when beta == 0) for a
// wave whose tile starts at (m_base, n_base).  The 128-bit variants hold blocks transposed
// (four consecutive columns per four registers: one 128-bit store); the others hold them
// upright (32 lanes along a row: coalesced 32-bit stores).
// (Scalars are passed by value: taking the argument struct by reference makes the compiler
// keep an addressable copy of it, which it may place in LDS.)
// The beta term's C values and the stores of one 32x32 block whose top-left element is (r0, c0),
// in the accumulators' layout.  Addresses are a wave-uniform row base plus a 32-bit per-lane byte
// offset (one register however many values are in flight; the block spans 32 rows, so the offset
// fits when ldc < 2^25 -- for a larger ldc a 64-bit address is formed for each value in turn).  At an edge
// the loads' rows and columns are clamped into the matrix (the values read for positions outside
// are never stored): no load sits under a per-lane condition.  A load under a per-lane branch makes
// the compiler, which cannot count the memory operations in flight across such branches, wait for
// every one of them before each later use of a loaded value -- one memory round trip per store.
template <bool VEC>
__device__ __attribute__((always_inline)) inline f32x16 mfma_block_c(int M, int N, const float* __restrict__ C,
                                                                     long ldc, int r0, int c0, int li, int lh) {
    f32x16 c;
    // (r0, c0) is the same in every lane; stated with readfirstlane, the row base lives in scalar
    // registers
    r0 = __builtin_amdgcn_readfirstlane(r0);
    c0 = __builtin_amdgcn_readfirstlane(c0);
    // rows min(r0 + rr, M - 1): offsets from row rb = min(r0, M - 1) are >= 0 even for a block
    // wholly below the matrix
    const int rb = imin(r0, M - 1), rlim = M - 1 - rb, rd = r0 - rb;
    const char* base = reinterpret_cast<const char*>(C + (long)rb * ldc);
    if (ldc >= (1L << 25)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = VEC ? li : (r >> 2) * 8 + (r & 3) + 4 * lh;
            const int cc = VEC ? imin(c0 + (r >> 2) * 8 + lh * 4, N - 4) + (r & 3) : imin(c0 + li, N - 1);
            c[r] = C[((long)rb + imin(rd + rr, rlim)) * ldc + cc];
            asm volatile("" ::: "memory");  // one value at a time: no 64-bit address held across loads
        }
        return c;
    }
    if (VEC) {
        const uint32_t row_off = (uint32_t)(imin(rd + li, rlim) * ldc) * 4u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t off = row_off + 4u * (uint32_t)imin(c0 + q * 8 + lh * 4, N - 4);  // N % 4 == 0
            const f32x4 v = *reinterpret_cast<const f32x4*>(base + off);
            asm volatile("" ::: "memory");  // in program order: each offset computed just before its load
#pragma unroll
            for (int e = 0; e < 4; ++e) c[4 * q + e] = v[e];
        }
    } else {
        // register r holds row 8*(r/4) + 4*lh + r%4 of the block
        const uint32_t col_off = 4u * (uint32_t)imin(c0 + li, N - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = imin(rd + (r >> 2) * 8 + (r & 3) + 4 * lh, rlim);
            c[r] = *reinterpret_cast<const float*>(base + ((uint32_t)(rr * ldc) * 4u + col_off));
            asm volatile("" ::: "memory");
        }
    }
    return c;
}
template <bool VEC>
__device__ __attribute__((always_inline)) inline void mfma_block_store(int M, int N, float* __restrict__ C, long ldc,
                                                                       int r0, int c0, int li, int lh,
                                                                       const f32x16& x) {
    if (VEC) {
        const int row = r0 + li;
        if (row >= M) return;
        float* prow = C + (long)row * ldc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = c0 + q * 8 + lh * 4;  // the 4 columns are all inside or all outside
            if (col < N)
                *reinterpret_cast<f32x4*>(prow + col) = f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
        }
    } else {
        const int lrow = r0 + lh * 4, col = c0 + li;
        if (col >= N) return;
        float* pl = C + (long)lrow * ldc + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dr = (r >> 2) * 8 + (r & 3);
            if (lrow + dr < M) pl[dr * ldc] = x[r];
        }
    }
}

// The C values of a wave's output blocks for the beta term, in the accumulators' layout.  Kernels
// of one-round grids read them at the start of the tile, after their first operand loads, so that
// the read's latency hides under the K loop instead of stalling the epilogue.
template <int FM, int FN, bool VEC>
__device__ __attribute__((always_inline)) inline void mfma_load_c(int M, int N, const float* __restrict__ C,
                                                                  long ldc, f32x16 (&cv)[FM][FN], int m_base,
                                                                  int n_base, int li, int lh) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) cv[i][j] = mfma_block_c<VEC>(M, N, C, ldc, m_base + i * 32, n_base + j * 32, li, lh);
}

// C := alpha * acc + beta * C over a wave's output blocks (C not read when beta == 0).  The C
// values come from cv (PRE), or are read here a block at a time, all of a block's reads before
// its first store (16 registers, whatever the number of blocks).
template <int FM, int FN, bool VEC, bool PRE = false>
__device__ __attribute__((always_inline)) inline void mfma_epilogue(int M, int N, float alpha, float beta,
                                                                    float* __restrict__ C, long ldc,
                                                                    const f32x16 (&acc)[FM][FN], int m_base,
                                                                    int n_base, int li, int lh,
                                                                    const f32x16 (*cv)[FN] = nullptr) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int r0 = m_base + i * 32, c0 = n_base + j * 32;
            // alpha * acc rounded, then beta * C added by one fused multiply-add, in the C values'
            // own registers
            f32x16 x;
            if (beta != 0.f) {
                x = PRE ? cv[i][j] : mfma_block_c<VEC>(M, N, C, ldc, r0, c0, li, lh);
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(beta, x[r], alpha * acc[i][j][r]);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = alpha * acc[i][j][r];
            }
            mfma_block_store<VEC>(M, N, C, ldc, r0, c0, li, lh, x);
        }
}

// 16x16x4 blocks (v_mfma_f32_16x16x4_f32): lane l brings X(l % 16, k) and Y(k, l % 16) with
// k = l / 16, and register r of lane l holds D(4 (l / 16) + r, l % 16).  TRANS (the 128-bit
// variants): X from B and Y from A, so register r of lane l holds C(m0 + l % 16, n0 + 4 (l / 16)
// + r) -- four consecutive columns, one 128-bit access.  Otherwise X from A and Y from B, and
// register r holds C(m0 + 4 (l / 16) + r, n0 + l % 16): 16 lanes along a row of C.
template <bool TRANS>
__device__ __attribute__((always_inline)) inline f32x4 mfma16_step(float a, float b, const f32x4& c) {
    return TRANS ? __builtin_amdgcn_mfma_f32_16x16x4f32(b, a, c, 0, 0, 0)
                 : __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The beta term's C values and the stores of one 16x16 block at (r0, c0), in the accumulators'
// layout, under the same rules as the 32x32 blocks' (a uniform row base and 32-bit per-lane byte
// offsets; clamped rows and columns at an edge, no load under a per-lane condition).
template <bool VEC>
__device__ __attribute__((always_inline)) inline f32x4 mfma16_block_c(int M, int N, const float* __restrict__ C,
                                                                      long ldc, int r0, int c0, int li, int lh) {
    f32x4 c;
    r0 = __builtin_amdgcn_readfirstlane(r0);
    c0 = __builtin_amdgcn_readfirstlane(c0);
    const int rb = imin(r0, M - 1), rlim = M - 1 - rb, rd = r0 - rb;  // as for the 32x32 blocks
    const char* base = reinterpret_cast<const char*>(C + (long)rb * ldc);
    if (ldc >= (1L << 25)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = VEC ? li : 4 * lh + r;
            const int cc = VEC ? imin(c0 + 4 * lh, N - 4) + r : imin(c0 + li, N - 1);
            c[r] = C[((long)rb + imin(rd + rr, rlim)) * ldc + cc];
            asm volatile("" ::: "memory");
        }
        return c;
    }
    if (VEC) {
        const uint32_t off = (uint32_t)(imin(rd + li, rlim) * ldc) * 4u + 4u * (uint32_t)imin(c0 + 4 * lh, N - 4);
        return *reinterpret_cast<const f32x4*>(base + off);  // N % 4 == 0
    }
    const uint32_t col_off = 4u * (uint32_t)imin(c0 + li, N - 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        c[r] = *reinterpret_cast<const float*>(base + ((uint32_t)(imin(rd + 4 * lh + r, rlim) * ldc) * 4u + col_off));
        asm volatile("" ::: "memory");
    }
    return c;
}
template <bool VEC>
__device__ __attribute__((always_inline)) inline void mfma16_block_store(int M, int N, float* __restrict__ C,
                                                                         long ldc, int r0, int c0, int li, int lh,
                                                                         const f32x4& x) {
    if (VEC) {
        // N % 4 == 0 and col % 4 == 0: the 4 columns are all inside or all outside
        const int row = r0 + li, col = c0 + 4 * lh;
        if (row < M && col < N) *reinterpret_cast<f32x4*>(C + (long)row * ldc + col) = x;
    } else {
        const int row = r0 + 4 * lh, col = c0 + li;
        if (col >= N) return;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (row + r < M) C[(long)(row + r) * ldc + col] = x[r];
    }
}

// The C values of a wave's 16x16 blocks in the accumulators' layout (li = lane % 16, lh = lane / 16).
template <int FM, int FN, bool VEC>
__device__ __attribute__((always_inline)) inline void mfma16_load_c(int M, int N, const float* __restrict__ C,
                                                                    long ldc, f32x4 (&cv)[FM][FN], int m_base,
                                                                    int n_base, int li, int lh) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) cv[i][j] = mfma16_block_c<VEC>(M, N, C, ldc, m_base + i * 16, n_base + j * 16, li, lh);
}

// C := alpha * acc + beta * C over a wave's 16x16 blocks (C not read when beta == 0).  All C
// values are read before the first store (four registers a block), or come from cv (PRE).
template <int FM, int FN, bool VEC, bool PRE = false>
__device__ __attribute__((always_inline)) inline void mfma16_epilogue(int M, int N, float alpha, float beta,
                                                                      float* __restrict__ C, long ldc,
                                                                      const f32x4 (&acc)[FM][FN], int m_base,
                                                                      int n_base, int li, int lh,
                                                                      const f32x4 (*cv)[FN] = nullptr) {
    f32x4 cl[FM][FN];
    if (!PRE && beta != 0.f) mfma16_load_c<FM, FN, VEC>(M, N, C, ldc, cl, m_base, n_base, li, lh);
    const f32x4 (*cs)[FN] = PRE ? cv : cl;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x[r] = beta != 0.f ? __builtin_fmaf(beta, cs[i][j][r], alpha * acc[i][j][r]) : alpha * acc[i][j][r];
            mfma16_block_store<VEC>(M, N, C, ldc, m_base + i * 16, n_base + j * 16, li, lh, x);
        }
}

// The accumulator type and the step, C load and epilogue of MFMA blocks of edge MB.
template <int MB>
struct MfmaBlock;
template <>
struct MfmaBlock<32> {
    using acc_t = f32x16;
    static constexpr int NR = 16;  // accumulator registers per block
};
template <>
struct MfmaBlock<16> {
    using acc_t = f32x4;
    static constexpr int NR = 4;
};
template <int MB, bool TRANS>
__device__ __attribute__((always_inline)) inline typename MfmaBlock<MB>::acc_t mfma_block_step(
    float a, float b, const typename MfmaBlock<MB>::acc_t& c) {
    if constexpr (MB == 32)
        return mfma_step<TRANS>(a, b, c);
    else
        return mfma16_step<TRANS>(a, b, c);
}
template <int MB, int FM, int FN, bool VEC>
__device__ __attribute__((always_inline)) inline void mfma_block_load_c(int M, int N, const float* __restrict__ C,
                                                                        long ldc,
                                                                        typename MfmaBlock<MB>::acc_t (&cv)[FM][FN],
                                                                        int m_base, int n_base, int li, int lh) {
    if constexpr (MB == 32)
        mfma_load_c<FM, FN, VEC>(M, N, C, ldc, cv, m_base, n_base, li, lh);
    else
        mfma16_load_c<FM, FN, VEC>(M, N, C, ldc, cv, m_base, n_base, li, lh);
}
template <int MB, int FM, int FN, bool VEC, bool PRE = false>
__device__ __attribute__((always_inline)) inline void mfma_block_epilogue(
    int M, int N, float alpha, float beta, float* __restrict__ C, long ldc,
    const typename MfmaBlock<MB>::acc_t (&acc)[FM][FN], int m_base, int n_base, int li, int lh,
    const typename MfmaBlock<MB>::acc_t (*cv)[FN] = nullptr) {
    if constexpr (MB == 32)
        mfma_epilogue<FM, FN, VEC, PRE>(M, N, alpha, beta, C, ldc, acc, m_base, n_base, li, lh, cv);
    else
        mfma16_epilogue<FM, FN, VEC, PRE>(M, N, alpha, beta, C, ldc, acc, m_base, n_base, li, lh, cv);
}

// Drain ordering.  A SIMD issues from its highest-priority ready wave, oldest first among equals,
// so of the workgroups sharing a CU the oldest runs nearly alone and finishes first; in a grid's
// last round nothing refills the freed slots, and the last workgroup ends up alone on its CU, where
// one wave per SIMD keeps the matrix pipe about two-thirds busy.  With FAIR, every wave starts at
// priority 3 and, in the last round only, steps down at three points of its K loop (schedule
// FAIR picks them): a wave ahead of the others on its SIMD drops below them until they catch up,
// so the last round's workgroups end together.
struct DrainPhases {
    int next, after, last;  // slabs of the remaining steps down (even; INT_MAX: none)
    int phase;              // 0..3
    // drain_from: first workgroup of the last round; INT_MAX turns the ordering off (a grid with no
    // more workgroups than CUs, where no two share a SIMD and priority changes only cost).
    __device__ inline void init(int fair, int nslab, int drain_from) {
        next = after = last = 0x7fffffff;
        phase = 0;
        if (drain_from == 0x7fffffff) return;
        const bool last_round = (int)blockIdx.x >= drain_from;
        // schedule 2: 1/2, 3/4, 7/8 of the K loop; 3: 3/4, 7/8, 15/16; 4: 7/8, 15/16, 31/32
        const int n1 = fair == 4 ? 28 : (fair == 3 ? 24 : 16);
        const int n2 = fair == 4 ? 30 : (fair == 3 ? 28 : 24);
        const int n3 = fair == 4 ? 31 : (fair == 3 ? 30 : 28);
        next = last_round ? (int)(((long)nslab * n1 / 32) & ~1L) : 0x7fffffff;
        after = (int)(((long)nslab * n2 / 32) & ~1L);
        last = (int)(((long)nslab * n3 / 32) & ~1L);
        __builtin_amdgcn_s_setprio(3);
    }
    __device__ inline void step(int s) {
        if (s >= next) {
            ++phase;
            if (phase == 1)
                __builtin_amdgcn_s_setprio(2);
            else if (phase == 2)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
            next = after;
            after = last;
            last = 0x7fffffff;
        }
    }
};

// LDS -> register fragments of one 8-deep group (the pipelined, deep and direct-to-LDS kernels).
template <int FM, int FN>
struct MfmaFrag {
    f32x4 a[FM];
    float b[FN][4];
};

// ---------------------------------------------------------------------------------
// C := beta * C (the alpha == 0 / K == 0 case; beta == 0 writes zeros without reading C).
// ---------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) sgemm_scale_kernel(int M, int N, float beta, float* C, long ldc) {
    const long total = (long)M * N;
    for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
        const long i = e / N, j = e - i * N;
        float* p = C + i * ldc + j;
        *p = (beta == 0.f) ? 0.f : beta * *p;
    }
}

}  // namespace libsgemm
