"""Host model of the kernels' index math: every global load stays inside the operand,
every output element of C is stored exactly once, nothing outside C's M x N window
is stored, and each MFMA accumulator receives every k of a slab exactly once.

The model restates, in numpy, the addressing of the kernel headers (PanelLoader,
the MFMA and VALU epilogues) for each variant the library reports, over a sweep
of shapes with ragged edges in every dimension.  It runs on the CPU and guards
the GPU against out-of-bounds accesses before any kernel is launched.
"""
import itertools

import numpy as np
import pytest

import fp32_gemm_05_amd as sg
from fp32_gemm_05_amd import _binding


def variants():
    out = []
    for i in range(sg.sgemm_num_variants()):
        out.append(sg.sgemm_variant_info(i))
    return out


VARIANTS = variants()


def panel_loads(ROWS, COLS, NT, vec, r0, c0, nrows, ncols, clamp_rows, clamp_cols):
    """(rows, cols, width, loaded) of every load issued for one panel, mirroring PanelLoader.fetch."""
    W = 4 if vec else 1
    CPR = COLS // W
    assert COLS % W == 0 and (ROWS * CPR) % NT == 0 and NT % CPR == 0
    L = ROWS * CPR // NT
    RPP = NT // CPR
    tid = np.arange(NT)
    row0 = tid // CPR
    col = (tid % CPR) * W
    c = c0 + col
    cok = c < ncols
    if clamp_cols:
        c = np.minimum(c, ncols - W)
        cok = np.ones_like(cok)
    rows, cols, ok = [], [], []
    for l in range(L):
        r = r0 + row0 + l * RPP
        rok = r < nrows
        if clamp_rows:
            r = np.minimum(r, nrows - 1)
            rok = np.ones_like(rok)
        # LDS destination stays inside the panel
        assert (row0 + l * RPP).max() < ROWS and (col + W).max() <= COLS
        rows.append(r)
        cols.append(c)
        ok.append(rok & cok)
    return np.concatenate(rows), np.concatenate(cols), W, np.concatenate(ok)


def kquad_loads(BK, BN, NT, k0, c0, K, N):
    """(rows, cols, width, loaded) of every load of one B slab, mirroring KQuadLoader.fetch: thread
    tid takes column tid % BN (clamped to N - 1) and the k-quads tid // BN + l * NT / BN, four 32-bit
    loads each; k past K is not loaded.  Also checks that the slab's (k, column) positions are each
    written to LDS exactly once, inside the [BN][BK + 4] panel."""
    QPP = NT // BN
    assert BK % 4 == 0 and NT % BN == 0 and (BK // 4) % QPP == 0
    L = (BK // 4) * BN // NT
    tid = np.arange(NT)
    col, q0 = tid % BN, tid // BN
    c = np.minimum(c0 + col, N - 1)
    rows, cols, ok, seen = [], [], [], []
    for l in range(L):
        q = q0 + l * QPP
        assert (q * 4 + 4).max() <= BK and (col * (BK + 4) + q * 4 + 4).max() <= BN * (BK + 4)
        for t in range(4):
            k = k0 + 4 * q + t
            rows.append(k)
            cols.append(c)
            ok.append(k < K)
            seen.append((4 * q + t) * BN + col)
    seen = np.concatenate(seen)
    assert np.array_equal(np.sort(seen), np.arange(BK * BN))
    return np.concatenate(rows), np.concatenate(cols), 1, np.concatenate(ok)


def check_loads_in_bounds(v, M, N, K):
    """Loads of every A and B panel stay inside the STORED operand: A is M x K, or K x M when the
    variant reads it transposed (a BK x BM panel whose columns past M are clamped); B is K x N, or
    N x K when transposed (a BN x BK panel whose rows past N are clamped)."""
    # split-K variants: each k-group loads its slabs with its own threads (threads / ksplit)
    BM, BN, BK, NT, vec = v["BM"], v["BN"], v["BK"], v["threads"] // v["ksplit"], bool(v["vec"])
    ta, tb = v.get("trans_a", 0), v.get("trans_b", 0)
    tiles_m, tiles_n = -(-M // BM), -(-N // BN)
    nslab = -(-K // BK)
    for tm in range(tiles_m):
        for s in range(nslab):
            if ta:
                r, c, W, ok = panel_loads(BK, BM, NT, vec, s * BK, tm * BM, K, M, False, True)
                rows, cols = K, M
            else:
                r, c, W, ok = panel_loads(BM, BK, NT, vec, tm * BM, s * BK, M, K, True, False)
                rows, cols = M, K
            r, c = r[ok], c[ok]
            assert (r >= 0).all() and (r < rows).all() and (c >= 0).all() and (c + W <= cols).all()
    for tn in range(tiles_n):
        for s in range(nslab):
            if tb:
                r, c, W, ok = panel_loads(BN, BK, NT, vec, tn * BN, s * BK, N, K, True, False)
                rows, cols = N, K
            elif v.get("b_kquad"):
                r, c, W, ok = kquad_loads(BK, BN, NT, s * BK, tn * BN, K, N)
                rows, cols = K, N
            else:
                r, c, W, ok = panel_loads(BK, BN, NT, vec, s * BK, tn * BN, K, N, False, True)
                rows, cols = K, N
            r, c = r[ok], c[ok]
            assert (r >= 0).all() and (r < rows).all() and (c >= 0).all() and (c + W <= cols).all()


def mfma_block(v):
    """Edge of a variant's MFMA blocks (32 or 16)."""
    return v.get("mfma_block") or 32


def stored_elements(v, M, N):
    """All (row, col) the epilogue stores, over every workgroup of the launch.

    In split-K variants only k-group 0 (the first threads / ksplit threads) stores."""
    BM, BN, NT = v["BM"], v["BN"], v["threads"] // v["ksplit"]
    tiles_m, tiles_n = -(-M // BM), -(-N // BN)
    # the launches group min(tiles_m, 4) tile-rows (group_rows in csrc/sgemm_launch.hpp)
    tm_of, tn_of = _binding.tile_order(tiles_m, tiles_n, min(tiles_m, 4))
    tid = np.arange(NT)
    rows_all, cols_all = [], []
    if v["kind"] == "mfma":
        WM, WN = v["WM_or_TM"], v["WN_or_TN"]
        waves_n = BN // WN
        lane, wave = tid % 64, tid // 64
        wm0, wn0 = (wave // waves_n) * WM, (wave % waves_n) * WN
        local = []
        if mfma_block(v) == 32:
            li, lh = lane % 32, lane // 32
            for i, j, r in itertools.product(range(WM // 32), range(WN // 32), range(16)):
                if v["vec"]:
                    # blocks accumulated transposed: register r holds row li, column 8*(r/4) + 4*lh + r%4
                    local.append((wm0 + i * 32 + li, wn0 + j * 32 + (r // 4) * 8 + lh * 4 + (r % 4)))
                else:
                    # upright blocks: register r holds row 8*(r/4) + 4*lh + r%4, column li
                    local.append((wm0 + i * 32 + (r // 4) * 8 + lh * 4 + (r % 4), wn0 + j * 32 + li))
        else:
            li, lh = lane % 16, lane // 16
            for i, j, r in itertools.product(range(WM // 16), range(WN // 16), range(4)):
                if v["vec"]:
                    # 16x16 blocks transposed: register r holds row li, column 4*lh + r
                    local.append((wm0 + i * 16 + li, wn0 + j * 16 + 4 * lh + r))
                else:
                    # upright: register r holds row 4*lh + r, column li
                    local.append((wm0 + i * 16 + 4 * lh + r, wn0 + j * 16 + li))
    else:
        TM, TN = v["WM_or_TM"], v["WN_or_TN"]
        TX = BN // TN
        SM, SN = BM // (TM // 4), BN // (TN // 4)
        tx, ty = tid % TX, tid // TX
        local = []
        for i, j in itertools.product(range(TM), range(TN)):
            local.append(((i // 4) * SM + ty * 4 + (i % 4), (j // 4) * SN + tx * 4 + (j % 4)))
    lr = np.concatenate([a for a, _ in local])
    lc = np.concatenate([b for _, b in local])
    for w in range(tiles_m * tiles_n):
        r = tm_of[w] * BM + lr
        c = tn_of[w] * BN + lc
        keep = (r < M) & (c < N)
        rows_all.append(r[keep])
        cols_all.append(c[keep])
    return np.concatenate(rows_all), np.concatenate(cols_all)


SHAPES = [(1, 1, 1), (1, 4, 4), (4, 1, 4), (33, 65, 9), (128, 128, 16), (129, 131, 17), (64, 64, 64),
          (257, 65, 33), (300, 260, 77), (65, 300, 8), (256, 64, 1024), (130, 68, 12), (4, 4, 4),
          (132, 132, 20), (68, 260, 36)]


def is_direct(v):
    """The LDS-free kernel (one wave per 32x32 tile, operands loaded straight into registers):
    its loads follow the MFMA operand layout, not the panel loader's, and have their own model."""
    return v["name"].startswith("mfma32r_")


@pytest.mark.parametrize("v", VARIANTS, ids=[v["name"] for v in VARIANTS])
def test_loads_in_bounds(v):
    if is_direct(v):
        pytest.skip("covered by test_direct_kernel_loads_in_bounds")
    if v.get("dl_stages"):
        pytest.skip("covered by test_dl_kernel_loads_and_fragments")
    for (M, N, K) in SHAPES:
        a_len = M if v["trans_a"] else K   # stored row lengths
        b_len = K if v["trans_b"] else N
        if v["vec"] and (N % 4 or a_len % 4 or b_len % 4):
            continue  # the variant refuses these shapes
        check_loads_in_bounds(v, M, N, K)


@pytest.mark.parametrize("v", VARIANTS, ids=[v["name"] for v in VARIANTS])
def test_every_output_stored_exactly_once(v):
    for (M, N, _) in SHAPES:
        r, c = stored_elements(v, M, N)
        assert (r >= 0).all() and (r < M).all() and (c >= 0).all() and (c < N).all()
        flat = r.astype(np.int64) * N + c
        counts = np.bincount(flat, minlength=M * N)
        assert counts.min() == 1 and counts.max() == 1, (v["name"], M, N)


def c_reads(v, M, N, ldc):
    """For every register of every MFMA block the epilogue handles (mfma_block_c / mfma16_block_c
    restated): the (row, col) it would store and the (row, col) its beta-term read loads, and
    the read's byte offset from its row base where the 32-bit form applies (ldc < 2^25).  Arrays
    over (block, lane), one entry per register."""
    BM, BN, NT = v["BM"], v["BN"], v["threads"] // v["ksplit"]
    WM, WN = v["WM_or_TM"], v["WN_or_TN"]
    MB = mfma_block(v)
    waves_n = BN // WN
    r0s, c0s = [], []
    for tm, tn in itertools.product(range(-(-M // BM)), range(-(-N // BN))):
        for wave in range(NT // 64):
            wm0, wn0 = (wave // waves_n) * WM, (wave % waves_n) * WN
            for i, j in itertools.product(range(WM // MB), range(WN // MB)):
                r0s.append(tm * BM + wm0 + i * MB)
                c0s.append(tn * BN + wn0 + j * MB)
    r0 = np.array(r0s)[:, None]
    c0 = np.array(c0s)[:, None]
    lane = np.arange(64)[None, :]
    li, lh = lane % MB, lane // MB
    rb = np.minimum(r0, M - 1)
    rlim, rd = M - 1 - rb, r0 - rb
    out = []
    for r in range(MB * MB // 64):
        if MB == 32 and v["vec"]:
            srow, scol = r0 + li, c0 + (r // 4) * 8 + lh * 4 + r % 4
            rr = np.minimum(rd + li, rlim)
            col = np.minimum(c0 + (r // 4) * 8 + lh * 4, N - 4) + r % 4
        elif MB == 32:
            srow, scol = r0 + (r // 4) * 8 + r % 4 + 4 * lh, c0 + li
            rr = np.minimum(rd + (r // 4) * 8 + r % 4 + 4 * lh, rlim)
            col = np.minimum(c0 + li, N - 1)
        elif v["vec"]:
            srow, scol = r0 + li, c0 + 4 * lh + r
            rr = np.minimum(rd + li, rlim)
            col = np.minimum(c0 + 4 * lh, N - 4) + r
        else:
            srow, scol = r0 + 4 * lh + r, c0 + li
            rr = np.minimum(rd + 4 * lh + r, rlim)
            col = np.minimum(c0 + li, N - 1)
        off = (rr.astype(np.int64) * ldc + col) * 4 if ldc < (1 << 25) else None
        out.append((srow, scol, rb + rr, np.broadcast_to(col, srow.shape), off))
    return out


@pytest.mark.parametrize("v", [v for v in VARIANTS if v["kind"] == "mfma"],
                         ids=[v["name"] for v in VARIANTS if v["kind"] == "mfma"])
def test_epilogue_c_reads_in_bounds(v):
    """The beta term's reads of C never leave the matrix (rows and columns clamped at an edge,
    a row base inside the matrix even for a block wholly below it), read exactly the element the
    same register stores wherever that element exists, and keep the 32-bit offsets of the
    ldc < 2^25 form non-negative and under 2^32."""
    cases = [(M, N, ldc) for (M, N, _) in SHAPES for ldc in (N, N + 4 if v["vec"] else N + 3)]
    cases += [(M, N, ldc) for (M, N, _) in SHAPES[3:8] for ldc in ((1 << 25) - 4, (1 << 25) + 4)]
    for M, N, ldc in cases:
        if v["vec"] and N % 4:
            continue
        for srow, scol, row, col, off in c_reads(v, M, N, ldc):
            assert (row >= 0).all() and (row < M).all() and (col >= 0).all() and (col < N).all()
            inside = (srow < M) & (scol < N)
            assert (row[inside] == srow[inside]).all() and (col[inside] == scol[inside]).all()
            if off is not None:
                assert (off >= 0).all() and (off < (1 << 32)).all()


@pytest.mark.parametrize("ks", [2, 4])
@pytest.mark.parametrize("K,BK", [(1, 16), (16, 16), (17, 16), (777, 16), (96, 32), (4096, 32)])
def test_splitk_slab_assignment_covers_k_once(ks, K, BK):
    """Group g multiplies slabs g, g+KS, ... for ceil(nslab/KS) steps; slabs past K load zeros.
    Every slab below nslab is taken by exactly one (step, group)."""
    nslab = -(-K // BK)
    niter = -(-nslab // ks)
    taken = [i * ks + g for i in range(niter) for g in range(ks)]
    real = [t for t in taken if t < nslab]
    assert sorted(real) == list(range(nslab))
    assert len(taken) - len(real) < ks


@pytest.mark.parametrize("BK", [8, 16, 32])
def test_mfma_k_mapping_covers_slab_once(BK):
    """Group kk, step t, half h uses k = 8*kk + 4*h + t for both operands: each k in the slab once."""
    ks = [8 * kk + 4 * h + t for kk in range(BK // 8) for t in range(4) for h in range(2)]
    assert sorted(ks) == list(range(BK))


DIRECT = [v for v in VARIANTS if is_direct(v)]


@pytest.mark.parametrize("v", DIRECT, ids=[v["name"] for v in DIRECT])
def test_direct_kernel_loads_in_bounds(v):
    """sgemm_mfma_direct_kernel's addressing, restated: lane (i, h) of the wave owning tile
    (m0, n0) reads A(min(m0+i, M-1), k) and B(k, min(n0+i, N-1)) for k = 8q + 4h + t of every
    group q < ceil(K/8) (in the ring's last trips, groups past the end too); in the tail, k past
    K is read at k = K-1 (K-4 for the 128-bit A load) and the value replaced by zero.  Every
    element read must lie inside the operand; every k < K must be read for every row/column."""
    D = v["BK"] // 16
    vec = bool(v["vec"])
    for (M, N, K) in SHAPES + [(64, 64, 8 * D), (33, 35, 16 * D + 5), (40, 64, 24 * D + 4)]:
        if vec and (N % 4 or K % 4):
            continue
        ngroups, nfull = -(-K // 8), K // 8
        # groups loaded: the prologue's D, then D per trip while q + D < ngroups
        loaded = set(range(D))
        q = 0
        while q + 2 * D <= nfull:
            loaded |= set(range(q + D, q + 2 * D))
            q += D
        while q + D < ngroups:
            loaded |= set(range(q + D, q + 2 * D))
            q += D
        consumed = set(range(q + D))  # every trip's slots, and the final D
        assert set(range(ngroups)) <= consumed <= loaded
        ks_a, ks_b = [], []
        for g in sorted(loaded):
            for h in range(2):
                kb = 8 * g + 4 * h
                if vec:
                    ka = min(kb, K - 4) if kb >= K or g >= nfull else kb
                    ks_a += [ka + t for t in range(4)]
                    ok = kb < K
                    assert ok or all(kb + t >= K for t in range(4))
                else:
                    ks_a += [min(kb + t, K - 1) if g >= nfull else kb + t for t in range(4)]
                ks_b += [min(kb + t, K - 1) if g >= nfull else kb + t for t in range(4)]
        ks_a, ks_b = np.array(ks_a), np.array(ks_b)
        assert ks_a.min() >= 0 and ks_a.max() < K and ks_b.min() >= 0 and ks_b.max() < K
        assert set(range(K)) <= set(ks_a.tolist()) and set(range(K)) <= set(ks_b.tolist())
        rows = np.minimum(np.arange(-(-M // 32) * 32), M - 1)
        cols = np.minimum(np.arange(-(-N // 32) * 32), N - 1)
        assert rows.max() < M and cols.max() < N


# ------------------------------------------------------------------------------------------
# the direct-to-LDS kernel (sgemm_mfma_dl_kernel): swizzled 16-byte loads straight into LDS
# ------------------------------------------------------------------------------------------

def dl_swz_a(r, qpr, mb=32):
    r = np.asarray(r)
    if mb == 16:
        return r & 15 if qpr == 16 else (r >> 1) & 7 if qpr == 8 else ((r >> 3) & 1) * 2
    if qpr == 16:
        return r & 15
    return ((r & 15) + ((r >> 3) & 1)) & 7 if qpr == 8 else (((r >> 1) & 7) + ((r >> 3) & 1)) & 3


def dl_swz_b(k, mb=32):
    """B row k's swizzle in quads for MFMA blocks of edge mb: column flip of mb * ((k >> 2) % G),
    G = 64 / mb lane groups."""
    return ((np.asarray(k) >> 2) & (64 // mb - 1)) * (mb // 4)


def dl_brow(k, bn):
    """The LDS row that holds B row k of a stage: rows of 32 floats trade rows 4-7 of every 8 in
    pairs (k ^ ((k >> 2) & 1)); wider rows keep k."""
    k = np.asarray(k)
    return k ^ ((k >> 2) & 1) if bn == 32 else k


def dl_b_read_offset(k, n, bn, mb, lh):
    """Float offset, in a B stage, of the fragment read of B row k (of the stage), column n (of the
    tile) by lane group lh: the column-flipped layout, or the row-permuted one for 32-float rows."""
    if bn == 32:
        return dl_brow(k, bn) * bn + n
    return k * bn + (n ^ (mb * lh))



DL = [v for v in VARIANTS if v.get("dl_stages")]


def dl_slab_model(v, M, N, K, tm, tn, s):
    """One slab of one workgroup of sgemm_mfma_dl_kernel, restated: returns the LDS contents of
    the A and B stages as the global (row, col) each element holds (-1 for a zeroed element past
    K), after every wave's loads and the tail fix-up.  Asserts every load address is inside the
    operand.  128-bit variants load W = 16 bytes per lane (a quad), 32-bit ones W = 4."""
    BM, BN, BK, NT = v["BM"], v["BN"], v["BK"], v["threads"]
    NW = NT // 64
    MB = mfma_block(v)
    E = 4 if v["vec"] else 1          # floats per lane load
    CH = 64 * E                       # floats one wave's load fills
    QA = BK // 4
    LA, LB = BM * BK // CH // NW, BK * BN // CH // NW
    m0, n0, k0 = tm * BM, tn * BN, s * BK
    tail = k0 + BK > K
    lane = np.arange(64)
    a_lds = np.full((BM * BK, 2), -2, dtype=np.int64)
    b_lds = np.full((BK * BN, 2), -2, dtype=np.int64)
    for wave in range(NW):
        for j in range(LA):
            f = (wave * LA + j) * CH + E * lane
            r = f // BK
            u = (f % BK) // 4
            kin = 4 * (u ^ dl_swz_a(r, QA, MB)) + f % 4
            row = np.minimum(m0 + r, M - 1)
            k = k0 + kin
            kl = np.minimum(k, K - E) if tail else k
            assert (row >= 0).all() and (row < M).all() and (kl >= 0).all() and (kl + E <= K).all()
            for e in range(E):
                a_lds[f + e, 0] = np.where(k < K, row, -1)
                a_lds[f + e, 1] = np.where(k < K, kl + e, -1)
        for j in range(LB):
            f = (wave * LB + j) * CH + E * lane
            kr = f // BN
            u = (f % BN) // 4
            n = np.minimum(n0 + 4 * (u if BN == 32 else u ^ dl_swz_b(kr, MB)) + f % 4, N - E)
            k = k0 + dl_brow(kr, BN)
            kl = np.minimum(k, K - 1) if tail else k
            assert (kl >= 0).all() and (kl < K).all() and (n >= 0).all() and (n + E <= N).all()
            for e in range(E):
                b_lds[f + e, 0] = np.where(k < K, kl, -1)
                b_lds[f + e, 1] = np.where(k < K, n + e, -1)
    assert (a_lds >= -1).all() and (b_lds >= -1).all()  # every LDS element written
    return a_lds, b_lds


@pytest.mark.parametrize("v", DL, ids=[v["name"] for v in DL])
def test_dl_kernel_loads_and_fragments(v):
    """sgemm_mfma_dl_kernel's loads stay inside A and B (rows past M and columns past N clamped, k
    of the slab that crosses K clamped), every LDS element of a stage is written, and the fragment
    read of lane (i, h) (i = lane % MB, h = lane / MB for MFMA blocks of edge MB), block (fi, fj),
    fragment group kk and step t -- at the kernel's swizzled offsets -- returns
    A(m0 + wm0 + MB fi + i, k) and B(k, n0 + wn0 + MB fj + i) with k = k0 + KG kk + 4 h + t
    (KG = 4 * 64 / MB; rows/columns clamped at the edges), or a zero past K."""
    BM, BN, BK, NT = v["BM"], v["BN"], v["BK"], v["threads"]
    WM, WN = v["WM_or_TM"], v["WN_or_TN"]
    MB = mfma_block(v)
    G, KG = 64 // MB, 4 * 64 // MB
    waves_n = BN // WN
    QA = BK // 4
    lane = np.arange(64)
    li, lh = lane % MB, lane // MB
    for (M, N, K) in [(64, 64, 32), (200, 136, 100), (131, 68, 36), (257, 260, 8), (1, 4, 4), (70, 67, 37),
                      (3, 130, 1), (129, 65, 130)]:
        if v["vec"] and (N % 4 or K % 4):
            continue
        tiles_m, tiles_n = -(-M // BM), -(-N // BN)
        for tm in {0, tiles_m - 1}:
            for tn in {0, tiles_n - 1}:
                for s in range(-(-K // BK)):
                    a_lds, b_lds = dl_slab_model(v, M, N, K, tm, tn, s)
                    k0 = s * BK
                    for wave in range(NT // 64):
                        wm0, wn0 = (wave // waves_n) * WM, (wave % waves_n) * WN
                        for kk in range(BK // KG):
                            a_frag = (wm0 + li) * BK + 4 * ((G * kk + lh) ^ dl_swz_a(wm0 + li, QA, MB))
                            for fi in range(WM // MB):
                                for t in range(4):
                                    got = a_lds[a_frag + fi * MB * BK + t]
                                    k = k0 + KG * kk + 4 * lh + t
                                    row = np.minimum(tm * BM + wm0 + MB * fi + li, M - 1)
                                    want_r = np.where(k < K, row, -1)
                                    want_k = np.where(k < K, k, -1)
                                    assert (got[:, 0] == want_r).all() and (got[:, 1] == want_k).all()
                            for fj in range(WN // MB):
                                for t in range(4):
                                    got = b_lds[dl_b_read_offset(KG * kk + 4 * lh + t, wn0 + fj * MB + li, BN, MB, lh)]
                                    k = k0 + KG * kk + 4 * lh + t
                                    col = np.minimum(tn * BN + wn0 + MB * fj + li, N - 1)
                                    # columns past N read a clamped column of the last 4-column
                                    # group (128-bit loads) or column N - 1 (32-bit loads)
                                    ok = (got[:, 1] == col) | \
                                         ((tn * BN + wn0 + MB * fj + li >= N) & (got[:, 1] >= N - 4))
                                    assert (np.where(k < K, ok, got[:, 1] == -1)).all()
                                    assert (got[:, 0] == np.where(k < K, k, -1)).all()


def test_dl_swizzles_are_row_permutations():
    for qpr in (4, 8, 16):
        for r in range(64):
            for mb in (32, 16):
                assert sorted((np.arange(qpr) ^ dl_swz_a(r, qpr, mb)).tolist()) == list(range(qpr))
    for mb in (32, 16):
        for k in range(64):
            assert sorted((np.arange(16) ^ dl_swz_b(k, mb)).tolist()) == list(range(16))
    # the 32-float rows' row permutation: a bijection of every 8 rows, its own inverse
    k = np.arange(64)
    assert sorted(dl_brow(k, 32).tolist()) == list(range(64)) and (dl_brow(dl_brow(k, 32), 32) == k).all()
    assert ((dl_brow(k, 32) >> 3) == (k >> 3)).all()


# How the LDS serves one access of 64 lanes (64 banks of 4 bytes), as measured on MI355X: two
# lanes reading different words of the same banks add conflict cycles exactly when they share a
# pass (SQ_LDS_BANK_CONFLICT over lane pairs, `python -m fp32_gemm_05_amd.profiling lds-passes`):
#   * 32-bit accesses: one pass of all 64 lanes;
#   * 64-bit accesses: two passes, lanes 0-31 and 32-63;
#   * 128-bit accesses: four passes of 16 lanes -- the lanes of one half-wave whose bits 2-4 have
#     the same parity (lanes 0-3, 12-15, 20-23, 24-27 / 4-11, 16-19, 28-31 / the same + 32).
# ds_read2st64_b32 goes through as two 32-bit accesses (its two words per lane are 64 words apart,
# the same bank, and the 32x32 kernels that use it measure no conflict cycles).
def lds_passes(width):
    lane = np.arange(64)
    if width == 16:
        par = np.array([bin(int(x) >> 2 & 7).count("1") & 1 for x in lane])
        return [list(lane[(lane >> 5 == h) & (par == p)]) for h in (0, 1) for p in (0, 1)]
    if width == 8:
        return [list(range(32)), list(range(32, 64))]
    return [list(range(64))]


def lds_extra_cycles(addr_bytes, width):
    """Bank-conflict cycles of one LDS access by 64 lanes: per pass, the largest number of distinct
    4-byte words one bank must serve, minus one, summed over the passes."""
    extra = 0
    for lanes in lds_passes(width):
        words = {}
        for ln in lanes:
            for w in range(width // 4):
                word = int(addr_bytes[ln]) // 4 + w
                words.setdefault(word % 64, set()).add(word)
        extra += max(len(x) for x in words.values()) - 1
    return extra


def dl_fragment_addresses(v, swz_a=dl_swz_a):
    """Byte addresses of every fragment read of sgemm_mfma_dl_kernel, one 64-lane array per read:
    ("a", addresses) for the 128-bit A reads and ("b", ...) for the 32-bit B reads (rows
    KG kk + 4 h + t of the lane groups at MB consecutive columns)."""
    BN, BK, WM, WN = v["BN"], v["BK"], v["WM_or_TM"], v["WN_or_TN"]
    MB = mfma_block(v)
    G, KG = 64 // MB, 4 * 64 // MB
    lane = np.arange(64)
    li, lh = lane % MB, lane // MB
    out = []
    for wave in range(v["threads"] // 64):
        wm0, wn0 = (wave // (BN // WN)) * WM, (wave % (BN // WN)) * WN
        for kk in range(BK // KG):
            for fi in range(WM // MB):
                out.append(("a", 4 * ((wm0 + li + MB * fi) * BK + 4 * ((G * kk + lh) ^ swz_a(wm0 + li, BK // 4, MB)))))
            for fj in range(WN // MB):
                for t in range(4):
                    out.append(("b", 4 * dl_b_read_offset(KG * kk + 4 * lh + t, wn0 + fj * MB + li, BN, MB, lh)))
    return out


@pytest.mark.parametrize("v", DL, ids=[v["name"] for v in DL])
def test_dl_fragment_reads_are_conflict_free(v):
    """Every fragment read of sgemm_mfma_dl_kernel is free of bank conflicts under the measured
    pass grouping."""
    for kind, addr in dl_fragment_addresses(v):
        assert lds_extra_cycles(addr, 16 if kind == "a" else 4) == 0, kind


def test_lds_bank_model_matches_measured_conflicts():
    """The pass model reproduces SQ_LDS_BANK_CONFLICT as measured on MI355X (the counter summaries of
    the kernels):
      * the 32x32-block direct-load kernels: 0 conflict cycles;
      * the 16x16-block kernel with the 32x32 blocks' A swizzle: 16384 cycles over 8192 LDS
        instructions on 256^3 (half of them 128-bit A reads), and the same count again after lane
        groups 1 and 2 swapped their k-quads -- 4 extra cycles per A read either way;
      * the plain kernel (128x128x16 tiles, A rows of BK + 4 = 20 floats, B rows of BN + 8): exactly
        1 conflict cycle per LDS instruction on 4096^3 -- its two 128-bit A stores per wave and slab
        take 8 each, and the other 14 of the wave's 16 LDS instructions (A reads, B stores and B
        reads) none."""
    by_name = {v["name"]: v for v in DL}
    for n in ("mfma32l_128x128x16_w64x64_s4_d3_vec", "mfma32l_64x64x32_w32x32_s3_cp_sp_vec",
              "mfma32l_64x64x16_w32x32_s3_sp_scalar"):
        assert all(lds_extra_cycles(a, 16 if k == "a" else 4) == 0 for k, a in dl_fragment_addresses(by_name[n]))
    v16 = by_name["mfma16l_64x64x32_w32x16_s3_cp_sp_vec"]
    swz32 = lambda r, qpr, mb: dl_swz_a(r, qpr, 32)  # the 32x32 blocks' swizzle
    old = dl_fragment_addresses(v16, swz_a=swz32)
    assert {lds_extra_cycles(a, 16) for k, a in old if k == "a"} == {4}
    assert {lds_extra_cycles(a, 4) for k, a in old if k == "b"} == {0}
    lane = np.arange(64)
    li, lh = lane % 16, lane // 16
    for kk in range(2):  # lane groups 1 and 2 swapped
        q = ((lh & 1) << 1) | (lh >> 1)
        for fi in range(2):
            a = 4 * ((li + 16 * fi) * 32 + 4 * ((4 * kk + q) ^ dl_swz_a(li, 8, 32)))
            assert lds_extra_cycles(a, 16) == 4
    # the plain kernel: A stores, thread t -> row t / 4 (+ 64 per pass), quad t % 4, rows of 20
    # floats; B stores, thread t -> row t / 32, quad t % 32, rows of 136; A reads row li + 32 i at
    # quad 2 kk + h; B reads row 4 h + t (+ 8 kk) at column li (+ 32 j)
    li, lh = lane % 32, lane // 32
    for wave in range(4):
        tid = 64 * wave + lane
        for l in range(2):
            assert lds_extra_cycles(4 * ((tid // 4 + 64 * l) * 20 + 4 * (tid % 4)), 16) == 8
            assert lds_extra_cycles(4 * ((tid // 32 + 8 * l) * 136 + 4 * (tid % 32)), 16) == 0
    for kk in range(2):
        for i in range(4):
            assert lds_extra_cycles(4 * ((li + 32 * i) * 20 + 4 * (2 * kk + lh)), 16) == 0
        for t in range(4):
            assert lds_extra_cycles(4 * ((8 * kk + 4 * lh + t) * 136 + li), 4) == 0


def test_lds_bank_model_sees_a_b_conflict():
    """The bank model reports the conflict of an unswizzled 16x16 B read (rows 4 h + t of four lane
    groups at the same 16 columns of 64-float rows share their banks)."""
    lane = np.arange(64)
    b = 4 * ((4 * (lane // 16)) * 64 + lane % 16)
    assert lds_extra_cycles(b, 4) == 3


# ------------------------------------------------------------------------------------------
# the direct-to-LDS ring: the order of requests, waits, tail fix-ups, barriers and reads
# ------------------------------------------------------------------------------------------

def dl_ring_events(stages, nslab, nfull, mine):
    """The sequence of ring operations one wave of sgemm_mfma_dl_kernel (mine = 1) or of the
    persistent sgemm_mfma_dlp_kernel performs, restated: ("issue", gs), ("wait", n) -- at most n
    slabs' loads still in flight --, ("fix", gs), ("barrier",), ("read", gs) and ("epilogue", i).
    Slab gs is slab gs % nslab of tile gs // nslab; its loads land in stage gs % stages."""
    D = stages - 1
    total = mine * nslab
    ev = []
    for gs in range(D):
        if gs < total:
            ev.append(("issue", gs))
    ev.append(("wait", min(D, total) - 1))
    if nfull == 0:
        ev.append(("fix", 0))
        ev.append(("wait", 0))
    ev.append(("barrier",))
    ev.append(("read", 0))
    for gs in range(total):
        if gs + D < total:
            ev.append(("issue", gs + D))
        ev.append(("read", gs))           # the slab's remaining 8-deep groups
        if gs + 1 < total:
            ev.append(("wait", min(gs + D, total - 1) - (gs + 1)))
            if (gs + 1) % nslab >= nfull:
                ev.append(("fix", gs + 1))
                ev.append(("wait", 0))
            ev.append(("barrier",))
            ev.append(("read", gs + 1))   # the next slab's first group
        if gs % nslab == nslab - 1:
            ev.append(("epilogue", gs // nslab))
    return ev


def dl_ring_events_eb(stages, nslab, nfull, KK, P):
    """The same for the early-barrier form (EB = P) of sgemm_mfma_dl_kernel, one tile: the whole
    ring requested up front; in slab s, P fragment groups before its end, the wait for slab s + 1,
    its fix-up, the barrier and the request of slab s + STAGES; fragment groups read P ahead of
    their MFMAs, so ("read", t) once per 8-deep group of slab t."""
    ev = []
    for t in range(min(stages, nslab)):
        ev.append(("issue", t))
    ev.append(("wait", min(stages, nslab) - 1))
    if nfull == 0:
        ev.append(("fix", 0))
        ev.append(("wait", 0))
    ev.append(("barrier",))
    for q in range(P):
        ev.append(("read", 0))
    for s in range(nslab):
        for kk in range(KK):
            if kk == KK - P and s + 1 < nslab:
                ev.append(("wait", min(s + stages - 1, nslab - 1) - (s + 1)))
                if s + 1 >= nfull:
                    ev.append(("fix", s + 1))
                    ev.append(("wait", 0))
                ev.append(("barrier",))
                if s + stages < nslab:
                    ev.append(("issue", s + stages))
            g = s * KK + kk + P
            if g < nslab * KK:
                ev.append(("read", g // KK))
    ev.append(("epilogue", 0))
    return ev


def check_dl_ring(stages, nslab, nfull, mine, ev=None):
    """Every wave runs the same sequence, so a barrier orders each wave's operations before it
    against every wave's operations after it.  Checks: a slab's loads have landed (and, if it
    crosses K, been fixed up) before the barrier that precedes its first read; a stage is requested
    again only after a barrier that follows the last read of its previous slab; every slab is
    requested once, and read; the epilogues come once per tile, in order."""
    if ev is None:
        ev = dl_ring_events(stages, nslab, nfull, mine)
    total = mine * nslab
    inflight, landed, fixed = [], set(), set()
    landed_at, fixed_at = {}, {}
    last_read = {}          # slab -> index of its last read
    last_barrier = -1
    stage_of_req = {}       # stage -> slab last requested into it
    requested, epis = [], []
    for idx, e in enumerate(ev):
        kind = e[0]
        if kind == "issue":
            gs = e[1]
            st = gs % stages
            prev = stage_of_req.get(st)
            if prev is not None:
                assert prev in last_read and last_read[prev] < last_barrier, (stages, nslab, nfull, mine, gs)
            stage_of_req[st] = gs
            inflight.append(gs)
            requested.append(gs)
        elif kind == "wait":
            n = e[1]
            while len(inflight) > max(n, 0):
                gs = inflight.pop(0)
                landed.add(gs)
                landed_at[gs] = idx
        elif kind == "fix":
            assert e[1] in landed and e[1] % nslab >= nfull
            fixed.add(e[1])
            fixed_at[e[1]] = idx
        elif kind == "barrier":
            last_barrier = idx
        elif kind == "read":
            gs = e[1]
            assert gs in landed, (stages, nslab, nfull, mine, gs)
            if gs % nslab >= nfull:
                assert gs in fixed
            # every wave's loads (and fix-ups) of the slab are done before the last barrier
            if gs not in last_read:
                assert landed_at[gs] < last_barrier, (stages, nslab, nfull, mine, gs)
                if gs % nslab >= nfull:
                    assert fixed_at[gs] < last_barrier
            last_read[gs] = idx
        elif kind == "epilogue":
            epis.append(e[1])
    assert requested == list(range(total)) and set(last_read) == set(range(total))
    assert epis == list(range(mine))


@pytest.mark.parametrize("stages", [2, 3, 4])
def test_dl_ring_protocol(stages):
    for nslab in (1, 2, 3, 4, 5, 7, 9):
        for tail in (False, True):
            nfull = nslab - 1 if tail else nslab
            for mine in (1, 2, 3, 5):
                check_dl_ring(stages, nslab, nfull, mine)


@pytest.mark.parametrize("stages", [2, 3, 4])
def test_dl_ring_protocol_early_barrier(stages):
    """The early-barrier form for every P the kernel accepts (P < KK, (STAGES KK) % (P + 1) == 0)."""
    n = 0
    for KK in (1, 2, 4, 8):
        for P in range(1, KK):
            if (stages * KK) % (P + 1):
                continue
            for nslab in (1, 2, 3, 4, 5, 7, 9, 12):
                for tail in (False, True):
                    nfull = nslab - 1 if tail else nslab
                    check_dl_ring(stages, nslab, nfull, 1, dl_ring_events_eb(stages, nslab, nfull, KK, P))
                    n += 1
    assert n > 0


def test_dl_ring_early_barrier_model_catches_mistakes():
    """Requesting slab s + STAGES before the early barrier, or reading slab s + 1's first group
    before the barrier that publishes it, is caught."""
    ev = dl_ring_events_eb(3, 8, 8, 4, 2)
    i = next(k for k, e in enumerate(ev) if e[0] == "issue" and e[1] >= 3)
    j = max(k for k in range(i) if ev[k][0] == "barrier")
    with pytest.raises(AssertionError):
        check_dl_ring(3, 8, 8, 1, ev[:j] + [ev[i]] + ev[j:i] + ev[i + 1:])
    b = next(k for k, e in enumerate(ev) if e[0] == "barrier" and k > 6)  # the first one in the loop
    r = next(k for k in range(b, len(ev)) if ev[k] == ("read", 1))
    with pytest.raises(AssertionError):
        check_dl_ring(3, 8, 8, 1, ev[:b] + [ev[r]] + ev[b:r] + ev[r + 1:])


def test_dl_ring_model_catches_a_short_wait():
    """The check is not vacuous: waiting for one slab fewer than the kernel does, or requesting a
    stage one slab too early, is caught."""
    orig = globals()["dl_ring_events"]

    def short_wait(stages, nslab, nfull, mine):
        return [("wait", e[1] + 1) if e[0] == "wait" else e for e in orig(stages, nslab, nfull, mine)]

    def early_request(stages, nslab, nfull, mine):
        ev = orig(stages, nslab, nfull, mine)
        # move the first request that reuses a stage to before the preceding barrier
        i = next(k for k, e in enumerate(ev) if e[0] == "issue" and e[1] >= stages)
        j = max(k for k in range(i) if ev[k][0] == "barrier")
        return ev[:j] + [ev[i]] + ev[j:i] + ev[i + 1:]

    try:
        for bad in (short_wait, early_request):
            globals()["dl_ring_events"] = bad
            with pytest.raises(AssertionError):
                check_dl_ring(3, 6, 6, 2)
    finally:
        globals()["dl_ring_events"] = orig


@pytest.mark.parametrize("nt,grid", [(1, 1), (7, 7), (8, 3), (3713, 2048), (4096, 512), (1000, 1), (1024, 1000)])
def test_persistent_grid_stride_covers_tiles_once(nt, grid):
    """Workgroup w of the persistent kernel runs tiles w, w + G, ... for (nt - w + G - 1) // G
    tiles: every tile exactly once."""
    seen = []
    for w in range(grid):
        mine = (nt - w + grid - 1) // grid
        assert mine >= 1
        seen += [w + i * grid for i in range(mine)]
    assert sorted(seen) == list(range(nt))
