"""Host model of the kernels' index math: every global load stays inside the operand,
every output element of C is stored exactly once, nothing outside C's M x N window
is stored, and each MFMA accumulator receives every k of a slab exactly once.

The model restates, in numpy, the addressing of sgemm_kernels.hpp (PanelLoader,
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
            else:
                r, c, W, ok = panel_loads(BK, BN, NT, vec, s * BK, tn * BN, K, N, False, True)
                rows, cols = K, N
            r, c = r[ok], c[ok]
            assert (r >= 0).all() and (r < rows).all() and (c >= 0).all() and (c + W <= cols).all()


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
        li, lh = lane % 32, lane // 32
        local = []
        for i, j, r in itertools.product(range(WM // 32), range(WN // 32), range(16)):
            if v["vec"]:
                # blocks accumulated transposed: register r holds row li, column 8*(r/4) + 4*lh + r%4
                local.append((wm0 + i * 32 + li, wn0 + j * 32 + (r // 4) * 8 + lh * 4 + (r % 4)))
            else:
                # upright blocks: register r holds row 8*(r/4) + 4*lh + r%4, column li
                local.append((wm0 + i * 32 + (r // 4) * 8 + lh * 4 + (r % 4), wn0 + j * 32 + li))
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
