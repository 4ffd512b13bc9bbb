"""The persistent direct-load kernels (`_ps` variants) on grids with more tiles than resident slots,
so that every workgroup runs several tiles through one LDS ring sequence: every element of C
against the oracle's full-matrix form, integer data exactly, with a K tail, beta != 0, and
sentinels around C.  (The reduced parity cases have at most 256 tiles, which every workgroup
covers with one tile.)
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from fp32_gemm_05_amd import _binding as sg  # noqa: E402
from gemm_cases import SENTINEL, assert_border_untouched, check_exact, check_within_bound, device_matrix  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _persistent_variants():
    out = []
    for i in range(sg.sgemm_num_variants()):
        info = sg.sgemm_variant_info(i)
        if info.get("persistent"):
            out.append((i, info["name"], bool(info["vec"])))
    return out


PS = _persistent_variants()
# (M, N, K, alpha, beta, int data): tiles of 64x64 / 128x64 / 128x128 well above the 512-1536 slots
CASES = [(4096, 2048, 200, 1.0, 0.0, True), (3001, 2003, 131, 0.5, -1.5, False), (2048, 4096, 64, 1.0, 0.5, True)]


@pytest.mark.parametrize("vid,name,vec", PS, ids=[p[1] for p in PS])
@pytest.mark.parametrize("M,N,K,alpha,beta,ints", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in CASES])
def test_persistent_multi_tile_elementwise(vid, name, vec, M, N, K, alpha, beta, ints):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    if vec and (N % 4 or K % 4):
        pytest.skip("128-bit variant: needs N and K multiples of 4")
    info = sg.sgemm_variant_info(vid)
    tiles = -(-M // info["BM"]) * -(-N // info["BN"])
    _say(f"[ps] {name} {M}x{N}x{K} alpha={alpha} beta={beta} ints={ints} tiles={tiles}")
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    if ints:
        A = rng.integers(-2, 3, (M, K)).astype(np.float32)
        B = rng.integers(-2, 3, (K, N)).astype(np.float32)
        C = rng.integers(-2, 3, (M, N)).astype(np.float32)
    else:
        A = rng.standard_normal((M, K), dtype=np.float32)
        B = rng.standard_normal((K, N), dtype=np.float32)
        C = rng.standard_normal((M, N), dtype=np.float32)
    if not vec:  # odd leading dimensions: the 32-bit-load forms' own precondition
        lda, ldb = K | 1, N | 1
    else:
        lda, ldb = K, N
    dA = torch.zeros((M, lda), dtype=torch.float32, device="cuda")
    dB = torch.zeros((K, ldb), dtype=torch.float32, device="cuda")
    dA[:, :K] = torch.from_numpy(A).cuda()
    dB[:, :N] = torch.from_numpy(B).cuda()
    bufC, vC, ldc = device_matrix(C, pad_cols=4 if vec else 5, pad_rows=2, fill=SENTINEL)
    sg.sgemm_ex(M, N, K, alpha, dA, lda, dB, ldb, beta, vC, ldc, variant=vid)
    assert sg.sgemm_last_variant() == vid
    torch.cuda.synchronize()
    host = bufC.cpu().numpy()
    assert_border_untouched(host, M, N, ldc, what=name)
    got = host[: M * ldc].reshape(M, ldc)[:, :N]
    ref, bound = oracle.ref_matmul(A, B, C, alpha, beta)
    if ints:
        check_exact(got, ref, name)
    else:
        worst = check_within_bound(got, ref, bound, name)
        _say(f"[ps] max err/bound {worst:.3g}")
