"""The early-barrier direct-load kernels (`_ebP` variants) on grids of many tiles and long K loops,
element by element against the oracle's full-matrix form: integer data exactly, random data within
the bound, with K tails (a slab that crosses K is fixed up before the barrier that publishes it),
beta != 0, odd leading dimensions for the 32-bit-load form, and sentinels around C.  (The reduced
parity cases have short K loops, where the early barrier's fast loop runs few trips.)
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


def _eb_variants():
    out = []
    for i in range(sg.sgemm_num_variants()):
        info = sg.sgemm_variant_info(i)
        if "_eb" in info["name"]:
            out.append((i, info["name"], bool(info["vec"])))
    return out


EB = _eb_variants()
# (M, N, K, alpha, beta, int data): K from one slab past the ring to several hundred slabs
CASES = [(1536, 2048, 1000, 1.0, 0.0, True), (777, 1000, 1364, 0.5, -1.5, False), (640, 704, 6144, 1.0, 0.5, True),
         (1100, 900, 132, 1.0, 1.0, True)]


@pytest.mark.parametrize("vid,name,vec", EB, ids=[p[1] for p in EB])
@pytest.mark.parametrize("M,N,K,alpha,beta,ints", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in CASES])
def test_early_barrier_elementwise(vid, name, vec, M, N, K, alpha, beta, ints):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    if vec and (N % 4 or K % 4):
        pytest.skip("128-bit variant: needs N and K multiples of 4")
    _say(f"[eb] {name} {M}x{N}x{K} alpha={alpha} beta={beta} ints={ints}")
    rng = np.random.default_rng(M + 5 * N + 11 * K)
    if ints:
        A = rng.integers(-2, 3, (M, K)).astype(np.float32)
        B = rng.integers(-2, 3, (K, N)).astype(np.float32)
        C = rng.integers(-2, 3, (M, N)).astype(np.float32)
    else:
        A = rng.standard_normal((M, K), dtype=np.float32)
        B = rng.standard_normal((K, N), dtype=np.float32)
        C = rng.standard_normal((M, N), dtype=np.float32)
    lda, ldb = (K, N) if vec else (K | 1, N | 1)
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
        _say(f"[eb] max err/bound {worst:.3g}")
