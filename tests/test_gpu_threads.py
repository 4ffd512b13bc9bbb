"""Concurrent calls: several host threads, each with its own HIP stream, call the library at once.

The header promises thread safety: the library's only global state (the dispatch table, each
kernel's occupancy, the device's compute-unit count) is computed once on first use and read-only
afterwards.  Each thread runs a mix of plain and transposed calls from several shape classes on its
own stream; every result must equal, bit for bit, the same call run alone beforehand (the kernels
are deterministic), and after each call sgemm_last_variant must name that thread's own variant.  The first-use case runs in a fresh process, so that the threads race to
initialise that state.
"""
from __future__ import annotations

import os
import subprocess
import sys
import threading

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (M, N, K, trans_a, trans_b, alpha, beta): tiny, small unaligned, small_shortk, large, transposed
SHAPES = [(300, 260, 600, False, False, 1.0, 0.0), (401, 333, 777, False, False, 0.5, -1.5),
          (256, 256, 256, False, False, 1.0, 0.5), (2048, 2048, 1536, False, False, 1.0, 0.0),
          (333, 257, 520, True, False, 1.0, 0.0), (640, 384, 1000, False, True, 2.0, 1.0),
          (1000, 64, 4096, False, False, 1.0, 0.0)]


def run_threads(n_threads: int = 6, reps: int = 3) -> int:
    """Return the number of mismatching results (0 on success)."""
    import fp32_gemm_05_amd as sg
    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(7)
    cases = []
    for (M, N, K, ta, tb, alpha, beta) in SHAPES:
        A = torch.rand((K, M) if ta else (M, K), generator=gen).to(dev) * 2 - 1
        B = torch.rand((N, K) if tb else (K, N), generator=gen).to(dev) * 2 - 1
        C0 = torch.rand((M, N), generator=gen).to(dev) * 2 - 1
        cases.append((A, B, C0, ta, tb, alpha, beta))
    torch.cuda.synchronize()  # the inputs exist before any side stream reads them
    outs = [[None] * len(cases) for _ in range(n_threads)]
    errors = []
    start = threading.Barrier(n_threads)

    def work(t):
        try:
            stream = torch.cuda.Stream(device=dev)
            start.wait()
            with torch.cuda.stream(stream):
                for r in range(reps):
                    for i, (A, B, C0, ta, tb, alpha, beta) in enumerate(cases[t % len(cases):] + cases[:t % len(cases)]):
                        j = (i + t) % len(cases)
                        C = C0.clone()
                        sg.gemm(A, B, C, alpha=alpha, beta=beta, trans_a=ta, trans_b=tb, stream=stream)
                        # sgemm_last_variant is per thread: it names this thread's call, whatever
                        # the other threads launched meanwhile
                        M, N = C.shape
                        K = A.shape[0] if ta else A.shape[1]
                        want = sg.sgemm_op_select_variant(ta, tb, M, N, K, A, A.shape[1], B, B.shape[1], C, N)
                        if sg.sgemm_last_variant() != want:
                            errors.append(f"thread {t}: last variant {sg.sgemm_last_variant()} != {want}")
                        if r == reps - 1:
                            outs[t][j] = C
                stream.synchronize()
        except Exception as e:  # reported by the caller
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    if errors:
        print("errors:", errors, flush=True)
        return len(errors)
    bad = 0
    for j, (A, B, C0, ta, tb, alpha, beta) in enumerate(cases):
        C = C0.clone()
        sg.gemm(A, B, C, alpha=alpha, beta=beta, trans_a=ta, trans_b=tb)
        torch.cuda.synchronize()
        ref = C.cpu().numpy().view(np.uint32)
        for t in range(n_threads):
            if not np.array_equal(outs[t][j].cpu().numpy().view(np.uint32), ref):
                print(f"thread {t} case {j} differs", flush=True)
                bad += 1
    return bad


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def test_concurrent_calls_in_process():
    print("threads: in-process, 6 threads x 7 cases x 3 reps", flush=True)
    assert run_threads() == 0


def test_concurrent_first_use_in_fresh_process():
    print("threads: fresh process, first use from 6 threads", flush=True)
    code = ("import sys; sys.path.insert(0, %r); from tests.test_gpu_threads import run_threads; "
            "sys.exit(min(run_threads(), 100))" % ROOT)
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=110)
    print(res.stdout[-2000:], res.stderr[-2000:], flush=True)
    assert res.returncode == 0
