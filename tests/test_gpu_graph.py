"""libsgemm calls captured into a HIP graph and replayed (torch.cuda.CUDAGraph).

The library allocates nothing and only enqueues kernels on the caller's stream, so a call can
be captured once and replayed.  Each case captures one call (the dispatch of a tiny, an
unaligned small, a large drain-ordered and a transposed problem, and the alpha = 0 scale path),
then replays the graph several times, with eager GEMMs and synchronizations between the
replays, resetting C before each one.  Every replay must equal the eager call bit for bit (same
kernel, same inputs: the kernels are deterministic) and the oracle within the tolerance of the
parity tests on sampled outputs.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from fp32_gemm_05_amd.workloads import WORKLOADS, make_inputs, sample_points
from tests.gemm_cases import check_within_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import fp32_gemm_05_amd as sg  # noqa: E402

CASES = [
    # (label, workload, M, N, K, trans_a, trans_b, alpha or None for the workload's)
    ("tiny_vec", "square256", 200, 256, 520, False, False, None),
    ("small_unaligned_beta", "ragged3001x5003x777", 601, 503, 777, False, False, None),
    ("large_drain", "square4096", 2048, 2048, 2048, False, False, None),
    ("trans_nt_beta", "square1024_beta", 257, 384, 300, False, True, None),
    ("scale_only", "square1024_beta", 130, 70, 40, False, False, 0.0),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("label,wname,M,N,K,ta,tb,alpha", CASES, ids=[c[0] for c in CASES])
def test_captured_call_replays(label, wname, M, N, K, ta, tb, alpha):
    w = WORKLOADS[wname]
    alpha = w.alpha if alpha is None else alpha
    beta = w.beta
    print(f"graph case {label}: {M}x{N}x{K} trans=({ta},{tb}) alpha={alpha} beta={beta}", flush=True)
    A, B, C0 = make_inputs(w, M=M, N=N, K=K)
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(np.ascontiguousarray(A.T) if ta else A).to(dev)
    dB = torch.from_numpy(np.ascontiguousarray(B.T) if tb else B).to(dev)
    dC0 = torch.from_numpy(C0).to(dev)
    dC = dC0.clone()

    def call():
        sg.gemm(dA, dB, dC, alpha=alpha, beta=beta, trans_a=ta, trans_b=tb)

    # eager reference run (also initialises the library's per-kernel launch data)
    call()
    torch.cuda.synchronize()
    eager = dC.cpu().numpy().copy()
    I, J = sample_points(M, N, 1024, seed=w.seed + 31, tile=32)
    ref, bound = oracle.ref_points(A, B, C0, I, J, alpha, beta)
    check_within_bound(eager[I, J], ref, bound, f"{label} eager")

    # capture one call on a side stream
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dC.copy_(dC0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    # other work between replays: an eager GEMM on separate buffers
    X = torch.rand(300, 200, device=dev)
    Y = torch.rand(200, 100, device=dev)
    Z = torch.zeros(300, 100, device=dev)
    for r in range(4):
        dC.copy_(dC0)
        sg.gemm(X, Y, Z)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = dC.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), \
            f"{label}: replay {r} differs from the eager call in {np.count_nonzero(got != eager)} elements"
        check_within_bound(got[I, J], ref, bound, f"{label} replay {r}")
    torch.cuda.synchronize()
    del graph
