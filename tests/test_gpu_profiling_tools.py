"""The measurement tools on the GPU: the phase-stamp build of libsgemm computes exactly what the
product library computes and leaves well-formed stamps, and the MFMA issue-rate reference measures
the rates the phase reports divide by.
"""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from fp32_gemm_05_amd import _binding as sg  # noqa: E402
from fp32_gemm_05_amd import build as hb  # noqa: E402
from fp32_gemm_05_amd import profiling  # noqa: E402


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def stamps_lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    if not os.path.exists(hb.STAMPS_LIB):
        pytest.skip("libsgemm_stamps.so not built")
    lib = sg.load_library(hb.STAMPS_LIB)
    lib.sgemm_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_uint]
    lib.sgemm_phase_stamps.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("M,N,K,vec", [(512, 512, 256, True), (333, 517, 129, False), (1024, 1024, 512, True)])
def test_phase_stamps_same_result_and_well_formed(stamps_lib, M, N, K, vec):
    """The stamped build's result equals the product library's bit for bit on integer data (the
    hooks only read clocks), every wave of the grid writes its five slots, the shader clock runs
    forward across the four phase boundaries, and HW_ID's SIMD field is 0..3."""
    _say(f"[stamps] {M}x{N}x{K} vec={vec}")
    rng = np.random.default_rng(M * 7 + K)
    A = rng.integers(-2, 3, (M, K)).astype(np.float32)
    B = rng.integers(-2, 3, (K, N)).astype(np.float32)
    lda, ldb, ldc = (K, N, N) if vec else (K | 1, N | 1, N | 1)
    dA = torch.zeros((M, lda), dtype=torch.float32, device="cuda")
    dB = torch.zeros((K, ldb), dtype=torch.float32, device="cuda")
    dA[:, :K] = torch.from_numpy(A).cuda()
    dB[:, :N] = torch.from_numpy(B).cuda()
    vid = sg.sgemm_select_variant(M, N, K, dA, lda, dB, ldb, dA, ldc)
    info = sg.sgemm_variant_info(vid)
    name = sg.sgemm_variant_name(vid)
    _say(f"[stamps] variant {name}")
    tiles = -(-M // info["BM"]) * -(-N // info["BN"])
    waves = tiles * info["threads"] // 64
    buf = torch.zeros(waves * 10, dtype=torch.int64, device="cuda")
    out = []
    for lib, stamped in ((sg.load_library(), False), (stamps_lib, True)):
        dC = torch.zeros((M, ldc), dtype=torch.float32, device="cuda")
        if stamped:
            assert lib.sgemm_phase_stamps(buf.data_ptr(), waves) == 0
        rc = lib.sgemm_ex(M, N, K, 1.0, dA.data_ptr(), lda, dB.data_ptr(), ldb, 0.0, dC.data_ptr(), ldc,
                          torch.cuda.current_stream().cuda_stream, vid)
        torch.cuda.synchronize()
        if stamped:
            assert lib.sgemm_phase_stamps(None, 0) == 0
        assert rc == 0
        out.append(dC[:, :N].cpu().numpy())
    assert np.array_equal(out[0], out[1])
    assert np.array_equal(out[0], A.astype(np.float64) @ B.astype(np.float64))
    x = buf.cpu().numpy().reshape(waves, 5, 2).astype(np.int64)
    if name.startswith(("mfma32l_", "mfma16l_", "mfma32_", "mfma32d_")) and "_ps" not in name:
        c = x[:, :4, 0]
        assert (c > 0).all(), "every wave writes its four phase stamps"
        assert (np.diff(c, axis=1) >= 0).all(), "the shader clock runs forward across the phases"
        assert (x[:, :4, 1] > 0).all() and (np.diff(x[:, :4, 1], axis=1) >= 0).all()
        hw = x[:, 4, 0]
        assert (((hw >> 4) & 3) <= 3).all() and (hw >= 0).all()


def test_mfma_issue_rates():
    """mfma_chain at one wave per SIMD: a 32x32x2 f32 MFMA takes ~64 cycles and a 16x16x4 f32 one
    ~32 with four interleaved accumulators (the issue rates that make 157.3 TFLOP/s at 2.4 GHz);
    one dependent chain is no faster."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    s = torch.cuda.current_stream()
    r32 = profiling.mfma_cycles(32, s, ilp=4)
    r16 = profiling.mfma_cycles(16, s, ilp=4)
    d16 = profiling.mfma_cycles(16, s, ilp=1)
    _say(f"[mfma] 32x32x2 {r32}, 16x16x4 {r16}, 16x16x4 dependent {d16}")
    assert 60.0 <= r32[0] <= 72.0
    assert 30.0 <= r16[0] <= 38.0
    assert d16[0] >= r16[0] - 0.5


@pytest.mark.parametrize("nt", [0, 1])
def test_write_reference_writes_every_element_once(nt):
    """The write reference stores each element of the M x N window exactly where the MFMA
    epilogue's lane order puts it (the value it writes depends on the row within a 32-row block
    only) and nothing in the row padding."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lib = profiling._hbm_read_lib()
    M, N, ldc = 128, 192, 256
    _say(f"[write reference] {M}x{N} ldc={ldc} nt={nt}")
    buf = torch.full((M, ldc), -7.0, dtype=torch.float32, device="cuda")
    assert lib.hbm_write_tiles(buf.data_ptr(), M, N, ldc, nt, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    rb = np.arange(M) % 32
    want = (1.0 + 4 * (rb // 8) + rb % 4).astype(np.float32)
    assert np.array_equal(got[:, :N], np.repeat(want[:, None], N, axis=1))
    assert np.all(got[:, N:] == -7.0)
