"""mt_gemm_noalloc, the GEMM entry point that allocates nothing, against
mt_gemm_ws with a caller workspace: bit for bit, on two calls in a row, the
second with a smaller input (the static buffer keeps the first call's
partial tiles, which must not leak into the second)."""
import ctypes

import numpy as np
import pytest

import host_memory_layer_amd as mt

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _operands(M, N, K, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    A = (torch.randn(M, K, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    B = (torch.randn(N, K, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    R = torch.randn(M, N, device="cuda", generator=g)
    return A, B, R


def _run(fn, A, B, R, M, N, K, epi, stream, extra=()):
    out = torch.empty(M, N, dtype=torch.bfloat16 if epi == 0 else torch.float32, device="cuda")
    rp = R.data_ptr() if epi == 2 else None
    mt.check(fn(A.data_ptr(), K, B.data_ptr(), K, out.data_ptr(), N, rp, N, M, N, K, epi, 0, *extra, stream))
    return out


def test_noalloc_gemm_matches_the_workspace_gemm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = mt.lib()
    assert L.mt_gemm_noalloc_max_ws() == 128 << 20
    s = torch.cuda.current_stream().cuda_stream
    # both shapes split their last round of tiles along K (320 and 300 tiles
    # of 256 x 256 on 256 workgroups); the second is smaller in every dimension
    for M, N, K, seed in ((4096, 5120, 8192, 1), (3840, 5000, 6144, 2)):
        need = L.mt_gemm_ws_bytes(M, N, K)
        print(f"noalloc GEMM {M}x{N}x{K}: split workspace {need} bytes", flush=True)
        assert 0 < need <= L.mt_gemm_noalloc_max_ws()
        A, B, R = _operands(M, N, K, seed)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        for epi in (0, 1, 2):
            ref = _run(L.mt_gemm_ws, A, B, R, M, N, K, epi, s, (ws.data_ptr(), need))
            got = _run(L.mt_gemm_noalloc, A, B, R, M, N, K, epi, s)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16) if epi == 0 else got.view(torch.int32),
                               ref.view(torch.int16) if epi == 0 else ref.view(torch.int32)), (M, N, K, epi)
    # a shape that does not split uses no scratch and is mt_gemm's result
    M, N, K = 1024, 1024, 512
    A, B, R = _operands(M, N, K, 3)
    assert L.mt_gemm_ws_bytes(M, N, K) == 0
    ref = torch.empty(M, N, dtype=torch.float32, device="cuda")
    mt.check(L.mt_gemm(mt.MT_BF16, A.data_ptr(), K, B.data_ptr(), K, ref.data_ptr(), N, None, 0, M, N, K, 1, 0, s))
    got = _run(L.mt_gemm_noalloc, A, B, R, M, N, K, 1, s)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


def test_noalloc_gemm_argument_errors():
    L = mt.lib()
    assert L.mt_gemm_noalloc(None, 0, None, 0, None, 0, None, 0, 4, 4, 4, 7, 0, None) == mt.MT_E_INVALID
    assert L.mt_gemm_noalloc(None, 0, None, 0, None, 0, None, 0, -1, 4, 4, 0, 0, None) == mt.MT_E_INVALID
    assert L.mt_gemm_noalloc(None, 2, None, 8, None, 8, None, 0, 4, 8, 8, 0, 0, None) == mt.MT_E_INVALID
