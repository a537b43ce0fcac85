"""Memory-bound kernels against the oracle's definitions, through the C ABI
(transpose) and through whole-step parity (RMSNorm, SwiGLU, RoPE run inside
every layer; their own checks are in test_gpu_step and test_gpu_kernels)."""
import numpy as np
import pytest

import host_memory_layer_amd as mt

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("R,C,ld_in,ld_out", [(64, 64, 64, 64), (200, 136, 144, 208), (8, 8, 8, 8),
                                              (130, 70, 70, 130), (4096, 5120, 5120, 4224)])
def test_transpose_exact(R, C, ld_in, ld_out):
    rng = np.random.default_rng(R + C)
    a = rng.integers(0, 65535, (R, ld_in), dtype=np.uint16)
    A = torch.from_numpy(a.view(np.int16)).to(dev())
    O = torch.full((C, ld_out), -1, dtype=torch.int16, device=dev())
    mt.check(mt.lib().mt_transpose(mt.MT_BF16, A.data_ptr(), ld_in, O.data_ptr(), ld_out, R, C, None))
    torch.cuda.synchronize()
    o = O.cpu().numpy().view(np.uint16)
    assert np.array_equal(o[:, :R], a[:, :C].T)
    assert np.all(o[:, R:] == 0xFFFF)
