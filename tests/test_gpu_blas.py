"""The block front end's library GEMM path (hipBLASLt, through the probe
build's qsa_probe_gemm): products against a float64 reference, and the same
shape bit for bit after the per-device plan cache has been emptied and
rebuilt (more shapes than it keeps)."""
import numpy as np
import pytest
import torch

from block_sparse_attention_keys_amd import qsa
from gpu_harness import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qsa.lib()
    yield


def _product(P, A, B, d_f32):
    M, K = A.shape
    N = B.shape[0]
    D = torch.empty(M, N, device="cuda", dtype=torch.float32 if d_f32 else torch.bfloat16)
    rc = P.qsa_probe_gemm(A.data_ptr(), B.data_ptr(), D.data_ptr(), int(d_f32), M, N, K,
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return rc, D


def _reference(A, B):
    return A.double().cpu().numpy() @ B.double().cpu().numpy().T


def test_library_gemm_matches_reference_and_survives_cache_rebuild():
    g = torch.Generator(device="cuda").manual_seed(0)
    K, N = 256, 512
    B = torch.randn(N, K, device="cuda", generator=g).to(torch.bfloat16)
    A0 = torch.randn(1024, K, device="cuda", generator=g).to(torch.bfloat16)
    with qsa.probe_library() as P:
        rc, D0 = _product(P, A0, B, True)
        if rc == 1:
            pytest.skip("hipBLASLt cannot run the product here")
        assert rc == 0
        ref = _reference(A0, B)
        # fp32 accumulation of K = 256 bf16 products: well inside 1e-5 of the row scale
        tol = 1e-5 * np.abs(ref).max()
        assert np.abs(D0.cpu().numpy() - ref).max() <= tol
        rc, H0 = _product(P, A0, B, False)  # bf16 output: one rounding of the fp32 result
        assert rc == 0
        assert np.abs(H0.float().cpu().numpy() - ref).max() <= 2.0 ** -8 * np.abs(ref).max()
        # 70 more shapes (more than the 64 plans a device keeps), each checked
        for i in range(70):
            M = 256 + 8 * i
            A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
            rc, D = _product(P, A, B, True)
            assert rc == 0, M
            r = _reference(A, B)
            assert np.abs(D.cpu().numpy() - r).max() <= 1e-5 * np.abs(r).max(), M
        rc, D1 = _product(P, A0, B, True)
        assert rc == 0
        assert torch.equal(D0, D1), "the rebuilt plan gives a different result"
        say("  70 shapes through the plan cache; the first shape bit-identical after the rebuild")
