"""sgemm_ws_noalloc (the entry point that allocates nothing) against
sgemm_ws with a caller's workspace, through the C ABI.

Two calls in a row on the no-allocation path, the second on a smaller
problem, each compared bit for bit with sgemm_ws on the same inputs (the
same plan and kernels) and with the oracle under the pass rule; a split-K
plan and a stream-K plan both go through the static scratch, and a problem
that needs no scratch goes through as well.  Nothing outside C is written."""
import numpy as np
import pytest
import torch

import fp32_gemm_03_amd as g
from fp32_gemm_03_amd import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(p, noalloc):
    """C after one call (sgemm_ws_noalloc, or sgemm_ws with the workspace it
    asks for, NaN-filled), with the guard band around C checked."""
    oa, _, a = gu.to_gpu(p.A)
    ob, _, b = gu.to_gpu(p.B)
    oc, first, c = gu.to_gpu(p.C)
    args = (p.M, p.N, p.K, p.alpha, a, p.lda, b, p.ldb, p.beta, c, p.ldc)
    if noalloc:
        g.sgemm_ws_noalloc(*args)
    else:
        need = g.sgemm_workspace_size(p.M, p.N, p.K)
        ws = torch.full((max(need, 256) // 4 + 64,), float("nan"), dtype=torch.float32, device="cuda")
        g.sgemm_ws(*args, workspace=ws)
    torch.cuda.synchronize()
    host = oc.cpu().numpy()
    n = p.C.numel()
    assert np.all(np.isnan(np.concatenate([host[:first], host[first + n:]]))), "write outside C"
    return host[first:first + n].reshape(p.C.shape)


# (M, N, K, alpha, beta): stream-K over 256 workers on 64 x 64 tiles (8 MiB of
# scratch), then split-K in 16 (4 MiB); split-K in 8 (8 MiB), then a shape
# that needs none; odd sizes (rows only 4-byte aligned): split-K in 8, then
# in 15
PAIRS = [((1536, 1536, 1536, 1.25, -0.5), (256, 256, 4096, 0.75, 0.5)),
         ((512, 512, 8192, 1.0, 0.0), (200, 130, 333, -1.5, 1.0)),
         ((511, 511, 8191, 1.0, 0.5), (255, 255, 4095, -0.75, 0.0))]


@pytest.mark.parametrize("pair", PAIRS, ids=["streamk-then-splitk", "splitk-then-none",
                                             "odd-splitk-twice"])
def test_noalloc_matches_sgemm_ws_on_two_calls(pair):
    for idx, (M, N, K, alpha, beta) in enumerate(pair):
        p = inputs.make_problem(M, N, K, dist="upm1", seed=61 + idx, alpha=alpha, beta=beta,
                                c_fill="upm1" if beta != 0 else "nan")
        need = g.sgemm_workspace_size(M, N, K)
        assert need <= g.SGEMM_NOALLOC_SCRATCH_BYTES
        if idx == 0:
            assert need > 0  # the first call of each pair goes through the scratch
        gu.say("noalloc", M, N, K, "scratch bytes", need, "plan", g.sgemm_ws_plan(M, N, K))
        got = _run(p, noalloc=True)
        want = _run(p, noalloc=False)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (M, N, K)
        assert gu.ratio_full(p, got) <= gu.TOL, (M, N, K)


def test_noalloc_refuses_a_plan_beyond_its_scratch():
    # 7168^3 shares K tiles stream-K on 256 x 256 tiles: 128 MiB of partials
    M = N = K = 7168
    assert g.sgemm_workspace_size(M, N, K) > g.SGEMM_NOALLOC_SCRATCH_BYTES
    a = torch.zeros(1, device="cuda")
    rc = g.sgemm_ws_noalloc(M, N, K, 1.0, a.data_ptr(), K, a.data_ptr(), N, 0.0, a.data_ptr(), N,
                            check=False)
    assert rc == -27
    torch.cuda.synchronize()
