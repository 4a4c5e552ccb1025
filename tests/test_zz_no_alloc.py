"""mxfp4_expert_proj_noalloc: the projection with the library's static scratch
in place of a caller's workspace.  Through the C ABI, its outputs equal those
of mxfp4_expert_proj with a workspace bit for bit (same kernels, same inputs),
on two calls in a row, the second smaller than the first (the scratch keeps
the first call's contents, which the second must not read), and both lie
within the parity bound of the oracle."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mxfp4_mixture_experts_amd import binding as B
from mxfp4_mixture_experts_amd import synthetic as S
from mxfp4_mixture_experts_amd.runner import DeviceProblem

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _noalloc_vs_workspace(p, path):
    dp = DeviceProblem(p, path=path)
    dp.route_group()
    dp.out.fill_(float("nan"))
    dp.expert_proj()                                   # caller's workspace
    torch.cuda.synchronize()
    want = dp.out.cpu().numpy()
    dp.out.fill_(float("nan"))
    B.mxfp4_expert_proj_noalloc(dp.blocks, dp.scales, dp.bias, p.E, p.N, p.K, dp.x, p.x_per_slot, p.T, p.k,
                                dp.offsets, dp.sorted_rows, dp.out, path)
    torch.cuda.synchronize()
    got = dp.out.cpu().numpy()
    np.testing.assert_array_equal(got, want)
    ref = O.run_problem(p)
    err = np.abs(got.astype(np.float64) - ref["out"])
    assert np.all(err <= O.parity_bound(ref["mag"])), "outside the parity bound"


def test_noalloc_matches_workspace_entry_point():
    # first: a large problem with outlier channels (extra activation terms in the scratch)
    big = S.make_custom(E=8, N=512, K=2880, T=512, k=4, route="logits", tag=950)
    big.x = S.scale_channels(big.x, [5, 700, 1400, 2801], 1000.0)
    assert B.mxfp4_expert_proj_workspace_size(big.E, big.N, big.T, big.k, big.K, 0, 2) > (16 << 20)
    _announce("noalloc: large, outlier channels, GEMM")
    _noalloc_vs_workspace(big, B.MXFP4_PATH_GEMM)
    # then smaller, different shapes, no extra terms: nothing of the first call may leak in
    small = S.make_custom(E=4, N=200, K=1024, T=37, k=3, x_per_slot=True, route="ids+logits", tag=951)
    _announce("noalloc: small, GEMM")
    _noalloc_vs_workspace(small, B.MXFP4_PATH_GEMM)
    # the GEMV path needs no scratch
    one = S.make_custom(E=32, N=96, K=2880, T=1, k=4, route="logits", tag=952)
    _announce("noalloc: one token, GEMV")
    _noalloc_vs_workspace(one, B.MXFP4_PATH_AUTO)

