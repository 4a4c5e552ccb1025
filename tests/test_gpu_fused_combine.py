"""The routed projection of many tokens with the gate-weighted combine fused in
(mxfp4_expert_proj_combine_routed; src/experts.linnet fn forward_routed).

Each case is compared with the oracle (routing bit for bit, per-slot outputs
and y within the projection's bound) and bit for bit with the separate calls
route_group + mxfp4_expert_proj + moe_combine on the same routing, on both
paths.  On the grouped-GEMM path the combine runs inside the GEMM, summed by
whichever tile brings a token's last routed row; the shapes below give tokens
whose slots land in different row tiles and weight panels, partial panels,
widths with N % 4 != 0 (the scalar store and sum), k = 1, k = E and more than
64 experts.  On the GEMV path, batches with T * k <= E run the projection and
the sums in one launch (a workgroup per token and row block).  The model-size down prefill is checked bit for bit against the
separate calls and for determinism over repeated runs (the tiles' finishing
order varies from run to run; y must not).
"""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mxfp4_mixture_experts_amd import binding as B
from mxfp4_mixture_experts_amd import synthetic as S
from mxfp4_mixture_experts_amd.runner import DeviceProblem
from test_gpu_parity import check_close, check_routing

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def _announce(msg):
    print(f"[case] {msg}", flush=True)


FUSED_CASES = {
    # name: make_custom kwargs
    "down_like_zipf": dict(E=32, N=576, K=512, T=300, k=4, x_per_slot=True, route="zipf+logits"),
    "ragged_shared": dict(E=8, N=200, K=320, T=137, k=3, route="logits"),
    "odd_width": dict(E=6, N=198, K=256, T=90, k=2, x_per_slot=True, route="logits"),
    "top1": dict(E=16, N=384, K=128, T=200, k=1, route="logits"),
    "many_experts": dict(E=100, N=136, K=96, T=120, k=5, route="logits"),
    "one_token": dict(E=8, N=96, K=64, T=1, k=2, route="logits"),
    "all_experts_k8": dict(E=8, N=192, K=128, T=64, k=8, x_per_slot=True, route="logits"),
    "given_ids": dict(E=12, N=392, K=2880, T=70, k=4, x_per_slot=True, route="ids+logits"),
    # T * k <= E: on the GEMV path a workgroup sums one token's slots (one launch)
    "small_batch_down": dict(E=32, N=2880, K=2880, T=4, k=4, x_per_slot=True, route="logits"),
    "small_batch_shared": dict(E=16, N=200, K=320, T=3, k=4, route="logits"),
    "small_given_ids": dict(E=12, N=96, K=256, T=3, k=4, x_per_slot=True, route="ids+logits"),
}


def _separate(p, path):
    dp = DeviceProblem(p, path=path)
    dp.run()
    return dp.results()


@pytest.mark.parametrize("path", [B.MXFP4_PATH_GEMV, B.MXFP4_PATH_GEMM])
@pytest.mark.parametrize("case", sorted(FUSED_CASES))
def test_fused_combine_cases(case, path):
    p = S.make_custom(**FUSED_CASES[case], combine=True)
    p.name = case
    _announce(f"fused combine {case} path={path}")
    ref = O.run_problem(p)
    dp = DeviceProblem(p, path=path)
    dp.route_group()
    dp.out.fill_(float("nan"))
    dp.y.fill_(float("nan"))
    dp.proj_combine_routed()
    g = dp.results()
    assert g["error_word"] == 0
    check_routing(g, ref)
    check_close(g["out"], ref["out"], ref["mag"], f"{case} out")
    check_close(g["y"], ref["y"], ref["mag_y"], f"{case} y")
    g2 = _separate(p, path)
    np.testing.assert_array_equal(g["out"], g2["out"])
    np.testing.assert_array_equal(g["y"], g2["y"])


def test_fused_combine_unrouted_tokens():
    """Tokens whose logits hold a NaN have no routed slot: y = 0 for them, as the
    separate combine gives (their gates are 0); given ids outside [0, E) leave
    single slots unrouted.  Every other token as the separate calls."""
    T, E, k = 137, 16, 4
    _announce("fused combine with unrouted tokens and slots")
    p = S.make_custom(E=E, N=400, K=256, T=T, k=k, x_per_slot=True, route="logits", combine=True, tag=640)
    p.logits = p.logits.copy()
    bad = [1, T // 2, T - 1]
    p.logits[1, 3] = NAN_BF16
    p.logits[T // 2, :] = NAN_BF16
    p.logits[T - 1, 0] = NAN_BF16
    for path in (B.MXFP4_PATH_GEMV, B.MXFP4_PATH_GEMM):
        dp = DeviceProblem(p, path=path)
        dp.route_group()
        dp.y.fill_(float("nan"))
        dp.proj_combine_routed()
        g = dp.results()
        assert g["error_word"] == B.MXFP4_ROUTE_ERR_ID_RANGE
        assert np.all(g["y"][bad] == 0.0)
        g2 = _separate(p, path)
        good = [t for t in range(T) if t not in bad]
        np.testing.assert_array_equal(g["y"], g2["y"])
        np.testing.assert_array_equal(g["out"][good], g2["out"][good])

    for T2, bad2 in ((50, [3, 7, 20]), (4, [0, 1, 3])):  # T2 * k <= E: the one-launch GEMV combine
        q = S.make_custom(E=E, N=200, K=128, T=T2, k=k, x_per_slot=True, route="ids+logits", combine=True,
                          tag=641 + T2)
        q.ids_in = np.array(q.ids_in, dtype=np.int32, copy=True)
        q.ids_in[bad2[0], 1] = -1
        q.ids_in[bad2[1], 0] = E + 5
        q.ids_in[bad2[2], :] = -2       # a token with no valid id at all
        for path in (B.MXFP4_PATH_GEMV, B.MXFP4_PATH_GEMM):
            dp = DeviceProblem(q, path=path)
            dp.route_group()
            dp.y.fill_(float("nan"))
            dp.proj_combine_routed()
            g = dp.results()
            assert g["error_word"] & B.MXFP4_ROUTE_ERR_ID_RANGE
            assert np.all(g["y"][bad2[2]] == 0.0)
            g2 = _separate(q, path)
            np.testing.assert_array_equal(g["y"], g2["y"])


def test_fused_combine_model_size_deterministic():
    """The down prefill of 2048 tokens (Zipf expert choice, 15 weight panels of
    192 columns): the fused y equals the separate calls' bit for bit, on every
    run."""
    p = S.make_config(4)
    _announce(f"fused combine {p.name} (model size)")
    g2 = _separate(p, B.MXFP4_PATH_GEMM)
    dp = DeviceProblem(p, path=B.MXFP4_PATH_GEMM)
    dp.route_group()
    for rep in range(3):
        dp.out.fill_(float("nan"))
        dp.y.fill_(float("nan"))
        dp.proj_combine_routed()
        g = dp.results()
        np.testing.assert_array_equal(g["out"], g2["out"])
        np.testing.assert_array_equal(g["y"], g2["y"])
    # the same workspace after a projection without the combine: the counters
    # are set again by every fused call
    dp.expert_proj()
    dp.y.fill_(float("nan"))
    dp.proj_combine_routed()
    np.testing.assert_array_equal(dp.results()["y"], g2["y"])


@pytest.mark.parametrize("T", [4, 50])
def test_fused_combine_ignores_the_gates_of_unrouted_slots(T):
    """A slot whose id lies outside [0, E) adds a zero product whatever its gate
    holds: with NaN written into those gates after the routing, y is bit-equal to
    the same call with the routing's own gates (0 there), on both paths (T = 4:
    the one-launch GEMV combine; T = 50: the GEMV projection then the combine,
    and the sums inside the grouped GEMM)."""
    E, k = 16, 4
    _announce(f"fused combine, NaN gates on unrouted slots, T={T}")
    q = S.make_custom(E=E, N=200, K=128, T=T, k=k, x_per_slot=True, route="ids+logits", combine=True, tag=660 + T)
    q.ids_in = np.array(q.ids_in, dtype=np.int32, copy=True)
    q.ids_in[0, 1] = -1
    q.ids_in[T - 1, 2] = E + 3
    for path in (B.MXFP4_PATH_GEMV, B.MXFP4_PATH_GEMM):
        dp = DeviceProblem(q, path=path)
        dp.route_group()
        dp.proj_combine_routed()
        ref = dp.results()["y"].copy()
        assert np.all(np.isfinite(ref))
        bad = (dp.topk_ids < 0) | (dp.topk_ids >= E)
        dp.gates[bad] = float("nan")
        dp.y.fill_(float("nan"))
        dp.proj_combine_routed()
        np.testing.assert_array_equal(dp.results()["y"], ref)
