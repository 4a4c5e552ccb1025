"""GPU parity of the router and of the whole MoE block chained through the C ABI.

Router logits: the GPU rounds an fp32 sum of exact bf16 products to bf16; the
oracle's value is exact.  Bound: half a bf16 ulp (at most 2^-8 |z|) plus the
fp32 summation error, at most 2^-16 * sum |x w| for these widths (a few dozen
fp32 roundings of partial sums, each at most 2^-24 of the magnitude).

The block: router -> route_group -> gate/up projection through the gated
activation -> down projection of the activations -> gate-weighted combine.
Each stage is compared with the oracle on the GPU's own inputs to that stage
(the logits the GPU rounded, the bf16 activations it wrote), so that the
checks are as tight as the single-stage ones and a near-tie in the logits
cannot flip an expert choice between the two sides.
"""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mxfp4_mixture_experts_amd import binding as B
from mxfp4_mixture_experts_amd import synthetic as S
from mxfp4_mixture_experts_amd.runner import DeviceProblem
from test_gpu_parity import check_act, check_close, check_routing

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def router_gpu(r: S.RouterProblem, with_bias=True):
    logits = torch.empty((r.T, r.E), dtype=torch.bfloat16, device="cuda")
    B.mxfp4_moe_router(_dev_bf16(r.x), _dev_bf16(r.w), _dev_bf16(r.bias) if with_bias else None, r.T, r.H, r.E,
                       logits)
    torch.cuda.synchronize()
    return logits.view(torch.int16).cpu().numpy().view(np.uint16)


def check_logits(bits, r: S.RouterProblem, with_bias=True):
    z, mag = O.router_logits(r.x, r.w, r.bias if with_bias else None)
    g = O.bf16_to_f64(bits)
    assert np.all(np.isfinite(g))
    bound = 2.0 ** -8 * np.abs(z) + 2.0 ** -16 * mag + 1e-30
    err = np.abs(g - z)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{len(bad)} logits outside the bound, worst {float((err / bound).max()):.3g}, first {bad[:3].tolist()}"


ROUTER_CASES = {
    "decode_t1": (1, 2880, 32),        # gpt-oss-20b decode: one workgroup per expert row
    "t17_first_tiles": (17, 2880, 32), # the smallest batch on 16-expert tiles: a ragged token tile
    "small_t64": (64, 2880, 32),       # the largest batch on 16-expert tiles
    "t65_wide_tiles": (65, 2880, 32),  # 32-expert tiles, a ragged token tile
    "ragged_experts": (37, 256, 100),  # E not a multiple of the tile
    "narrow_h": (300, 32, 7),          # one K step: 15 of the 16 waves contribute nothing
    "long_h": (20, 8192, 32),          # several chunks per wave
    "one_expert": (5, 96, 1),
    # up to 16 tokens: one workgroup per expert row
    "rows_t3": (3, 2880, 32),
    "rows_t8": (8, 2880, 32),
    "rows_t16": (16, 2880, 32),
    "rows_t7_ragged": (7, 160, 13),
    "rows_t2_narrow": (2, 96, 7),
    "rows_t4_long_h": (4, 8192, 100),
}


@pytest.mark.parametrize("case", sorted(ROUTER_CASES))
def test_router(case):
    T, H, E = ROUTER_CASES[case]
    _announce(f"router {case} T={T} H={H} E={E}")
    r = S.make_router(T, H, E, tag=200 + sorted(ROUTER_CASES).index(case))
    check_logits(router_gpu(r), r)


def test_router_without_bias_and_deterministic():
    r = S.make_router(40, 2880, 32, tag=11)
    _announce("router without bias, twice")
    a = router_gpu(r, with_bias=False)
    check_logits(a, r, with_bias=False)
    np.testing.assert_array_equal(a, router_gpu(r, with_bias=False))


def test_router_model_size_prefill():
    """T = 4096 tokens of the gpt-oss-20b hidden width, every logit checked."""
    r = S.make_router(4096, 2880, 32, tag=12)
    _announce("router T=4096 H=2880 E=32")
    check_logits(router_gpu(r), r)


def test_router_t0_is_a_noop():
    logits = torch.full((1, 32), 7.0, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    B.mxfp4_moe_router(x, w, None, 0, 64, 32, logits)
    torch.cuda.synchronize()
    assert bool((logits == 7.0).all())


BLOCK_CASES = {
    # T, H, Inner, E, k
    "small": (37, 256, 128, 8, 2),
    "ragged": (90, 96, 160, 6, 3),
    "gpt_oss_decode_t1": (1, 2880, 2880, 32, 4),
    "batch_t64_narrow_inner": (64, 2880, 512, 32, 4),
}


@pytest.mark.parametrize("case", sorted(BLOCK_CASES))
def test_moe_block_chain(case):
    T, H, Inner, E, k = BLOCK_CASES[case]
    _announce(f"moe block {case} T={T} H={H} Inner={Inner} E={E} k={k}")
    seed_tag = 300 + sorted(BLOCK_CASES).index(case)
    r = S.make_router(T, H, E, tag=seed_tag)
    logits = router_gpu(r)
    check_logits(logits, r)
    # gate/up through the gated activation, routed by the GPU's logits
    gu = S.make_custom(E=E, N=2 * Inner, K=H, T=T, k=k, route="logits", tag=seed_tag + 50, combine=False)
    gu.x, gu.logits = r.x, logits
    dp1 = DeviceProblem(gu)
    dp1.route_group()
    dp1.expert_proj_swiglu()
    g1 = dp1.results()
    ref1 = O.run_problem(gu)
    check_routing(g1, ref1)
    check_act(g1["act"], ref1["out"], ref1["mag"], f"{case} activation")
    # down projection of the GPU's activations, combined with the router weights
    dn = S.make_custom(E=E, N=H, K=Inner, T=T, k=k, x_per_slot=True, route="logits", tag=seed_tag + 90,
                       combine=True)
    dn.x = np.ascontiguousarray(g1["act"].reshape(T, k, Inner))
    dn.logits = logits
    dp2 = DeviceProblem(dn)
    dp2.run()
    g2 = dp2.results()
    ref2 = O.run_problem(dn)
    check_routing(g2, ref2)
    check_close(g2["out"], ref2["out"], ref2["mag"], f"{case} down")
    check_close(g2["y"], ref2["y"], ref2["mag_y"], f"{case} y")
