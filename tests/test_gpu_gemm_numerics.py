"""The grouped GEMM's activation split on activations of wide dynamic range.

The GEMM multiplies each bf16 activation block of 32 as MX-FP6 terms sharing
one E8M0 scale per term.  Two terms keep the parity bound for blocks of like
magnitudes; a block with an outlier channel, or a heavy-tailed one, takes a
third and a fourth term (chosen per block by the pre-pass), so that its small
elements keep their precision.  Every case is compared element by element
with the oracle (2e-3 * sum |w x| + 1e-5 per output); the GEMV path, whose
products are exact, runs beside it.
"""
import numpy as np
import pytest

import oracle.moe_oracle as O
from mxfp4_mixture_experts_amd import binding as B
from mxfp4_mixture_experts_amd import synthetic as S
from mxfp4_mixture_experts_amd.runner import DeviceProblem
from test_gpu_parity import check_act, check_close, check_routing, full_parity

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


# (outlier channels, factor): gate_up-like shapes, K = 2880 (the compiled
# 12-stage pipeline) and K = 1024 (the looped one)
OUTLIER_CASES = {
    "one_channel_x100": ([7], 100.0),
    "four_channels_x1000": ([5, 700, 1400, 2801], 1000.0),
    "four_channels_x1e4": ([5, 700, 1400, 2801], 1e4),
    "two_channels_x1e5": ([33, 1500], 1e5),
    "adjacent_channels_x1000": ([64, 65, 66, 67], 1000.0),
}


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("case", sorted(OUTLIER_CASES))
def test_outlier_channels(case, path):
    channels, factor = OUTLIER_CASES[case]
    p = S.make_custom(E=8, N=512, K=2880, T=256, k=4, route="logits", tag=900)
    p.x = S.scale_channels(p.x, channels, factor)
    p.name = case
    full_parity(p, path)


@pytest.mark.parametrize("path", [1, 2])
def test_outlier_channels_looped_pipeline(path):
    """K = 1024: the GEMM's looped main loop, per-slot inputs."""
    p = S.make_custom(E=6, N=300, K=1024, T=200, k=3, x_per_slot=True, route="ids+logits", tag=901)
    p.x = S.scale_channels(p.x, [3, 500, 1023], 3000.0)
    p.name = "outliers K=1024"
    full_parity(p, path)


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("sigma", [1.0, 2.0, 3.0])
def test_heavy_tailed_activations(sigma, path):
    """sign * exp(sigma * N(0,1)): most blocks span several binades."""
    p = S.make_custom(E=8, N=384, K=2880, T=200, k=4, route="logits", tag=902)
    p.x = S.lognormal_bf16(p.x.shape, sigma, tag=902)
    p.name = f"lognormal sigma={sigma}"
    full_parity(p, path)


def test_outliers_through_gated_activation():
    """The gated-activation epilogue after the extra terms."""
    p = S.make_custom(E=8, N=512, K=2880, T=128, k=4, route="logits", tag=903)
    p.x = S.scale_channels(p.x, [5, 700, 1400, 2801], 1000.0)
    _announce("outliers + gated activation")
    ref = O.run_problem(p)
    dp = DeviceProblem(p, path=B.MXFP4_PATH_GEMM)
    dp.route_group()
    dp.expert_proj_swiglu()
    g = dp.results()
    check_routing(g, ref)
    check_act(g["act"], ref["out"], ref["mag"], "outliers act")


def _swiglu_range_inputs(shape, seed):
    """Down-projection inputs with the range of the gated activation: the
    oracle's activation of gate/up values drawn N(0, 3^2), rounded to bf16."""
    rng = np.random.default_rng(seed)
    gu = 3.0 * rng.standard_normal(size=shape[:-1] + (2 * shape[-1],))
    return S.f32_to_bf16_bits(O.swiglu(gu).astype(np.float32))


@pytest.mark.parametrize("path", [0, 1])
def test_swiglu_range_down_prefill(path):
    """The Zipf down prefill (E=32, N=K=2880, T=2048, top-4) with the gated
    activation's range as input, every output against the oracle."""
    p = S.make_config(4)
    p.x = _swiglu_range_inputs(p.x.shape, 904)
    p.name = "down prefill, gated-activation inputs"
    full_parity(p, path)
