"""The entry points inside a captured HIP graph: every replay must reproduce the
eager result bit for bit (the kernels are deterministic and none of them clears
memory with a memset node).  Between replays the outputs are overwritten and
other eager work runs, with synchronisations, as a program would do."""
import numpy as np
import pytest
import torch

from mxfp4_mixture_experts_amd import binding as B
from mxfp4_mixture_experts_amd import synthetic as S
from mxfp4_mixture_experts_amd.runner import DeviceProblem

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _replay_matches(step, outputs):
    """Run step eagerly, capture it, then replay REPLAYS times; each replay's
    outputs (NaN-filled first) must equal the eager ones."""
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # one eager call on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        for o in outputs:
            if o.dtype.is_floating_point:
                o.fill_(float("nan"))
            else:
                o.fill_(-7)
        junk = torch.randn(1 << 20, device="cuda") * 3.0   # unrelated eager work
        junk.sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(o.view(torch.int8) if o.dtype == torch.bfloat16 else o,
                               w.view(torch.int8) if w.dtype == torch.bfloat16 else w), f"replay {r} differs"
    del g


@pytest.mark.parametrize("path", [1, 2])
def test_graph_route_project_combine(path):
    p = S.make_custom(E=8, N=200, K=320, T=37, k=3, route="logits")
    _announce(f"graph: route_group + expert_proj + combine, path {path}")
    dp = DeviceProblem(p, path=path)
    _replay_matches(dp.run, [dp.topk_ids, dp.gates, dp.offsets, dp.sorted_rows, dp.out, dp.y])


@pytest.mark.parametrize("path", [1, 2])
def test_graph_fused_combine(path):
    """route_group + the projection with the combine fused in: the arrival
    counters are set by the grouped GEMM's own pre-pass each replay (no memset
    node), so every replay sums each token once."""
    p = S.make_custom(E=16, N=400, K=256, T=300, k=4, x_per_slot=True, route="zipf+logits", combine=True)
    _announce(f"graph: route_group + expert_proj_combine_routed, path {path}")
    dp = DeviceProblem(p, path=path)
    _replay_matches(dp.run_fused, [dp.topk_ids, dp.gates, dp.offsets, dp.sorted_rows, dp.out, dp.y])


def test_graph_swiglu_gemm():
    p = S.make_custom(E=8, N=512, K=320, T=300, k=4, route="logits")
    _announce("graph: route_group + expert_proj_swiglu (GEMM)")
    dp = DeviceProblem(p, path=B.MXFP4_PATH_GEMM)

    def step():
        dp.route_group()
        dp.expert_proj_swiglu()
    _replay_matches(step, [dp.sorted_rows, dp.act])


def test_graph_decode_block():
    """The one-token MoE block: router -> single-launch gated decode -> projection + combine."""
    H, Inner, E, k = 2880, 512, 32, 4
    _announce("graph: one-token MoE block")
    r = S.make_router(1, H, E, tag=41)
    gu = S.make_custom(E=E, N=2 * Inner, K=H, T=1, k=k, route="logits", tag=42)
    gu.x = r.x
    dn = S.make_custom(E=E, N=H, K=Inner, T=1, k=k, x_per_slot=True, route="logits", tag=43, combine=True)
    d1, d2 = DeviceProblem(gu, path=B.MXFP4_PATH_GEMV), DeviceProblem(dn, path=B.MXFP4_PATH_GEMV)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    rw, rb = bf(r.w), bf(r.bias)
    d2.x = d1.act
    d2.topk_ids, d2.gates, d2.offsets, d2.sorted_rows = d1.topk_ids, d1.gates, d1.offsets, d1.sorted_rows

    def step():
        B.mxfp4_moe_router(d1.x, rw, rb, 1, H, E, d1.logits)
        d1.decode_swiglu()
        d2.proj_combine()
    _replay_matches(step, [d1.logits, d1.topk_ids, d1.act, d2.out, d2.y])
