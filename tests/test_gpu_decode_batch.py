"""The decode batch in one launch (mxfp4_moe_decode_batch and its gated form;
README "Dense routing", src/experts.linnet fn forward_topk).

Each case is compared with the separate calls route_group + expert_proj (or
expert_proj_swiglu) on the GEMV path bit for bit -- ids, gates, offsets,
sorted rows, error word and every output -- and with the oracle (routing bit
for bit, outputs within the projection's bound).  The shapes take both kernel
shapes of the multi-token GEMV (up to 4 tokens, and more), experts with more
rows than one pass holds, k = 1, k = E, up to 64 experts and tokens, partial
weight-row blocks, shared and per-slot inputs, T = 1 (the one-token decode),
batches with no more routed rows than experts (a workgroup row per routed
row), tokens with a NaN logit, and the model-size down decode of 64 tokens.
"""
import numpy as np
import pytest

import oracle.moe_oracle as O
from mxfp4_mixture_experts_amd import binding as B
from mxfp4_mixture_experts_amd import synthetic as S
from mxfp4_mixture_experts_amd.runner import DeviceProblem
from test_gpu_parity import check_close, check_routing, check_act

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0

BATCH_CASES = {
    # name: make_custom kwargs
    "two_tokens": dict(E=8, N=200, K=320, T=2, k=2, route="logits"),
    "four_tokens_per_slot": dict(E=32, N=192, K=2880, T=4, k=4, x_per_slot=True, route="logits"),
    "five_tokens": dict(E=16, N=136, K=256, T=5, k=3, route="logits"),
    "crowded_expert": dict(E=4, N=160, K=384, T=48, k=2, route="logits"),   # ~24 rows per expert: two passes
    "t37_top1": dict(E=32, N=392, K=640, T=37, k=1, route="logits"),
    "all_experts": dict(E=8, N=96, K=128, T=20, k=8, x_per_slot=True, route="logits"),
    "e64_t64": dict(E=64, N=130, K=3072, T=64, k=4, route="logits"),
    "e5_odd": dict(E=5, N=77, K=96, T=33, k=3, x_per_slot=True, route="logits"),
    "one_token": dict(E=32, N=200, K=2880, T=1, k=4, route="logits"),
    # T * k = E: the largest batch with one routed row per workgroup row
    "eight_tokens_rows_eq_experts": dict(E=32, N=192, K=2880, T=8, k=4, route="logits"),
    # T * k = E + 4: the smallest gpt-oss batch on the multi-token kernel
    "nine_tokens_rows_over_experts": dict(E=32, N=192, K=2880, T=9, k=4, x_per_slot=True, route="logits"),
}


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _separate(p, swiglu=False):
    dp = DeviceProblem(p, path=B.MXFP4_PATH_GEMV)
    dp.route_group()
    if swiglu:
        dp.expert_proj_swiglu()
    else:
        dp.expert_proj()
    return dp.results()


def _batch(p, swiglu=False):
    dp = DeviceProblem(p, path=B.MXFP4_PATH_GEMV)
    dp.out.fill_(float("nan"))
    dp.offsets.fill_(-7)
    dp.error_word.fill_(-1)
    if swiglu:
        dp.decode_batch_swiglu()
    else:
        dp.decode_batch()
    return dp.results()


def _same_routing(g, g2):
    for key in ("ids", "offsets", "error_word"):
        np.testing.assert_array_equal(g[key], g2[key], err_msg=key)
    np.testing.assert_array_equal(g["gates"], g2["gates"], err_msg="gates")
    n = int(g2["offsets"][-1])
    np.testing.assert_array_equal(g["sorted_rows"][:n], g2["sorted_rows"][:n], err_msg="sorted_rows")


@pytest.mark.parametrize("case", sorted(BATCH_CASES))
def test_decode_batch_cases(case):
    p = S.make_custom(**BATCH_CASES[case])
    p.name = case
    _announce(f"decode batch {case}")
    ref = O.run_problem(p)
    g = _batch(p)
    assert g["error_word"] == 0
    check_routing(g, ref)
    check_close(g["out"], ref["out"], ref["mag"], f"{case} out")
    g2 = _separate(p)
    _same_routing(g, g2)
    np.testing.assert_array_equal(g["out"], g2["out"])


@pytest.mark.parametrize("case", ["two_tokens", "five_tokens", "crowded_expert", "e64_t64", "one_token"])
def test_decode_batch_swiglu_cases(case):
    kw = dict(BATCH_CASES[case])
    kw["N"] += kw["N"] % 2
    kw.pop("x_per_slot", None)
    p = S.make_custom(**kw)
    p.name = case
    _announce(f"decode batch swiglu {case}")
    ref = O.run_problem(p)
    g = _batch(p, swiglu=True)
    assert g["error_word"] == 0
    check_routing(g, ref)
    check_act(g["act"], ref["out"], ref["mag"], f"{case} act")
    g2 = _separate(p, swiglu=True)
    _same_routing(g, g2)
    np.testing.assert_array_equal(g["act"], g2["act"])


@pytest.mark.parametrize("T,E,k", [(40, 16, 4), (6, 32, 4), (3, 8, 2)])
def test_decode_batch_nan_tokens(T, E, k):
    """Tokens with a NaN logit keep no expert: ids -1, gates 0, their rows left
    out of the grouping and of out, the range error; the other tokens as the
    separate calls.  (T * k <= E: the one-row-per-workgroup kernel.)"""
    N = 96
    _announce(f"decode batch with NaN logits T={T} E={E} k={k}")
    p = S.make_custom(E=E, N=N, K=256, T=T, k=k, route="logits", tag=810 + T)
    p.logits = p.logits.copy()
    bad = sorted({0, T // 2, T - 1})
    p.logits[0, 3] = NAN_BF16
    p.logits[T // 2, :] = NAN_BF16
    p.logits[T - 1, E - 1] = NAN_BF16
    g = _batch(p)
    assert g["error_word"] == B.MXFP4_ROUTE_ERR_ID_RANGE
    assert np.all(g["ids"][bad] == -1) and np.all(g["gates"][bad] == 0.0)
    out = g["out"].reshape(T, k, N)
    assert np.all(np.isnan(out[bad]))  # never written
    g2 = _separate(p)
    _same_routing(g, g2)
    good = [t for t in range(T) if t not in bad]
    np.testing.assert_array_equal(out[good], g2["out"].reshape(T, k, N)[good])


def test_decode_batch_model_size():
    """The gpt-oss-20b down decode of 64 tokens (E=32, N=K=2880, per-slot
    inputs): every output and the routing bit for bit against the separate
    calls, on repeated launches."""
    p = S.make_config(2)
    _announce(f"decode batch {p.name} (model size)")
    g2 = _separate(p)
    dp = DeviceProblem(p, path=B.MXFP4_PATH_GEMV)
    for rep in range(2):
        dp.out.fill_(float("nan"))
        dp.decode_batch()
        g = dp.results()
        assert g["error_word"] == 0
        _same_routing(g, g2)
        np.testing.assert_array_equal(g["out"], g2["out"])
