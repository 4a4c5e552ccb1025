"""Tokens whose router logits hold a NaN.

A NaN compares false against every logit, so under the rank definition it
ranks first beside the largest finite logit and more than k experts qualify.
The routing then gives such a token id -1 in every slot (its rows are left out
of the grouping, as an out-of-range given id is), writes none of its gates and
reports MXFP4_ROUTE_ERR_ID_RANGE; every other token is routed and grouped as
the oracle does it.  The one-launch decode gives the same routing outputs and
projects nothing.
"""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mxfp4_mixture_experts_amd import binding as B
from mxfp4_mixture_experts_amd import synthetic as S
from test_gpu_parity import GATE_TOL

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0
SENT = -7


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _outputs(T, E, k):
    i32 = dict(dtype=torch.int32, device="cuda")
    return (torch.full((T, k), SENT, **i32), torch.full((T, k), 5.0, device="cuda"),
            torch.full((E + 1,), SENT, **i32), torch.full((T * k,), SENT, **i32), torch.full((1,), SENT, **i32))


def _np(ts):
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ts]


@pytest.mark.parametrize("T,E,k", [(8, 32, 4), (37, 32, 3), (300, 100, 5)])
def test_nan_tokens_left_out(T, E, k):
    """T * k <= 64 takes the one-workgroup route, larger T the grouping launch."""
    _announce(f"NaN logits route_group T={T} E={E} k={k}")
    p = S.make_custom(E=E, N=64, K=64, T=T, k=k, route="logits", tag=500 + T)
    lg = p.logits.copy()
    bad = sorted({1, T // 2})
    lg[1, 3] = NAN_BF16            # one NaN among finite logits
    lg[T // 2, :] = NAN_BF16       # a whole row of NaN
    outs = _outputs(T, E, k)
    B.mxfp4_moe_route_group(_dev_bf16(lg), None, T, E, k, *outs)
    ids, gates, off, rows, err = _np(outs)
    assert err[0] == B.MXFP4_ROUTE_ERR_ID_RANGE
    good = np.array([t for t in range(T) if t not in bad])
    ref_ids, ref_gates = O.route_topk(lg[good], k)
    np.testing.assert_array_equal(ids[good], ref_ids)
    assert np.all(ids[bad] == -1)
    assert np.all(gates[bad] == 5.0)               # not written
    assert np.abs(gates[good].astype(np.float64) - ref_gates).max() <= GATE_TOL
    # the grouping of the valid rows: stable by expert, the NaN tokens' rows absent
    flat = ids.reshape(-1)
    valid = np.flatnonzero(flat >= 0)
    want_rows = valid[np.argsort(flat[valid], kind="stable")]
    want_off = np.zeros(E + 1, dtype=np.int64)
    want_off[1:] = np.cumsum(np.bincount(flat[valid], minlength=E))
    np.testing.assert_array_equal(off, want_off)
    np.testing.assert_array_equal(rows[:valid.size], want_rows)
    assert np.all(rows[valid.size:] == SENT)


@pytest.mark.parametrize("whole_row", [False, True])
def test_nan_decode_projects_nothing(whole_row):
    E, k, N, K = 32, 4, 5760, 2880
    _announce(f"NaN logits one-launch decode whole_row={whole_row}")
    p = S.make_custom(E=E, N=N, K=K, T=1, k=k, route="logits", tag=520 + int(whole_row))
    lg = p.logits.copy()
    if whole_row:
        lg[0, :] = NAN_BF16
    else:
        lg[0, 7] = NAN_BF16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    blocks, scales, bias, x = dev(p.blocks), dev(p.scales), _dev_bf16(p.bias), _dev_bf16(p.x)
    ids, gates, off, rows, err = _outputs(1, E, k)
    out = torch.full((1, k, N), 3.0, device="cuda")
    B.mxfp4_moe_decode(_dev_bf16(lg), E, k, blocks, scales, bias, N, K, x, False, ids, gates, off, rows, out, err)
    ids, gates, off, rows, err, out = _np([ids, gates, off, rows, err, out])
    assert err[0] == B.MXFP4_ROUTE_ERR_ID_RANGE
    assert np.all(ids == -1)
    assert np.all(off == 0)
    assert np.all(rows == SENT) and np.all(gates == 5.0)
    assert np.all(out == 3.0)
    # the same routing outputs as the routing launch
    r = _outputs(1, E, k)
    B.mxfp4_moe_route_group(_dev_bf16(lg), None, 1, E, k, *r)
    rids, _, roff, rrows, rerr = _np(r)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_array_equal(off, roff)
    np.testing.assert_array_equal(rows, rrows)
    assert rerr[0] == err[0]
