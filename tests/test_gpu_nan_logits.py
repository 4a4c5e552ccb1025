"""Tokens whose router logits hold a NaN.

A NaN compares false against every logit, so it has no place under the rank
definition.  The routing gives such a token id -1 and gate 0 in every slot
(its rows are left out of the grouping, as an out-of-range given id is) and
reports MXFP4_ROUTE_ERR_ID_RANGE; every other token is routed and grouped as
the oracle does it, and the combine gives the NaN token y = 0.  The one-launch
decode gives the same routing outputs and projects nothing.  With k = E every
expert is kept, so the NaN must be detected as such (counting the experts of
rank below k would find exactly k of them).
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


@pytest.mark.parametrize("T,E,k", [(8, 32, 4), (37, 32, 3), (300, 100, 5), (12, 4, 4), (40, 8, 8)])
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
    assert np.all(gates[bad] == 0.0)
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
    # the combine of the routed rows: the NaN tokens' rows were never written
    # (NaN here), their zero gates give y = 0; the others as the oracle's combine
    N = 24
    proj = torch.full((T, k, N), float("nan"), device="cuda")
    vals = torch.from_numpy(np.random.default_rng(T).standard_normal((T, k, N)).astype(np.float32)).cuda()
    for t in good:
        proj[t] = vals[t]
    y = torch.full((T, N), 9.0, device="cuda")
    B.moe_combine(proj, outs[1], T, k, N, y)
    y, vals = _np([y, vals])
    assert np.all(y[bad] == 0.0)
    y_ref, mag = O.combine(vals[good].astype(np.float64), gates[good].astype(np.float64),
                           np.abs(vals[good]).astype(np.float64))
    assert np.all(np.abs(y[good] - y_ref) <= 1e-6 * mag + 1e-12)


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
    assert np.all(rows == SENT) and np.all(gates == 0.0)
    assert np.all(out == 3.0)
    # the same routing outputs as the routing launch
    r = _outputs(1, E, k)
    B.mxfp4_moe_route_group(_dev_bf16(lg), None, 1, E, k, *r)
    rids, rgates, roff, rrows, rerr = _np(r)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_array_equal(gates, rgates)
    np.testing.assert_array_equal(off, roff)
    np.testing.assert_array_equal(rows, rrows)
    assert rerr[0] == err[0]


def test_nan_decode_all_experts_kept():
    """k = E: every expert is kept, so a NaN logit must still be caught."""
    E = k = 8
    N, K = 96, 256
    _announce("NaN logits one-launch decode k = E")
    p = S.make_custom(E=E, N=N, K=K, T=1, k=k, route="logits", tag=530)
    lg = p.logits.copy()
    lg[0, 5] = NAN_BF16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    blocks, scales, bias, x = dev(p.blocks), dev(p.scales), _dev_bf16(p.bias), _dev_bf16(p.x)
    ids, gates, off, rows, err = _outputs(1, E, k)
    out = torch.full((1, k, N), 3.0, device="cuda")
    B.mxfp4_moe_decode(_dev_bf16(lg), E, k, blocks, scales, bias, N, K, x, False, ids, gates, off, rows, out, err)
    ids, gates, off, rows, err, out = _np([ids, gates, off, rows, err, out])
    assert err[0] == B.MXFP4_ROUTE_ERR_ID_RANGE
    assert np.all(ids == -1) and np.all(gates == 0.0) and np.all(off == 0)
    assert np.all(rows == SENT) and np.all(out == 3.0)
