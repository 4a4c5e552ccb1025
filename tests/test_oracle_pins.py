"""Pins of the CPU oracle to what the pages fix and to independent computations.

No GPU.  Each test names the passage it follows (gpt-oss-20b files page).
"""
import numpy as np
import pytest

import oracle.moe_oracle as O
from conftest import read_golden
from mxfp4_mixture_experts_amd import synthetic as S


def _bf16(vals):
    return S.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


# ----------------------------------------------------------------- E2M1 codes
def test_e2m1_table_matches_page_fixture():
    """README "MXFP4": the sixteen code values."""
    table = O.e2m1_table()
    rows = [r.split() for r in read_golden("e2m1_codes.txt")]
    assert len(rows) == 16
    for code, val in rows:
        v = float(val)
        assert table[int(code)] == v
        assert np.signbit(table[int(code)]) == np.signbit(v)


def _e2m1_from_bits(c):
    """Independent decode from the bit fields: sign, 2 exponent bits (bias 1), 1 mantissa bit."""
    sign = -1.0 if (c >> 3) & 1 else 1.0
    e = (c >> 1) & 3
    m = c & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return sign * mag


def test_e2m1_bitfield_decode_and_twice_integer():
    """README "MXFP4": sign / exponent / mantissa fields; twice each value is an integer in 0..12."""
    table = O.e2m1_table()
    for c in range(16):
        assert table[c] == _e2m1_from_bits(c)
        twice = 2 * abs(table[c])
        assert twice == int(twice) and 0 <= twice <= 12
    assert sorted(set(2 * abs(table))) == [0, 1, 2, 3, 4, 6, 8, 12]


# ----------------------------------------------------------------- E8M0 scales
def test_e8m0_scale_examples():
    """README "MXFP4": 2 ** (scale - 127); 127 is x1, 115..136 is 2**-12..2**9."""
    for row in read_golden("e8m0_scales.txt"):
        b, lg = map(int, row.split())
        assert O.e8m0_factor(np.array([b], np.uint8))[0] == 2.0 ** lg


def test_e8m0_extremes_exact():
    f = O.e8m0_factor(np.array([0, 1, 254], np.uint8))
    assert f[0] == np.ldexp(1.0, -127) and f[1] == np.ldexp(1.0, -126) and f[2] == np.ldexp(1.0, 127)


# ----------------------------------------------------------------- layout facts
def test_format_counting_facts():
    """README "MXFP4" tensor table: 90 * 32 = 2880, 4.25 bits per weight, 530M elements."""
    facts = dict(r.split() for r in read_golden("mxfp4_format_facts.txt"))
    shape = tuple(int(v) for v in facts["gate_up_blocks_shape"].split(","))
    sshape = tuple(int(v) for v in facts["gate_up_scales_shape"].split(","))
    E, N, KB, B = shape
    assert B == int(facts["block_bytes"]) and sshape == (E, N, KB)
    assert KB * int(facts["block_elements"]) == int(facts["input_width"]) == 2880
    assert KB == int(facts["blocks_per_row"])
    # bits per weight from the storage of one block: 16 code bytes + 1 scale byte per 32 weights
    blocks = np.zeros((1, 1, 1, 16), np.uint8)
    scales = np.zeros((1, 1, 1), np.uint8)
    w = O.dequantize_mxfp4(blocks, scales)
    assert (blocks.nbytes + scales.nbytes) * 8 / w.size == float(facts["bits_per_weight"])
    # the page quotes the count truncated to millions (530,841,600 -> "530M")
    assert (E * N * KB * 32) // 10**6 == int(facts["gate_up_elements_per_layer_millions"])
    dshape = tuple(int(v) for v in facts["down_blocks_shape"].split(","))
    assert dshape[2] * 32 == 2880 and dshape[1] == 2880


# ----------------------------------------------------------------- nibble order
@pytest.mark.parametrize("j", [0, 1, 2, 7, 30, 31, 32, 33, 63])
@pytest.mark.parametrize("code", [1, 7, 9, 15])
def test_nibble_order_one_hot(j, code):
    """README "MXFP4": low nibble is the even element, high nibble the odd one.

    One nonzero code at element j, scale 127, x = e_j: the output is that code's value."""
    K, KB = 64, 2
    blocks = np.zeros((1, 1, KB, 16), np.uint8)
    byte = blocks[0, 0, j // 32, (j % 32) // 2]
    blocks[0, 0, j // 32, (j % 32) // 2] = byte | (code << (4 * (j % 2)))
    scales = np.full((1, 1, KB), 127, np.uint8)
    w = O.dequantize_mxfp4(blocks, scales)[0, 0]
    expect = np.zeros(K)
    expect[j] = O.E2M1_MAGNITUDES[code & 7] * (-1 if code & 8 else 1)
    np.testing.assert_array_equal(w, expect)
    x = np.zeros((1, K), np.float32)
    x[0, j] = 1.0
    out, mag = O.expert_proj(blocks, scales, _bf16(np.zeros((1, 1))), _bf16(x), False, np.zeros((1, 1), np.int32))
    assert out[0, 0, 0] == expect[j] and mag[0, 0, 0] == abs(expect[j])


# ----------------------------------------------------------------- external converter
def test_dequant_matches_transformers_converter():
    """README "Validation": the dequantization is bitwise equal to transformers'
    convert_moe_packed_tensors over random blocks and scales, all sixteen codes.
    The converter is called as a black box; it returns [E, K, Rows]."""
    torch = pytest.importorskip("torch")
    mx = pytest.importorskip("transformers.integrations.mxfp4")
    rng = np.random.default_rng(7)
    blocks = np.arange(256, dtype=np.uint8).reshape(1, 16, 1, 16).repeat(3, axis=2)
    blocks = np.concatenate([blocks, rng.integers(0, 256, (1, 16, 3, 16), dtype=np.uint8)], axis=0)
    scales = rng.integers(110, 145, (2, 16, 3), dtype=np.uint8)
    scales[0, :, 0] = 127
    ref = mx.convert_moe_packed_tensors(torch.from_numpy(blocks), torch.from_numpy(scales),
                                        dtype=torch.float32).numpy().astype(np.float64)
    ours = O.dequantize_mxfp4(blocks, scales)
    np.testing.assert_array_equal(ours.transpose(0, 2, 1), ref)


# ----------------------------------------------------------------- closed forms
@pytest.mark.parametrize("s", [127, 118, 130])
def test_closed_form_all_codes_one(s):
    """All codes 2 (value 1.0) and scale s: out[n] = 2**(s-127) * sum(x) + bias[n]."""
    E, N, K, T, k = 2, 5, 96, 3, 2
    blocks = np.full((E, N, K // 32, 16), 0x22, np.uint8)
    scales = np.full((E, N, K // 32), s, np.uint8)
    rng = np.random.default_rng(0)
    bias = _bf16(rng.normal(0, 0.02, (E, N)))
    x = _bf16(rng.standard_normal((T, K)))
    ids = np.array([[0, 1], [1, 0], [1, 0]], np.int32)
    out, _ = O.expert_proj(blocks, scales, bias, x, False, ids)
    xs = O.bf16_to_f64(x).sum(axis=1)
    b = O.bf16_to_f64(bias)
    for t in range(T):
        for sl in range(k):
            np.testing.assert_allclose(out[t, sl], 2.0 ** (s - 127) * xs[t] + b[ids[t, sl]], rtol=1e-14, atol=1e-14)


def test_projection_matches_dense_bruteforce():
    """The sparse top-k projection equals the dense form (every expert on every token,
    README "Dense routing") restricted to the chosen experts; the dense weights come from
    the independent bit-field decode, not from the oracle's table."""
    p = S.make_config(0)
    codes = np.stack([p.blocks & 15, p.blocks >> 4], axis=-1).reshape(p.E, p.N, p.K)
    dec = np.vectorize(_e2m1_from_bits)(codes)
    W = dec * (2.0 ** (np.repeat(p.scales.astype(np.int64), 32, axis=-1) - 127))
    x = O.bf16_to_f64(p.x)
    b = O.bf16_to_f64(p.bias)
    dense = np.einsum("enk,tk->ten", W, x) + b[None]            # [T, E, N]
    expect = np.take_along_axis(dense, p.ids_in[:, :, None].astype(np.int64), axis=1)
    out, mag = O.expert_proj(p.blocks, p.scales, p.bias, p.x, False, p.ids_in)
    np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-12)
    magd = np.einsum("enk,tk->ten", np.abs(W), np.abs(x))
    np.testing.assert_allclose(mag, np.take_along_axis(magd, p.ids_in[:, :, None].astype(np.int64), axis=1), rtol=1e-12)


def test_sampled_matches_full():
    p = S.make_custom(3, 40, 96, 5, 2, x_per_slot=True, route="ids")
    out, mag = O.expert_proj(p.blocks, p.scales, p.bias, p.x, True, p.ids_in)
    rows = np.array([0, 3, 9, 9, 4]); cols = np.array([0, 39, 17, 2, 5])
    v, m = O.expert_proj_sampled(p.blocks, p.scales, p.bias, p.x, True, p.ids_in, rows, cols)
    np.testing.assert_allclose(v, out.reshape(-1, 40)[rows, cols], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(m, mag.reshape(-1, 40)[rows, cols], rtol=1e-13)


# ----------------------------------------------------------------- routing
def _route_by_sorting(l, k):
    """Brute force: order experts by (-logit, index) and keep the first k."""
    return [sorted(range(len(l)), key=lambda e: (-l[e], e))[:k]]


def test_routing_tie_fixture():
    """README "Dense routing" / fn ranks: ties to the lower index, highest first."""
    for row in read_golden("routing_ties.txt"):
        ks, ls, es = [part.split() for part in row.split(";")]
        k = int(ks[0]); l = [float(v) for v in ls]; expect = [int(v) for v in es]
        ids, gates = O.route_topk(_bf16([l]), k)
        assert ids[0].tolist() == expect
        assert ids[0].tolist() == _route_by_sorting(l, k)[0]


@pytest.mark.parametrize("E,k", [(32, 4), (8, 2), (5, 5), (64, 8)])
def test_routing_matches_sort_with_many_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    l = rng.integers(-3, 4, (200, E)).astype(np.float32) * 0.5       # heavy ties, exact in bf16
    ids, _ = O.route_topk(_bf16(l), k)
    for t in range(200):
        assert ids[t].tolist() == _route_by_sorting(l[t].tolist(), k)[0]


def test_routing_matches_torch_topk_without_ties():
    """Without ties, the ranked selection is torch.topk's (README "Dense routing")."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    l = np.stack([rng.permutation(32) for _ in range(100)]).astype(np.float32) - 16
    ids, _ = O.route_topk(_bf16(l), 4)
    tk = torch.topk(torch.from_numpy(l), 4, dim=1, sorted=True).indices.numpy()
    np.testing.assert_array_equal(ids, tk)


def test_gates_equal_floored_full_softmax():
    """fn route: push every expert ranked TopK or worse to -1e30 and softmax over all
    experts: the floored entries are exactly zero and the kept ones are the gates."""
    rng = np.random.default_rng(5)
    bits = _bf16(rng.standard_normal((300, 32)))
    ids, gates = O.route_topk(bits, 4)
    l = O.bf16_to_f64(bits)
    ranks = O.expert_ranks(l)
    kept = np.where(ranks < 4, l, -1e30)
    z = np.exp(kept - kept.max(axis=1, keepdims=True))
    full = z / z.sum(axis=1, keepdims=True)
    assert np.all(full[ranks >= 4] == 0.0)
    np.testing.assert_allclose(np.take_along_axis(full, ids.astype(np.int64), axis=1), gates, rtol=1e-15, atol=0)
    np.testing.assert_allclose(gates.sum(axis=1), 1.0, rtol=1e-15)
    assert np.all(np.diff(gates, axis=1) <= 0)      # highest first


def test_dense_route_is_scattered_gates():
    """The oracle's dense weights: the sparse gates at the top-k ids, exact zeros
    elsewhere, rows summing to 1 (and ties ranked like the sparse routing)."""
    rng = np.random.default_rng(8)
    bits = _bf16(rng.standard_normal((200, 32)))
    bits[:20, 5] = bits[:20, 9]                          # ties
    ids, gates = O.route_topk(bits, 4)
    dense = O.dense_route(bits, 4)
    want = np.zeros_like(dense)
    np.put_along_axis(want, ids.astype(np.int64), gates, axis=1)
    np.testing.assert_allclose(dense, want, rtol=1e-15, atol=0)
    assert np.count_nonzero(dense, axis=1).max() == 4
    np.testing.assert_allclose(dense.sum(axis=1), 1.0, rtol=1e-15)


# ----------------------------------------------------------------- grouping
@pytest.mark.parametrize("T,E,k", [(0, 4, 2), (1, 32, 4), (37, 8, 3), (500, 32, 4)])
def test_grouping_bruteforce(T, E, k):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32) if T else np.zeros((0, k), np.int32)
    offsets, rows = O.group_by_expert(ids, E)
    flat = ids.reshape(-1).tolist()
    expect_rows, expect_off = [], [0]
    for e in range(E):
        mine = [r for r in range(len(flat)) if flat[r] == e]
        expect_rows += mine
        expect_off.append(expect_off[-1] + len(mine))
    assert offsets.tolist() == expect_off and rows.tolist() == expect_rows
    assert offsets[-1] == T * k


# ----------------------------------------------------------------- combine identities
def test_dense_routing_identity():
    """README "Dense routing": every expert on every token weighed by router
    probabilities that are zero outside the top k gives the same sum as the sparse
    form (here: projection + combine)."""
    p = S.make_custom(6, 48, 64, 7, 3, route="logits")
    ids, gates = O.route_topk(p.logits, p.k)
    out, mag = O.expert_proj(p.blocks, p.scales, p.bias, p.x, False, ids)
    y, _ = O.combine(out, gates, mag)
    l = O.bf16_to_f64(p.logits)
    ranks = O.expert_ranks(l)
    kept = np.where(ranks < p.k, l, -1e30)
    z = np.exp(kept - kept.max(axis=1, keepdims=True))
    prob = z / z.sum(axis=1, keepdims=True)                     # [T, E]
    W = O.dequantize_mxfp4(p.blocks, p.scales)                  # [E, N, K]
    dense = np.einsum("enk,tk->ten", W, O.bf16_to_f64(p.x)) + O.bf16_to_f64(p.bias)[None]
    y_dense = np.einsum("te,ten->tn", prob, dense)
    np.testing.assert_allclose(y, y_dense, rtol=1e-12, atol=1e-12)


def test_weight_before_down_identity():
    """README "Dense routing": weighing each expert's input by its router weight before
    the down projection equals weighing its output after (bias weighed separately)."""
    p = S.make_custom(5, 32, 64, 4, 2, x_per_slot=True, route="ids+logits")
    gates = O.gates_for_ids(p.logits, p.ids_in)
    out, _ = O.expert_proj(p.blocks, p.scales, p.bias, p.x, True, p.ids_in)
    y, _ = O.combine(out, gates)
    W = O.dequantize_mxfp4(p.blocks, p.scales)
    b = O.bf16_to_f64(p.bias)
    x = O.bf16_to_f64(p.x)                                       # [T, k, K]
    y2 = np.zeros_like(y)
    for t in range(p.T):
        for s in range(p.k):
            e = p.ids_in[t, s]
            y2[t] += W[e] @ (gates[t, s] * x[t, s]) + gates[t, s] * b[e]
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- planted mistakes
def test_pins_catch_swapped_nibbles(monkeypatch):
    """A plausible oracle mistake (high nibble read as the even element) must fail a pin."""
    def wrong_unpack(blocks):
        codes = np.stack([blocks >> 4, blocks & 0x0F], axis=-1)
        return codes.reshape(blocks.shape[:-2] + (blocks.shape[-2] * 32,))
    monkeypatch.setattr(O, "unpack_codes", wrong_unpack)
    with pytest.raises(AssertionError):
        test_nibble_order_one_hot(0, 7)


def test_pins_catch_wrong_scale_bias(monkeypatch):
    monkeypatch.setattr(O, "e8m0_factor", lambda s: np.ldexp(1.0, np.asarray(s).astype(np.int64) - 128))
    with pytest.raises(AssertionError):
        test_e8m0_scale_examples()


def test_pins_catch_tie_to_higher_index(monkeypatch):
    def wrong_ranks(logits):
        l = np.asarray(logits, dtype=np.float64)
        idx = np.arange(l.shape[-1])
        lj, le = l[:, None, :], l[:, :, None]
        return ((lj > le) | ((lj == le) & (idx[None, None, :] > idx[None, :, None]))).sum(-1)
    monkeypatch.setattr(O, "expert_ranks", wrong_ranks)
    with pytest.raises(AssertionError):
        test_routing_tie_fixture()


# ----------------------------------------------------------------- gated activation
def test_swiglu_constants_match_page_fixture():
    """src/experts.linnet: LIMIT and ALPHA."""
    vals = dict(r.split() for r in read_golden("swiglu_constants.txt"))
    assert O.SWIGLU_LIMIT == float(vals["LIMIT"]) and O.SWIGLU_ALPHA == float(vals["ALPHA"])


def _swiglu_scalar(g, u):
    """fn activate, one (gate, up) pair, with the math module."""
    import math
    g = min(g, 7.0)
    u = min(max(u, -7.0), 7.0)
    z = -1.702 * g
    if z > 700.0:
        return 0.0 * (u + 1.0)
    return (u + 1.0) * g / (1.0 + math.exp(z))


def test_swiglu_interleave_and_formula():
    """Even rows gate, odd rows multiply (the gate_up_blocks comment), fn activate's formula."""
    rng = np.random.default_rng(7)
    p = np.concatenate([rng.normal(0, 4, (5, 40)), [[9.0, 0.5, -9.0, 8.0, 0.3, -8.0, 7.5, 7.5, -1e4, 3.0, 1e4, -1.0]
                                                    + [0.0] * 28]], axis=0)
    f = O.swiglu(p)
    assert f.shape == (6, 20)
    for r in range(6):
        for i in range(20):
            assert f[r, i] == pytest.approx(_swiglu_scalar(p[r, 2 * i], p[r, 2 * i + 1]), rel=1e-13, abs=1e-300)


def test_swiglu_gate_term_matches_torch_silu():
    """g * sigmoid(ALPHA g) = silu(ALPHA g) / ALPHA, torch's float64 silu as the library routine."""
    import torch
    g = np.linspace(-60.0, 60.0, 2001)
    ref = torch.nn.functional.silu(torch.tensor(1.702 * g, dtype=torch.float64)).numpy() / 1.702
    np.testing.assert_allclose(O.gate_term(g), ref, rtol=1e-14, atol=1e-300)


def test_swiglu_special_cases():
    """fn activate: no gate gives nothing; an up of -1 cancels the + 1; the clamps."""
    h = lambda g: g / (1.0 + np.exp(-1.702 * g))
    cases = [((0.0, 3.0), 0.0), ((2.0, -1.0), 0.0), ((50.0, 0.0), h(7.0)), ((7.0, 100.0), 8.0 * h(7.0)),
             ((1.5, -100.0), -6.0 * h(1.5)), ((-1e6, 5.0), 0.0), ((-0.5, 2.0), 3.0 * h(-0.5))]
    for (g, u), want in cases:
        got = O.swiglu(np.array([g, u]))[0]
        assert np.isfinite(got) and got == pytest.approx(want, rel=1e-14, abs=1e-300), (g, u)


def test_gate_term_minimum():
    """The one minimum of g * sigmoid(ALPHA g), against scipy's bounded scalar minimizer."""
    from scipy.optimize import minimize_scalar
    res = minimize_scalar(lambda g: float(O.gate_term(np.float64(g))), bounds=(-3.0, 0.0), method="bounded",
                          options={"xatol": 1e-10})
    assert abs(res.x - O.GATE_TERM_ARGMIN) < 1e-6
    d = 1e-4
    assert O.gate_term(O.GATE_TERM_ARGMIN - d) > O.gate_term(O.GATE_TERM_ARGMIN)
    assert O.gate_term(O.GATE_TERM_ARGMIN + d) > O.gate_term(O.GATE_TERM_ARGMIN)


def test_swiglu_range_is_exact_on_boxes():
    """Brute force: the activation over a dense grid of each error box stays inside
    swiglu_range, and the range's ends are reached (to the grid's resolution)."""
    rng = np.random.default_rng(3)
    centers = np.concatenate([rng.normal(0, 3, (300, 2)), [[-0.75, 1.0], [6.9, 6.9], [-7.2, -6.9], [0.0, -1.0]]])
    half = np.concatenate([rng.uniform(0, 1.5, (300, 2)), [[0.3, 0.2], [0.3, 0.3], [0.5, 0.5], [0.4, 0.4]]])
    lo, hi = O.swiglu_range(centers - half, centers + half)
    t = np.linspace(0.0, 1.0, 81)
    for i in range(len(centers)):
        gg = centers[i, 0] - half[i, 0] + 2 * half[i, 0] * t
        uu = centers[i, 1] - half[i, 1] + 2 * half[i, 1] * t
        G, U = np.meshgrid(gg, uu)
        vals = O.swiglu(np.stack([G.ravel(), U.ravel()], axis=-1))[:, 0]
        assert vals.min() >= lo[i, 0] - 1e-12 and vals.max() <= hi[i, 0] + 1e-12, i
        span = hi[i, 0] - lo[i, 0]
        assert vals.min() <= lo[i, 0] + 0.02 * span + 1e-12 and vals.max() >= hi[i, 0] - 0.02 * span - 1e-12, i


def test_swiglu_bound_covers_bf16_rounding():
    """Exact projections: the bound is at least the bf16 rounding of the activation."""
    rng = np.random.default_rng(5)
    p = rng.normal(0, 3, (50, 64))
    f = O.swiglu(p)
    rounded = O.bf16_to_f64(S.f32_to_bf16_bits(f.astype(np.float32)))
    assert np.all(np.abs(rounded - f) <= O.swiglu_bound(p, np.zeros_like(p)))


def test_pins_catch_swapped_gate_and_up(monkeypatch):
    def wrong(gate_up):
        p = np.asarray(gate_up, dtype=np.float64)
        g = np.minimum(p[..., 1::2], 7.0)
        u = np.clip(p[..., 0::2], -7.0, 7.0)
        return (u + 1.0) * O.gate_term(g)
    monkeypatch.setattr(O, "swiglu", wrong)
    with pytest.raises(AssertionError):
        test_swiglu_interleave_and_formula()


def test_pins_catch_two_sided_gate_clamp(monkeypatch):
    def wrong(gate_up):
        p = np.asarray(gate_up, dtype=np.float64)
        g = np.clip(p[..., 0::2], -7.0, 7.0)
        u = np.clip(p[..., 1::2], -7.0, 7.0)
        return (u + 1.0) * O.gate_term(g)
    monkeypatch.setattr(O, "swiglu", wrong)
    with pytest.raises(AssertionError):
        test_swiglu_interleave_and_formula()


def test_pins_catch_wrong_slope(monkeypatch):
    monkeypatch.setattr(O, "SWIGLU_ALPHA", 1.0)
    with pytest.raises(AssertionError):
        test_swiglu_gate_term_matches_torch_silu()


# ----------------------------------------------------------------- router
def _bf16(a):
    return S.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_router_matches_loops():
    """src/experts.linnet, sub router (a Linear from H to the experts): brute force
    over (token, expert, j) with Python floats."""
    rng = np.random.default_rng(5)
    T, H, E = 3, 64, 5
    x = _bf16(rng.standard_normal((T, H)))
    w = _bf16(rng.standard_normal((E, H)) * 0.05)
    b = _bf16(rng.standard_normal(E) * 0.1)
    z, mag = O.router_logits(x, w, b)
    assert z.shape == (T, E) and mag.shape == (T, E)
    xf, wf, bf = O.bf16_to_f64(x), O.bf16_to_f64(w), O.bf16_to_f64(b)
    for t in range(T):
        for e in range(E):
            acc, m = float(bf[e]), abs(float(bf[e]))
            for j in range(H):
                p_ = float(xf[t, j]) * float(wf[e, j])
                acc += p_
                m += abs(p_)
            assert abs(z[t, e] - acc) <= 1e-12 * m
            assert abs(mag[t, e] - m) <= 1e-12 * m


def test_router_unit_rows_pick_columns():
    """Expert e's weight row is the unit vector at column c_e: its logit is
    x[t, c_e] + bias[e], exactly (a transposed operand or a shifted index fails)."""
    rng = np.random.default_rng(6)
    T, H, E = 4, 96, 6
    cols = [0, 5, 31, 32, 63, 95]
    w = np.zeros((E, H), np.float32)
    w[np.arange(E), cols] = 1.0
    x = _bf16(rng.standard_normal((T, H)))
    b = _bf16(rng.standard_normal(E))
    z, _ = O.router_logits(x, _bf16(w), b)
    np.testing.assert_array_equal(z, O.bf16_to_f64(x)[:, cols] + O.bf16_to_f64(b)[None, :])


def test_router_zero_input_is_bias():
    rng = np.random.default_rng(7)
    w = _bf16(rng.standard_normal((8, 64)))
    b = _bf16(rng.standard_normal(8))
    x = _bf16(np.zeros((2, 64)))
    z, mag = O.router_logits(x, w, b)
    np.testing.assert_array_equal(z, np.broadcast_to(O.bf16_to_f64(b), (2, 8)))
    z0, _ = O.router_logits(x, w, None)
    np.testing.assert_array_equal(z0, np.zeros((2, 8)))


def test_pins_catch_router_without_bias(monkeypatch):
    real = O.router_logits
    monkeypatch.setattr(O, "router_logits", lambda x, w, b=None: real(x, w, None))
    with pytest.raises(AssertionError):
        test_router_zero_input_is_bias()


# ----------------------------------------------------------------- inputs
def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], np.float32)
    bits = S.f32_to_bf16_bits(v)
    np.testing.assert_array_equal(O.bf16_to_f64(bits), [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0])


def test_tiny_config_matches_spec():
    p = S.make_config(0)
    assert p.blocks.shape == (4, 256, 4, 16) and p.scales.shape == (4, 256, 4)
    assert p.scales.min() >= 120 and p.scales.max() <= 132
    assert p.x.shape == (8, 128) and p.ids_in.shape == (8, 2)
    assert all(len(set(r)) == 2 for r in p.ids_in.tolist())
    assert abs(O.bf16_to_f64(p.bias).std() - 0.02) < 0.004
