"""CPU oracle for the MXFP4 mixture-of-experts expert projection.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The product path (the HIP library
and its binding) never calls it, and it shares no code with that path.

Everything here is the plain definition written out, in float64 with numpy,
without blocking, fusion or reordering:

* decode of one MXFP4 weight: the E2M1 code's value times 2 ** (scale - 127)
  (gpt-oss-20b files page, README section "MXFP4": the block format, the
  nibble order and the code set);
* routing: each expert's rank among a token's logits, ties to the lower index,
  the TopK best kept highest rank first, and the router weights as a softmax
  over the kept logits (same page, README section "Dense routing", and
  src/experts.linnet functions ``ranks``, ``route``, ``experts_of``,
  ``weights_of``);
* grouping: the routed rows (token, slot) bucketed by expert, ascending row
  index inside a bucket (README section "Loading": the tokens each expert was
  chosen for, one product over the tokens sorted by expert);
* projection: out[t, s, n] = bias[e, n] + sum_j W[e, n, j] * x_src[j] with
  e = ids[t, s] and x_src the token's input (gate/up, shared by the slots) or
  the slot's own input (down) (src/experts.linnet ``forward_topk``, the
  gate_up and down products);
* combine: y[t, n] = sum over slots of gate[t, s] * out[t, s, n]
  (src/experts.linnet ``forward_topk``: the f32 sum over k and the down bias
  carried by the router weights);
* router: logits[t, e] = bias[e] + sum_j x[t, j] * w[e, j], the Linear from
  the hidden width to the experts (src/experts.linnet block
  ``MixtureOfExperts``, ``sub router``; its output feeds ``ranks`` and
  ``route``), exact in float64 for bf16 inputs up to the final rounding;
* gated activation of the gate/up projection: even output rows are the gate,
  odd rows the multiplier; the gate is clamped from above at LIMIT = 7, the
  multiplier to [-7, 7], and the result is (up + 1) * gate *
  sigmoid(1.702 * gate) (src/experts.linnet: constants ``LIMIT`` and
  ``ALPHA``, fn ``activate``, the interleave comment on ``gate_up_blocks``).

Every function also returns, where the tolerance needs it, the magnitude
M = sum_j |W x| used by the parity bound |gpu - oracle| <= 2e-3 * M + 1e-5.

Parity status: every function here is pinned by tests/test_oracle_pins.py to
facts the pages fix or to an independent computation (see each docstring).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# MXFP4 decode
# ---------------------------------------------------------------------------

#: E2M1 magnitudes in code order 0..7 (README "MXFP4": the nibble is a sign,
#: two exponent bits and one mantissa bit selecting one of these, or its negative).
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_table() -> np.ndarray:
    """The 16 code values as float64: bit 3 is the sign, bits 0..2 index the magnitudes.

    Code 8 is negative zero.  Pinned by the page's code list, by an independent
    bit-field decode, and by the transformers converter.
    """
    mags = np.array(E2M1_MAGNITUDES, dtype=np.float64)
    return np.concatenate([mags, -mags])


def e8m0_factor(scale_bytes: np.ndarray) -> np.ndarray:
    """2 ** (scale - 127) exactly, as float64 (README "MXFP4": an exponent biased by 127).

    Bytes 0..254 are exact in float64.  Byte 255 is outside the format's use here.
    """
    s = np.asarray(scale_bytes).astype(np.int64)
    return np.ldexp(np.ones(s.shape, dtype=np.float64), s - 127)


def unpack_codes(blocks: np.ndarray) -> np.ndarray:
    """u8 [..., KB, 16] -> codes u8 [..., KB*32]: byte i holds element 2i in its
    low nibble and element 2i+1 in its high nibble (README "MXFP4")."""
    lo = blocks & 0x0F
    hi = blocks >> 4
    codes = np.stack([lo, hi], axis=-1)              # [..., KB, 16, 2]
    shape = blocks.shape[:-2] + (blocks.shape[-2] * 32,)
    return codes.reshape(shape)


def dequantize_mxfp4(blocks: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 -> float64 weights [..., Rows, K], in the checkpoint's own layout.

    blocks u8 [..., Rows, KB, 16], scales u8 [..., Rows, KB]; element j of a row
    is code (j) of block j // 32 times 2 ** (scales[..., j // 32] - 127).
    """
    blocks = np.asarray(blocks, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    assert blocks.shape[-1] == 16 and blocks.shape[:-1] == scales.shape
    values = e2m1_table()[unpack_codes(blocks)]                 # [..., Rows, KB*32]
    factor = np.repeat(e8m0_factor(scales), 32, axis=-1)        # [..., Rows, KB*32]
    return values * factor


# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (u16) -> float64, exactly (a bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# routing and grouping
# ---------------------------------------------------------------------------

def expert_ranks(logits: np.ndarray) -> np.ndarray:
    """rank[t, e] = #{j : l[t, j] > l[t, e] or (l[t, j] == l[t, e] and j < e)}.

    src/experts.linnet ``ranks``: the number of experts that beat expert e, ties
    going to the lower index; 0 is the largest.  logits float64 [T, E].
    """
    l = np.asarray(logits, dtype=np.float64)
    E = l.shape[-1]
    idx = np.arange(E)
    lj = l[:, None, :]          # [T, 1(e), E(j)]
    le = l[:, :, None]          # [T, E(e), 1]
    beats = (lj > le) | ((lj == le) & (idx[None, None, :] < idx[None, :, None]))
    return beats.sum(axis=-1).astype(np.int64)


def route_topk(logits_bits: np.ndarray, k: int):
    """Top-k routing from bf16 logits [T, E].

    Returns (ids int32 [T, k], gates float64 [T, k]): slot s holds the expert of
    rank s (``experts_of``: the highest-ranked first) and its router weight, the
    softmax over the k kept logits (``route``: the floored entries are exactly
    zero, so the kept probabilities are the softmax over the kept logits).
    """
    l = bf16_to_f64(logits_bits)
    T, E = l.shape
    assert 1 <= k <= E
    ranks = expert_ranks(l)
    ids = np.empty((T, k), dtype=np.int32)
    for s in range(k):
        ids[:, s] = np.argmax(ranks == s, axis=1)      # the unique expert of rank s
    return ids, softmax_at(l, ids)


def softmax_at(logits_f64: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over the logits at the given expert ids, per token, in float64."""
    kept = np.take_along_axis(np.asarray(logits_f64, dtype=np.float64), ids.astype(np.int64), axis=1)
    z = np.exp(kept - kept.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def dense_route(logits_bits: np.ndarray, k: int) -> np.ndarray:
    """The dense-routing weights [T, E] (``route``; README "Dense routing"): every
    expert ranked k or worse is floored to -1e30 and the softmax is taken over
    all E, in float64; the floored entries come out exactly zero."""
    l = bf16_to_f64(logits_bits)
    floored = np.where(expert_ranks(l) < k, l, -1e30)
    z = np.exp(floored - floored.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def router_logits(x_bits: np.ndarray, w_bits: np.ndarray, bias_bits: np.ndarray | None = None):
    """Router logits before any rounding (``sub router``, a Linear from H to the
    experts): z[t, e] = bias[e] + sum_j x[t, j] * w[e, j] in float64, with the
    magnitude mag[t, e] = |bias[e]| + sum_j |x[t, j] * w[e, j]|.

    x_bits [T, H] and w_bits [E, H] (row e = expert e) and bias_bits [E] are bf16
    bit patterns.  Pinned by loops over tiny inputs, unit weight rows (the
    logits are then columns of x plus the bias) and x = 0 (the bias)."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    z = x @ w.T
    mag = np.abs(x) @ np.abs(w).T
    if bias_bits is not None:
        b = bf16_to_f64(bias_bits)
        z = z + b[None, :]
        mag = mag + np.abs(b)[None, :]
    return z, mag


def gates_for_ids(logits_bits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Router weights for given expert ids: softmax over the chosen logits."""
    return softmax_at(bf16_to_f64(logits_bits), ids)


def group_by_expert(ids: np.ndarray, E: int):
    """Stable counting sort of the routed rows r = t * k + slot by expert.

    Returns (offsets int32 [E + 1], sorted_rows int32 [T * k]): offsets is the
    exclusive prefix sum of the per-expert row counts, offsets[E] = T * k, and
    the rows of expert e are sorted_rows[offsets[e]:offsets[e + 1]] in
    ascending order.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E)[:E]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_rows = np.empty(flat.size, dtype=np.int64)
    fill = offsets[:-1].copy()
    for r in range(flat.size):
        e = flat[r]
        sorted_rows[fill[e]] = r
        fill[e] += 1
    return offsets.astype(np.int32), sorted_rows.astype(np.int32)


# ---------------------------------------------------------------------------
# projection and combine
# ---------------------------------------------------------------------------

def _x_rows(x_bits: np.ndarray, x_per_slot: bool, T: int, k: int) -> np.ndarray:
    """float64 inputs per routed row [T * k, K]."""
    x = bf16_to_f64(x_bits)
    if x_per_slot:
        return x.reshape(T * k, -1)
    return np.repeat(x.reshape(T, -1), k, axis=0)


def expert_proj(blocks, scales, bias_bits, x_bits, x_per_slot: bool, ids: np.ndarray):
    """out[t, s, n] = bias[e, n] + sum_j W[e, n, j] * x_src[j], e = ids[t, s].

    Returns (out float64 [T, k, N], mag float64 [T, k, N]) where
    mag = sum_j |W[e, n, j] * x_src[j]| (the parity bound's scale; bias excluded).
    Each expert is dequantized once and multiplied by the rows routed to it.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    E, N = blocks.shape[0], blocks.shape[1]
    xr = _x_rows(x_bits, x_per_slot, T, k)
    bias = bf16_to_f64(bias_bits)
    out = np.zeros((T * k, N), dtype=np.float64)
    mag = np.zeros((T * k, N), dtype=np.float64)
    flat = ids.reshape(-1)
    for e in range(E):
        rows = np.nonzero(flat == e)[0]
        if rows.size == 0:
            continue
        w = dequantize_mxfp4(blocks[e], scales[e])           # [N, K]
        xe = xr[rows]                                         # [M, K]
        out[rows] = xe @ w.T + bias[e][None, :]
        mag[rows] = np.abs(xe) @ np.abs(w).T
    return out.reshape(T, k, N), mag.reshape(T, k, N)


def expert_proj_sampled(blocks, scales, bias_bits, x_bits, x_per_slot: bool, ids: np.ndarray,
                        rows: np.ndarray, cols: np.ndarray):
    """The same definition evaluated one output at a time, for sampled
    (row r = t * k + slot, column n) pairs.  Returns (values, mags) float64."""
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1)
    bias = bf16_to_f64(bias_bits)
    vals = np.empty(len(rows), dtype=np.float64)
    mags = np.empty(len(rows), dtype=np.float64)
    for i, (r, n) in enumerate(zip(rows, cols)):
        e = int(flat[r])
        w = dequantize_mxfp4(blocks[e, n], scales[e, n])     # [K]
        xs = bf16_to_f64(x_bits[r // k, r % k] if x_per_slot else x_bits[r // k])
        prod = w * xs
        vals[i] = prod.sum() + bias[e, n]
        mags[i] = np.abs(prod).sum()
    return vals, mags


def combine(out: np.ndarray, gates: np.ndarray, mag: np.ndarray | None = None):
    """y[t, n] = sum_s gates[t, s] * out[t, s, n]; also mag_y = sum_s gates * mag."""
    out = np.asarray(out, dtype=np.float64)
    g = np.asarray(gates, dtype=np.float64)
    y = np.einsum("ts,tsn->tn", g, out)
    mag_y = None if mag is None else np.einsum("ts,tsn->tn", np.abs(g), np.asarray(mag, dtype=np.float64))
    return y, mag_y


# ---------------------------------------------------------------------------
# gated activation (the gate/up projection's output -> the down projection's input)
# ---------------------------------------------------------------------------

#: ``swiglu_limit`` and the gate's sigmoid slope (src/experts.linnet, ``LIMIT`` and ``ALPHA``)
SWIGLU_LIMIT = 7.0
SWIGLU_ALPHA = 1.702


def gate_term(g: np.ndarray) -> np.ndarray:
    """h(g) = g * sigmoid(ALPHA * g) in float64; the logistic function is
    evaluated as 1 / (1 + e^-z) for z >= 0 and e^z / (1 + e^z) for z < 0, so
    no exponent overflows."""
    g = np.asarray(g, dtype=np.float64)
    z = SWIGLU_ALPHA * g
    ez = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1.0 / (1.0 + ez), ez / (1.0 + ez))
    return g * sig


def swiglu(gate_up: np.ndarray) -> np.ndarray:
    """activated[..., i] = (up + 1) * h(gate) with gate = min(p[..., 2 i], LIMIT)
    and up = clip(p[..., 2 i + 1], -LIMIT, LIMIT), for the biased gate/up
    projection p (fn ``activate``).  float64, last axis halved."""
    p = np.asarray(gate_up, dtype=np.float64)
    assert p.shape[-1] % 2 == 0
    g = np.minimum(p[..., 0::2], SWIGLU_LIMIT)
    u = np.clip(p[..., 1::2], -SWIGLU_LIMIT, SWIGLU_LIMIT)
    return (u + 1.0) * gate_term(g)


def _gate_term_argmin() -> float:
    """The g where h(g) = g * sigmoid(ALPHA * g) is smallest: h'(g) = 0 means
    1 + z * (1 - sigmoid(z)) = 0 for z = ALPHA * g, solved by bisection on
    [-3, 0] (h falls before it and rises after)."""
    lo, hi = -3.0, 0.0
    for _ in range(200):
        z = 0.5 * (lo + hi)
        if 1.0 + z * (1.0 - 1.0 / (1.0 + np.exp(-z))) > 0.0:
            hi = z
        else:
            lo = z
    return 0.5 * (lo + hi) / SWIGLU_ALPHA


GATE_TERM_ARGMIN = _gate_term_argmin()


def swiglu_range(gate_up_lo: np.ndarray, gate_up_hi: np.ndarray):
    """Exact range [min, max] of the activation over every projection between
    gate_up_lo and gate_up_hi (element-wise boxes).  The factor up + 1 is
    monotone in up; h(min(g, LIMIT)) is monotone except for its one minimum at
    GATE_TERM_ARGMIN; the range of a product of two intervals lies at the
    products of their ends."""
    lo = np.asarray(gate_up_lo, dtype=np.float64)
    hi = np.asarray(gate_up_hi, dtype=np.float64)
    a_lo = np.clip(lo[..., 1::2], -SWIGLU_LIMIT, SWIGLU_LIMIT) + 1.0
    a_hi = np.clip(hi[..., 1::2], -SWIGLU_LIMIT, SWIGLU_LIMIT) + 1.0
    g_lo = np.minimum(lo[..., 0::2], SWIGLU_LIMIT)
    g_hi = np.minimum(hi[..., 0::2], SWIGLU_LIMIT)
    h_lo_end, h_hi_end = gate_term(g_lo), gate_term(g_hi)
    inside = (g_lo <= GATE_TERM_ARGMIN) & (GATE_TERM_ARGMIN <= g_hi)
    b_lo = np.where(inside, gate_term(np.float64(GATE_TERM_ARGMIN)), np.minimum(h_lo_end, h_hi_end))
    b_hi = np.maximum(h_lo_end, h_hi_end)
    corners = np.stack([a_lo * b_lo, a_lo * b_hi, a_hi * b_lo, a_hi * b_hi])
    return corners.min(axis=0), corners.max(axis=0)


def swiglu_bound(gate_up: np.ndarray, mag: np.ndarray) -> np.ndarray:
    """|gpu - swiglu(p)| allowed per bf16 activation when each fp32 projection
    output may be off by parity_bound(mag): the activation's exact deviation
    over that error box, plus the final rounding to bf16 (half a unit in the
    last of 8 significant bits, <= 2^-8 relative), plus fp32 evaluation
    (the fp32 rounding of ALPHA * log2(e) * gate and hardware exp2 and
    reciprocal within 1 ulp each: 4e-6 relative, and 2e-5 absolute)."""
    p = np.asarray(gate_up, dtype=np.float64)
    e = parity_bound(mag)
    f = swiglu(p)
    f_min, f_max = swiglu_range(p - e, p + e)
    dev = np.maximum(f_max - f, f - f_min)
    return dev + (2.0 ** -8 + 4e-6) * (np.abs(f) + dev) + 2e-5


def parity_bound(mag: np.ndarray) -> np.ndarray:
    """|gpu - oracle| allowed per fp32 output: 2e-3 * sum|w x| + 1e-5."""
    return 2e-3 * np.asarray(mag, dtype=np.float64) + 1e-5


def run_problem(p):
    """The whole path for one synthetic problem: routing (or given ids), grouping,
    projection and, where the problem asks, the combine.  Returns a dict."""
    res = {}
    if p.ids_in is not None:
        ids = np.asarray(p.ids_in, dtype=np.int32)
        gates = gates_for_ids(p.logits, ids) if p.logits is not None else None
    else:
        ids, gates = route_topk(p.logits, p.k)
    res["ids"], res["gates"] = ids, gates
    res["offsets"], res["sorted_rows"] = group_by_expert(ids, p.E)
    res["out"], res["mag"] = expert_proj(p.blocks, p.scales, p.bias, p.x, p.x_per_slot, ids)
    if p.combine and gates is not None:
        res["y"], res["mag_y"] = combine(res["out"], gates, res["mag"])
    return res
