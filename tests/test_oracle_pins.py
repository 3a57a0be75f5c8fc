"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed forms,
brute force on tiny inputs, special cases that reduce to a numpy library routine
(``@`` on matrices decoded here by numpy's own fp16/bf16 views), exact round
trips, byte layouts written out from the pages' figure, and byte counts printed
on the pages.  No GPU is involved.
"""
import dataclasses
import itertools
import math
import os

import numpy as np
import pytest

import qsmoe_synth as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ independent decoders
def np_f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def np_bf16(bits):
    with np.errstate(invalid="ignore"):
        return np_bf16_raw(bits)


def np_bf16_raw(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_codes(codes_row_bytes, bits):
    """unsigned codes of one stack of rows, [..., cols]; 4-bit: low nibble first."""
    c = np.asarray(codes_row_bytes, dtype=np.uint8)
    if bits == 8:
        return c.astype(np.float64)
    lo = (c & 0x0F).astype(np.float64)
    hi = (c >> 4).astype(np.float64)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def np_dequant(qm, e, row0=0, rows=None):
    rows = qm.codes.shape[1] - row0 if rows is None else rows
    q = np_codes(qm.codes[e, row0:row0 + rows], qm.bits)
    dec = np_bf16 if qm.sb_dtype == "bf16" else np_f16
    s = np.repeat(dec(qm.scales[e, row0:row0 + rows]), 64, axis=1)
    b = np.repeat(dec(qm.biases[e, row0:row0 + rows]), 64, axis=1)
    return s * q + b


def np_silu(z):
    return z / (1.0 + np.exp(-z))


def np_mlp(L, gu, dn, e, xf):
    """dense SwiGLU MLP of expert e on rows xf [T, H] via numpy matmul."""
    I = L.inter
    Wg = np_dequant(gu, e, 0, I)
    Wu = np_dequant(gu, e, I, I)
    Wd = np_dequant(dn, e)
    h = np_silu(xf @ Wg.T) * (xf @ Wu.T)
    return h @ Wd.T


def np_logits(L, x):
    l = np_bf16(x) @ np_bf16(L.router_w).T
    if L.router_bias is not None:
        l = l + L.router_bias.astype(np.float64)
    return l


def np_layer(L, x, idx, w):
    """a second, vectorised numpy implementation of the whole layer."""
    xf = np_bf16(x)
    T = xf.shape[0]
    y = np.zeros((T, L.hidden))
    for e in np.unique(idx):
        rows, js = np.nonzero(idx == e)
        o = np_mlp(L, L.gate_up, L.down, int(e), xf[rows])
        y[rows] += w[rows, js][:, None] * o
    if L.has_shared:
        g = 1.0
        if L.shared_gate_w is not None:
            g = (1.0 / (1.0 + np.exp(-(xf @ np_bf16(L.shared_gate_w)))))[:, None]
        y += g * np_mlp(L, L.s_gate_up, L.s_down, 0, xf)
    return y


# ------------------------------------------------------------------- 16-bit formats
def test_f16_decoder_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = np_f16(bits)
    got = np.array([orc.f16_to_double(int(b)) for b in bits[::7]])
    r = ref[::7]
    fin = np.isfinite(r)
    assert np.array_equal(got[fin], r[fin])
    assert np.array_equal(np.isnan(got), np.isnan(r))
    assert np.array_equal(np.isinf(got), np.isinf(r))
    # special values named by IEEE 754 binary16
    assert orc.f16_to_double(0x3C00) == 1.0
    assert orc.f16_to_double(0x0001) == 2.0 ** -24
    assert orc.f16_to_double(0x7BFF) == 65504.0
    assert orc.f16_to_double(0xC000) == -2.0


def test_f16_encoder_matches_numpy(orc):
    """The oracle's binary64 -> binary16 encoder (it writes the Q8_0 scales) against
    numpy's own conversion, which rounds a double to the nearest half directly, ties to
    even: 1e5 random doubles over the whole half range (normal, subnormal, overflow),
    then every kind of exact halfway point between neighbouring halves and the doubles
    just beside them, where a wrong tie rule or a double rounding would show."""
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-27.0, 17.0, 100_000)) * rng.choice([-1.0, 1.0], 100_000)
    with np.errstate(over="ignore"):
        ref = mag.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.f64_to_f16(mag), ref)
    # halfway points: between half h and its successor (all finite non-negative halves)
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2                                    # exact in binary64
    for v in (mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf), -mid):
        assert np.array_equal(orc.f64_to_f16(v), v.astype(np.float16).view(np.uint16))
    even = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(orc.f64_to_f16(mid), even)       # ties to the even pattern
    # the largest half, the overflow threshold (65520 = 65504 + half an ulp) and zero signs
    edge = np.array([65504.0, 65519.99, 65520.0, 1e9, 0.0, -0.0, 2.0 ** -25, 2.0 ** -24 * 1.5])
    assert orc.f64_to_f16(edge).tolist() == [0x7BFF, 0x7BFF, 0x7C00, 0x7C00, 0x0000, 0x8000, 0x0000, 0x0002]


def test_bf16_decoder_all_patterns(orc):
    bits = np.arange(0, 65536, 5, dtype=np.uint32).astype(np.uint16)
    ref = np_bf16(bits)
    got = np.array([orc.bf16_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert orc.bf16_to_double(0x3F80) == 1.0
    assert orc.bf16_to_double(0x0001) == 2.0 ** -133


# ------------------------------------------------------------------ affine codes
@pytest.mark.parametrize("bits", [4, 8])
def test_affine_requant_identity(orc, bits):
    """(W - b) / s recovers every code exactly: pins nibble order and group index."""
    L = syn.make_layer(256, 128, 4, 2, bits, seed=3)
    qm = L.gate_up
    for e in range(L.n_experts):
        W = orc.dequant_matrix(qm, e)
        s = np.repeat(np_f16(qm.scales[e]), 64, axis=1)
        b = np.repeat(np_f16(qm.biases[e]), 64, axis=1)
        q = (W - b) / s
        assert np.array_equal(np.round(q), np_codes(qm.codes[e], bits))
        assert np.max(np.abs(q - np.round(q))) < 1e-9


def test_affine_hand_built_row(orc):
    """A row built by hand: codes 0..15 repeating, s = 2^-4, b = -1/2 in group 0 and
    s = 1, b = 3 in group 1 -> W values written out directly."""
    q = np.array([c % 16 for c in range(128)], dtype=np.uint8)
    packed = (q[0::2] | (q[1::2] << 4)).astype(np.uint8)       # column 2i -> low nibble
    qm = syn.QMat(codes=packed.reshape(1, 1, 64),
                  scales=np.array([[[0x2C00, 0x3C00]]], dtype=np.uint16),   # 2^-4, 1.0
                  biases=np.array([[[0xB800, 0x4200]]], dtype=np.uint16),   # -0.5, 3.0
                  bits=4)
    W = orc.dequant_matrix(qm, 0)[0]
    expect = [(c % 16) / 16.0 - 0.5 for c in range(64)] + [(c % 16) + 3.0 for c in range(64, 128)]
    assert W.tolist() == expect


# ------------------------------------------------------------------------- router
def test_topk_brute_force_tiny(orc):
    """Every C(16,2) subset is tried: the selected set is the unique one whose every
    member beats every non-member."""
    L = syn.make_layer(**syn.TINY)
    x = syn.make_x(64, L.hidden, seed=5)
    ol = orc.OracleLayer(L)
    logits = np_logits(L, x)
    assert np.allclose(orc.router_logits(ol, x), logits, rtol=0, atol=1e-12)
    idx, w, gap = orc.route(ol, x)
    E, k = L.n_experts, L.top_k
    for t in range(x.shape[0]):
        winners = [S for S in itertools.combinations(range(E), k)
                   if min(logits[t, list(S)]) > max(np.delete(logits[t], list(S)))]
        assert len(winners) == 1
        assert tuple(idx[t]) == winners[0]
        srt = np.sort(logits[t])[::-1]
        assert gap[t] == pytest.approx(srt[k - 1] - srt[k], abs=1e-12)


def test_route_zero_input_closed_form(orc):
    """x = 0 and no bias: every logit is 0, ties go to the lowest ids, w = 1/k."""
    L = syn.make_layer(**syn.TINY)
    x = np.zeros((3, L.hidden), dtype=np.uint16)
    idx, w, _ = orc.route(orc.OracleLayer(L), x)
    assert (idx == np.arange(L.top_k)).all()
    assert (w == 1.0 / L.top_k).all()


def test_route_k_equals_E_is_full_softmax(orc):
    L = syn.make_layer(256, 128, 16, 16, 8, seed=1, router_std=0.05)
    x = syn.make_x(8, 256, seed=2)
    idx, w, gap = orc.route(orc.OracleLayer(L), x)
    l = np_logits(L, x)
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    assert (idx == np.arange(16)).all()
    assert np.allclose(w, p, rtol=1e-13, atol=0)
    assert np.isinf(gap).all()


def test_route_weights_are_softmax_of_selection(orc):
    """renormalised full-softmax probabilities equal a softmax over the selected
    logits alone, and sum to one (with and without a router bias)."""
    for zipf in (None, 1.1):
        L = syn.make_layer(256, 128, 64, 8, 4, seed=4, zipf_s=zipf)
        x = syn.make_x(16, 256, seed=9)
        idx, w, _ = orc.route(orc.OracleLayer(L), x)
        l = np.take_along_axis(np_logits(L, x), idx, axis=1)
        p = np.exp(l - l.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        assert np.allclose(w, p, rtol=1e-13, atol=0)
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
        assert (np.diff(idx, axis=1) > 0).all()          # ascending expert id


# ----------------------------------------------------------------------- FFN paths
def test_single_expert_reduces_to_dense_mlp(orc):
    """E = 1, k = 1, no shared expert: w = 1 exactly and y is the dense SwiGLU MLP,
    i.e. three dense GEMVs (numpy matmul on independently decoded weights)."""
    for bits in (4, 8):
        L = syn.make_layer(256, 128, 1, 1, bits, seed=6, has_shared=False)
        x = syn.make_x(5, 256, seed=1)
        y, idx, w = orc.layer_forward(orc.OracleLayer(L), x)
        assert (idx == 0).all() and (w == 1.0).all()
        ref = np_mlp(L, L.gate_up, L.down, 0, np_bf16(x))
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_zero_routed_weights_leaves_shared_only(orc):
    L = syn.make_layer(**syn.TINY)
    for qm in (L.gate_up, L.down):
        qm.scales[:] = 0
        qm.biases[:] = 0
    x = syn.make_x(4, L.hidden, seed=0)
    y, _, _ = orc.layer_forward(orc.OracleLayer(L), x)
    ref = np_mlp(L, L.s_gate_up, L.s_down, 0, np_bf16(x))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_no_shared_is_routed_only(orc):
    L = syn.make_layer(256, 128, 16, 2, 8, seed=0, router_std=0.02, has_shared=False)
    x = syn.make_x(6, 256, seed=4)
    y, idx, w = orc.layer_forward(orc.OracleLayer(L), x)
    ref = np_layer(L, x, idx, w)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("cfg,T", [("TINY", 4), ("DECODE", 2)])
def test_whole_layer_matches_numpy_implementation(orc, cfg, T):
    L = syn.make_layer(**getattr(syn, cfg))
    x = syn.make_x(T, L.hidden, seed=0)
    y, idx, w = orc.layer_forward(orc.OracleLayer(L), x)
    ref = np_layer(L, x, idx, w)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(y - ref)) <= 1e-12 * rms


@pytest.mark.parametrize("variant", ["bf16", "gate", "bf16+gate"])
def test_checkpoint_variants_match_numpy_implementation(orc, variant):
    """bf16 scales and biases, and the shared-expert gate, through the whole layer
    against the numpy implementation (its own bf16 decoder and sigmoid)."""
    L = syn.make_layer(**syn.TINY, scale_dtype="bf16" if "bf16" in variant else "f16",
                       shared_gate="gate" in variant)
    x = syn.make_x(5, L.hidden, seed=3)
    y, idx, w = orc.layer_forward(orc.OracleLayer(L), x)
    ref = np_layer(L, x, idx, w)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


def test_bf16_scales_equal_fp16_scales_on_common_values(orc):
    """Scale and bias values held exactly by both formats (8 significant bits, fp16
    normal range) give the same layer bit for bit whichever format stores them."""
    Lh = syn.make_layer(**syn.TINY)
    for qm in (Lh.gate_up, Lh.down, Lh.s_gate_up, Lh.s_down):
        for arr in (qm.scales, qm.biases):
            v = syn.bf16_bits_to_f32(syn.to_bf16_bits(np_f16(arr)))       # 8 significant bits
            arr[:] = v.astype(np.float16).view(np.uint16)
            assert np.array_equal(np_f16(arr), v.astype(np.float64))
    Lb = dataclasses.replace(Lh, scale_dtype="bf16")
    for name in ("gate_up", "down", "s_gate_up", "s_down"):
        qh = getattr(Lh, name)
        setattr(Lb, name, dataclasses.replace(qh, sb_dtype="bf16", scales=syn.to_bf16_bits(np_f16(qh.scales)),
                                              biases=syn.to_bf16_bits(np_f16(qh.biases))))
    x = syn.make_x(4, Lh.hidden, seed=9)
    yh, ih, wh = orc.layer_forward(orc.OracleLayer(Lh), x)
    yb, ib, wb = orc.layer_forward(orc.OracleLayer(Lb), x)
    assert np.array_equal(yh, yb) and np.array_equal(ih, ib)


def test_shared_gate_closed_forms(orc):
    """The gate only scales the shared expert's output: with g = 0 it is exactly 1/2 of
    it; with g x >> 0 the whole of it, with g x << 0 none of it; per token the
    difference to the no-shared layer is sigmoid(g . x) times the ungated difference."""
    L = syn.make_layer(**syn.TINY, shared_gate=True)
    x = syn.make_x(6, L.hidden, seed=5)
    ol = orc.OracleLayer(L)
    y, idx, w = orc.layer_forward(ol, x)
    y1 = orc.layer_forward_with_routing(orc.OracleLayer(dataclasses.replace(L, shared_gate_w=None)), x, idx, w)
    y0 = orc.layer_forward_with_routing(orc.OracleLayer(dataclasses.replace(L, has_shared=False,
                                                                            shared_gate_w=None)), x, idx, w)
    sig = 1.0 / (1.0 + np.exp(-(np_bf16(x) @ np_bf16(L.shared_gate_w))))
    assert np.allclose(y - y0, sig[:, None] * (y1 - y0), rtol=1e-12, atol=1e-14)
    half = orc.layer_forward_with_routing(orc.OracleLayer(dataclasses.replace(
        L, shared_gate_w=np.zeros(L.hidden, np.uint16))), x, idx, w)
    assert np.allclose(half - y0, 0.5 * (y1 - y0), rtol=1e-13, atol=1e-15)
    xs = syn.make_x(1, L.hidden, seed=6)
    big = syn.to_bf16_bits(np_bf16(xs[0]) * 40.0 / np.sum(np_bf16(xs[0]) ** 2) * 2)  # g . x ~ 80
    for sign, ref in ((1, y1), (-1, y0)):
        gw = big if sign > 0 else big ^ np.uint16(0x8000)
        ys = orc.layer_forward_with_routing(orc.OracleLayer(dataclasses.replace(L, shared_gate_w=gw)),
                                            xs, idx[:1], w[:1])
        r1 = orc.layer_forward_with_routing(orc.OracleLayer(dataclasses.replace(
            L, shared_gate_w=None, has_shared=sign > 0)), xs, idx[:1], w[:1])
        assert np.allclose(ys, r1, rtol=1e-12, atol=1e-14)


def test_fused_equals_separate_gate_up(orc):
    """[gate; up] concatenated along the output axis gives the same result as two
    separate matrices (oMLX, fusion principle: rows are independent)."""
    L = syn.make_layer(**syn.TINY)
    x = syn.make_x(4, L.hidden, seed=2)
    y1, _, _ = orc.layer_forward(orc.OracleLayer(L, separate=False), x)
    y2, _, _ = orc.layer_forward(orc.OracleLayer(L, separate=True), x)
    assert np.array_equal(y1, y2)


def test_forward_with_given_routing(orc):
    L = syn.make_layer(**syn.TINY)
    x = syn.make_x(4, L.hidden, seed=7)
    ol = orc.OracleLayer(L)
    y, idx, w = orc.layer_forward(ol, x)
    assert np.array_equal(orc.layer_forward_with_routing(ol, x, idx, w), y)
    # a different routing changes y exactly as the numpy implementation says
    idx2 = (idx + 3) % L.n_experts
    w2 = np.full_like(w, 0.5)
    y2 = orc.layer_forward_with_routing(ol, x, idx2, w2)
    assert np.allclose(y2, np_layer(L, x, idx2, w2), rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- Q8_0
def _read_golden_tile():
    entries, scales = [], []
    with open(os.path.join(GOLDEN, "q8_tile_layout.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            kind, *vals = line.split()
            if kind == "code":
                entries.append(tuple(int(v) for v in vals))
            elif kind == "scale":
                scales.append(tuple(int(v) for v in vals))
    return entries, scales


def test_q8_tile_layout_golden(orc):
    """Byte positions inside one 544-byte tile, written out from the page's figure."""
    N, K = 16, 32
    rows = np.zeros((N, 1, 34), dtype=np.uint8)
    for r in range(16):
        rows[r, 0, 0] = 0xA0 + r          # scale low byte
        rows[r, 0, 1] = 0x30 + r          # scale high byte
        rows[r, 0, 2:] = [(r * 32 + c) % 251 for c in range(32)]
    tile = orc.q8_pack_rows16(rows, N, K)
    assert tile.size == 544 == 16 * 34
    entries, scales = _read_golden_tile()
    assert len(entries) >= 16 and len(scales) == 16
    for r, c, off in entries:
        assert tile[off] == (r * 32 + c) % 251, (r, c, off)
    for r, off in scales:
        assert tile[off] == 0xA0 + r and tile[off + 1] == 0x30 + r


def test_q8_pack_unpack_identity(orc):
    N, K = 64, 256
    rows = syn.make_q8_rows(N, K, seed=3)
    tiles = orc.q8_pack_rows16(rows, N, K)
    assert tiles.size == rows.size
    back = orc.q8_unpack_rows16(tiles, N, K)
    assert np.array_equal(back, rows)
    # packing moves bytes only: same multiset of bytes per 16-row panel / block
    assert np.array_equal(np.sort(tiles), np.sort(rows.reshape(-1)))
    # packing twice from the same rows gives the same bytes (pure, idempotent)
    assert np.array_equal(orc.q8_pack_rows16(rows, N, K), tiles)


def test_q8_gemv_reduces_to_numpy(orc):
    N, K = 48, 512
    rows = syn.make_q8_rows(N, K, seed=1)
    x = syn.make_x(1, K, seed=2)[0]
    y = orc.q8_gemv(rows, N, K, x)
    d = np_f16(rows[:, :, 0:2].copy().view(np.uint16)[..., 0])           # [N, K/32]
    q = rows[:, :, 2:].view(np.int8).astype(np.float64)                 # [N, K/32, 32]
    W = (d[:, :, None] * q).reshape(N, K)
    ref = W @ np_bf16(x)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


def test_q8_block_round_trips(orc):
    rng = np.random.default_rng(0)
    K = 32 * 64
    # quant(dequant(q, d)) == (q, d) whenever max|q| == 127 in the block
    blocks = syn.make_q8_rows(1, K, seed=8)[0]
    q = blocks[:, 2:].view(np.int8)
    q[:, 0] = np.where(rng.random(K // 32) < 0.5, 127, -127).astype(np.int8)
    v = orc.q8_dequantize_row(blocks, K).astype(np.float32)
    assert np.array_equal(v.astype(np.float64), orc.q8_dequantize_row(blocks, K))  # exact in fp32
    again = orc.q8_quantize_row(v)
    assert np.array_equal(again, blocks)
    # |dequant(quant(v)) - v| <= d/2 + 127 |d - fp16(d)| for arbitrary floats
    v = rng.standard_normal(K).astype(np.float32) * 3
    blk = orc.q8_quantize_row(v)
    back = orc.q8_dequantize_row(blk, K)
    vb = v.reshape(-1, 32).astype(np.float64)
    d = (np.abs(v.reshape(-1, 32)).max(1) / np.float32(127)).astype(np.float64)
    d16 = np_f16(blk[:, 0:2].copy().view(np.uint16)[:, 0])
    bound = d / 2 + 127 * np.abs(d - d16)
    err = np.abs(back.reshape(-1, 32) - vb)
    assert (err <= bound[:, None] * (1 + 1e-6)).all()
    # all-zero block: d = 0, q = 0
    z = orc.q8_quantize_row(np.zeros(32, dtype=np.float32))
    assert (z == 0).all()


def bf16_bits(vals):
    """bf16 bit patterns of values that bf16 holds exactly (checked)."""
    v = np.asarray(vals, dtype=np.float32)
    b = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(np_bf16(b), v.astype(np.float64))
    return b


def test_q8x_quantizer_hand_example(orc):
    """Activation blocks whose codes follow by hand from the reading: d = max|x| / 127,
    q = x / d rounded half away from zero.  max|x| = 127 gives d = 1 (codes = x rounded);
    max|x| = 254 gives d = 2; a zero block gives d = 0 and zero codes.  The halves (0.5,
    -2.5, 63.5, -100.5, 3 / 2) tell half-away-from-zero from round-to-nearest-even."""
    b0 = [127, -127, 0.5, -0.5, 1.5, -2.5, 63.5, 0, 2.25, -100.5] + [0] * 22
    q0 = [127, -127, 1, -1, 2, -3, 64, 0, 2, -101] + [0] * 22
    b1 = [254, 3, -5, 7, -1, 0.5] + [0] * 26
    q1 = [127, 2, -3, 4, -1, 0] + [0] * 26          # 3/2 -> 2, -5/2 -> -3, 7/2 -> 4, -1/2 -> -1
    x = bf16_bits(b0 + b1 + [0] * 32)
    q, d = orc.q8_quantize_x(x)
    assert q.tolist() == q0 + q1 + [0] * 32
    assert np_f16(d).tolist() == [1.0, 2.0, 0.0]


def test_q8x_quantizer_invariants(orc):
    """Random activations: codes in [-127, 127], each nonzero block reaches |q| = 127,
    q(-x) = -q(x), q(2x) = q(x) with d doubled (powers of two are exact), and the round
    trip |fp16(d) q - x| <= d/2 + 127 |d - fp16(d)| with d = max|x| / 127."""
    K = 32 * 96
    x = syn.make_x(1, K, seed=12)[0]
    x[32:64] = 0                                    # one all-zero block
    q, d = orc.q8_quantize_x(x)
    qb = q.reshape(-1, 32).astype(np.int64)
    assert np.abs(qb).max() <= 127
    xv = np_bf16(x).reshape(-1, 32)
    nz = np.abs(xv).max(1) > 0
    assert (np.abs(qb[nz]).max(1) == 127).all() and (qb[~nz] == 0).all() and (np_f16(d)[~nz] == 0).all()
    qn, dn = orc.q8_quantize_x(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(dn, d)
    x2 = bf16_bits(np_bf16(x).astype(np.float32) * 2)
    q2, d2 = orc.q8_quantize_x(x2)
    assert np.array_equal(q2, q) and np.array_equal(np_f16(d2), 2 * np_f16(d))
    dex = np.abs(xv).max(1) / 127.0
    d16 = np_f16(d)
    err = np.abs(d16[:, None] * qb - xv)
    bound = dex / 2 + 127 * np.abs(dex - d16)
    assert (err <= bound[:, None] * (1 + 1e-6) + 1e-300).all()


def test_q8x_gemv_reduces_to_exact_path(orc):
    """When the activation is exactly a Q8_0 vector (x = e q with max|q| = 127 and e a
    power of two) its quantization is lossless, so the integer-dot GEMV equals the exact
    Q8_0 GEMV (pinned to numpy above) on x; it scales exactly with x; a single nonzero
    code pair gives dw dx qw qx."""
    N, K = 48, 512
    rows = syn.make_q8_rows(N, K, seed=4)
    rng = np.random.default_rng(5)
    qx = rng.integers(-127, 128, size=K)
    qx[::32] = 127                                   # every block reaches 127
    x = bf16_bits(np.ldexp(qx.astype(np.float32), -6))
    q, d = orc.q8_quantize_x(x)
    assert np.array_equal(q.astype(np.int64), qx) and (np_f16(d) == 2.0 ** -6).all()
    y = orc.q8_gemv_q8x(rows, N, K, q, d)
    ref = orc.q8_gemv(rows, N, K, x)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    q2, d2 = orc.q8_quantize_x(bf16_bits(np_bf16(x).astype(np.float32) * 4))
    assert np.array_equal(orc.q8_gemv_q8x(rows, N, K, q2, d2), 4 * y)
    one = np.zeros((16, 1, 34), dtype=np.uint8)
    one[:, 0, 0:2] = np.array([np.float16(0.5)]).view(np.uint8)      # dw = 0.5
    one[3, 0, 2 + 7] = np.uint8(np.int8(-9).view(np.uint8))
    xq = np.zeros(32, dtype=np.int8)
    xq[7] = 11
    xd = np.array([np.float16(0.25)]).view(np.uint16)
    yy = orc.q8_gemv_q8x(one, 16, 32, xq, xd)
    assert yy[3] == 0.5 * 0.25 * -9 * 11 and (np.delete(yy, 3) == 0).all()


def test_q8x_gemv_error_bound(orc):
    """Random activations: the integer-dot GEMV differs from the exact path by at most
    sum_b |dw| sum_c |qw| (d_b/2 + 127 |d_b - fp16(d_b)|) per row."""
    N, K = 32, 1024
    rows = syn.make_q8_rows(N, K, seed=6)
    x = syn.make_x(1, K, seed=7)[0]
    q, d = orc.q8_quantize_x(x)
    y = orc.q8_gemv_q8x(rows, N, K, q, d)
    ref = orc.q8_gemv(rows, N, K, x)
    dw = np_f16(rows[:, :, 0:2].copy().view(np.uint16)[..., 0])
    qw = np.abs(rows[:, :, 2:].view(np.int8).astype(np.float64)).sum(2)
    xv = np_bf16(x).reshape(-1, 32)
    dex = np.abs(xv).max(1) / 127.0
    tol = (np.abs(dw) * qw * (dex / 2 + 127 * np.abs(dex - np_f16(d)))[None, :]).sum(1)
    assert (np.abs(y - ref) <= tol * (1 + 1e-9)).all()
    assert np.abs(y - ref).max() > 0                 # the quantization did change x


def test_q8_page_byte_counts():
    """Ember's packed selections for Llama-3.2-1B (16 layers, Q8_0 = 34 bytes per 32
    weights): gate/up + Q/K/V/O = 714.0 MiB, and down adds 272.0 MiB."""
    import bench
    layers = 16
    qkv, o, gu, dn = syn.Q8_SHAPES
    sel = layers * sum(bench.q8_weight_bytes(n, k) for n, k in (qkv, o, gu))
    down = layers * bench.q8_weight_bytes(*dn)
    assert sel / 2 ** 20 == pytest.approx(714.0, abs=0.05)
    assert down / 2 ** 20 == pytest.approx(272.0, abs=0.05)


def test_page_assignment_count():
    """2K-token prompt, top-8 of 256: 16,384 assignments, mean 64 rows/expert."""
    T, k, E = 2048, 8, 256
    assert T * k == 16384 and T * k / E == 64


# --------------------------------------------------------------- input generators
def test_skew_generator_hot_experts():
    """the Zipf(1.1) router bias gives a few experts > 10x the mean load."""
    L = syn.make_layer(**syn.SKEW)
    x = syn.make_x(4096, L.hidden, seed=0)
    l = np_logits(L, x)
    top = np.argsort(-l, axis=1, kind="stable")[:, :L.top_k]
    counts = np.bincount(top.reshape(-1), minlength=L.n_experts)
    mean = counts.sum() / L.n_experts
    assert (counts > 10 * mean).sum() >= 3
    assert (counts == 0).sum() > 0


def test_decode_generator_logit_scale():
    L = syn.make_layer(**syn.DECODE)
    x = syn.make_x(256, L.hidden, seed=0)
    l = np_logits(L, x)
    assert 0.8 < l.std() < 1.2
    assert L.expert_bytes == 1769472
