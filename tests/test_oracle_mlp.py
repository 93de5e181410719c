"""Pins of the oracle's expert MLP, combine and MXFP8 quantisation (no GPU):
dense brute force, closed forms, linearity, textbook rounding cases."""
import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from mxfp4_routed_expert_renorm_amd import workloads as W


def test_sparse_equals_dense_brute_force_tiny():
    cfg = W.WORKLOADS["tiny"]
    d = W.make_layer_inputs(cfg, W.WORKLOADS["tiny"]["seed"])
    E, H, I, k = cfg["E"], cfg["H"], cfg["I"], cfg["k"]
    x = d["x"].astype(np.float64)
    logits = O.router_logits(x, d["router_w"])
    ids, w = O.route(logits, k)
    sparse = O.layer_forward(x, ids, w, lambda e: d["bank"][e], H, I)
    weights_all = [O.expert_weights(d["bank"][e], H, I) for e in range(E)]
    gate = np.zeros((x.shape[0], E))
    for t in range(x.shape[0]):
        gate[t, ids[t]] = w[t]
    dense = O.dense_layer_forward(x, gate, weights_all)
    assert np.allclose(sparse, dense, rtol=0, atol=1e-12 * np.abs(dense).max())


def _const_record(H, I, code, expo):
    rec = np.zeros(O.fp4_expert_nbytes(H, I), np.uint8)
    p = O.split_record(rec, H, I, 4)
    for m in ("w1", "w3", "w2"):
        p[m + "_codes"][:] = code | (code << 4)
        p[m + "_scales"][:] = expo
    return rec


def test_all_ones_expert_closed_form():
    H, I = 64, 32
    rec = _const_record(H, I, 2, 127)            # code 2 = 1.0, scale 2^0
    x = np.random.default_rng(0).standard_normal(H)
    s = x.sum()
    want = I * (s / (1 + math.exp(-s))) * s      # every g and u equal sum(x)
    y = O.expert_mlp(x, *O.expert_weights(rec, H, I))
    assert np.allclose(y, want, rtol=1e-13)


def test_one_hot_input_selects_a_column():
    cfg = W.WORKLOADS["tiny"]
    H, I = cfg["H"], cfg["I"]
    rec = W.fp4_record(3, 1, 0, H, I)
    W1, W3, W2 = O.expert_weights(rec, H, I)
    j = 37
    x = np.zeros(H)
    x[j] = 1.0
    g, u = W1[:, j], W3[:, j]
    want = W2 @ (g / (1 + np.exp(-g)) * u)
    assert np.allclose(O.expert_mlp(x, W1, W3, W2), want, rtol=1e-14)


def test_scale_byte_plus_one_doubles():
    """E8M0 +1 on every w2 scale doubles the output (linearity in W2);
    +1 on every w3 scale doubles u and so the output too."""
    H, I = 256, 128
    rec = W.fp4_record(9, 1, 0, H, I)
    x = W.f32_normal(9, (2,), (H,)).astype(np.float64)
    y0 = O.expert_mlp(x, *O.expert_weights(rec, H, I))
    for m in ("w2", "w3"):
        r2 = rec.copy()
        O.split_record(r2, H, I, 4)[m + "_scales"][:] += 1
        y1 = O.expert_mlp(x, *O.expert_weights(r2, H, I))
        assert np.allclose(y1, 2 * y0, rtol=1e-13)


def test_combine_rank_order_and_shared():
    y = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    w = np.array([0.5, 0.25, 0.25])
    assert O.combine(y, w).tolist() == [28.0, 56.0]
    assert O.combine(y, w, np.array([1.0, -1.0])).tolist() == [29.0, 55.0]


def test_layer_forward_dropped_rank_contributes_nothing():
    cfg = W.WORKLOADS["tiny"]
    H, I = cfg["H"], cfg["I"]
    bank = W.fp4_bank(1, 1, 4, H, I)
    x = W.f32_normal(1, (3,), (1, H)).astype(np.float64)
    ids = np.array([[0, 1, 2]])
    w = np.array([[0.5, 0.3, 0.2]])
    prec = np.array([[0, -1, 0]])
    out = O.layer_forward(x, ids, w, lambda e, p: bank[e], H, I, prec=prec)
    want = 0.5 * O.expert_mlp(x[0], *O.expert_weights(bank[0], H, I)) \
        + 0.2 * O.expert_mlp(x[0], *O.expert_weights(bank[2], H, I))
    assert np.allclose(out[0], want, rtol=1e-14)


# ---------------------------------------------------------------- rounding

def test_round_to_bf16_textbook_cases():
    cases = [
        (1.0, 1.0),
        (1.0 + 2 ** -8, 1.0),                    # exact tie -> even (1.0)
        (1.0 + 3 * 2 ** -8, 1.0 + 2 ** -6),      # exact tie -> even mantissa
        (1.0 + 2 ** -8 + 2 ** -30, 1.0 + 2 ** -7),
        (-3.0, -3.0),
        (2.0 ** -130, 2.0 ** -130),              # subnormal, representable
        (3.0 * 2 ** -134, 2.0 ** -132),          # tie between 2^-133 and 2*2^-133 -> even
    ]
    for v, want in cases:
        assert O.round_to_bf16(np.array([v]))[0] == want, v
    # agrees with float32 -> bf16 truncation-with-carry on float32 inputs
    x = np.random.default_rng(2).standard_normal(2000).astype(np.float32)
    bits = W.bf16_bits_from_f32(x)
    assert np.array_equal(O.round_to_bf16(x.astype(np.float64)), O.bf16_bits_to_f64(bits))


# ---------------------------------------------------------------- MXFP8

def test_e4m3_encode_roundtrip_and_ties():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_value(codes)
    fin = ~np.isnan(vals)
    enc = O.e4m3_encode(vals[fin])
    assert np.array_equal(enc, codes[fin])               # every finite code round-trips
    # midpoint between 1.0 (0x38) and 1.125 (0x39) goes to the even code 0x38
    assert O.e4m3_encode(np.array([1.0625]))[0] == 0x38
    # midpoint between 1.125 (0x39) and 1.25 (0x3a) goes to 0x3a
    assert O.e4m3_encode(np.array([1.1875]))[0] == 0x3a
    # midpoint between the largest subnormal (0x07) and the smallest normal (0x08)
    assert O.e4m3_encode(np.array([(7 / 8 + 1) / 2 * 2 ** -6]))[0] == 0x08
    # saturation
    assert O.e4m3_encode(np.array([1e9, -500.0, 464.0]))[:].tolist() == [0x7e, 0xfe, 0x7e]
    assert O.e4m3_encode(np.array([-2 ** -12]))[0] == 0x80   # rounds to -0


def test_mxfp8_closed_forms():
    v = np.zeros((2, 64))
    v[0, :32] = 1.0                 # amax 1 -> shared exponent 0 - 8 = -8
    v[0, 32:] = 448.0               # amax 448 -> floor(log2 448) = 8 -> shared 0
    v[1, 0], v[1, 1], v[1, 2] = 7.75, 0.25, -3.0
    codes, scales = O.quant_mxfp8(v)
    assert scales[0].tolist() == [127 - 8, 127]
    assert np.all(codes[0, :32] == 0x78)           # 1.0 / 2^-8 = 256 = 0x78
    assert np.all(codes[0, 32:] == 0x7e)
    assert scales[1, 1] == 0 and np.all(codes[1, 32:] == 0)                # all-zero group
    # amax 7.75 -> floor(log2) = 2 -> shared -6; 7.75 * 64 = 496 saturates to 448
    assert scales[1, 0] == 127 - 6
    assert codes[1, :3].tolist() == [0x7e, 0x58, 0xf4]   # 448, 16, -192
    deq = O.dequant_mxfp8(codes, scales)
    assert np.all(deq[0] == v[0])
    assert deq[1, :3].tolist() == [7.0, 0.25, -3.0]
    assert np.all(deq[1, 3:] == 0)


def test_mxfp8_relative_error_bound():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((8, 256))
    c, s = O.quant_mxfp8(v)
    d = O.dequant_mxfp8(c, s)
    g = v.reshape(8, 8, 32)
    amax = np.abs(g).max(axis=2, keepdims=True)
    err = np.abs(d - v).reshape(8, 8, 32)
    # normal range: half an ulp (2^-4 relative); below 2^-6 * scale: absolute
    scale = 2.0 ** (np.floor(np.log2(amax)) - 8)
    bound = np.maximum(np.abs(g) * 2 ** -4, 2 ** -10 * scale)
    # values pushed past 448 by the floor in the shared exponent saturate
    sat = np.abs(g) / scale > 448
    assert np.all((err <= bound * (1 + 1e-12)) | sat)


def test_prefill_forward_error_bound_against_exact_layer():
    """With activations already on the MXFP8 grid, the prefill oracle differs
    from the exact layer only through the MXFP8 rounding of h, which is bounded
    elementwise by |W2| |dh| with |dh| <= 2^-4 |h| + 2^-10 * group scale."""
    cfg = W.WORKLOADS["tiny"]
    H, I, E, k = cfg["H"], cfg["I"], cfg["E"], 2
    bank = W.fp4_bank(21, 1, E, H, I)
    x = W.f32_normal(21, (2,), (3, H)).astype(np.float64)
    xc, xs = O.quant_mxfp8(x)
    xg = O.dequant_mxfp8(xc, xs)                    # on the grid
    c2, s2 = O.quant_mxfp8(xg)
    assert np.array_equal(O.dequant_mxfp8(c2, s2), xg)
    lg = W.router_logits(21, (3,), 3, E)
    ids, w = O.route(lg, k)
    pre = O.prefill_forward(xg, ids, w, lambda e: bank[e], H, I)
    exact = O.layer_forward(xg, ids, w, lambda e: bank[e], H, I)
    bound = np.zeros_like(exact)
    for t in range(3):
        for r in range(k):
            W1, W3, W2 = O.expert_weights(bank[ids[t, r]], H, I)
            g, u = W1 @ xg[t], W3 @ xg[t]
            h = O.silu(g) * u
            amax = np.abs(h.reshape(-1, 32)).max(axis=1)
            sc = np.repeat(2.0 ** (np.floor(np.log2(amax)) - 8), 32)
            dh = np.abs(h) * 2 ** -4 + 2 ** -10 * sc
            bound[t] += w[t, r] * (np.abs(W2) @ dh)
    err = np.abs(pre - exact)
    assert np.all(err <= bound * (1 + 1e-9))
    assert err.max() > 0                            # h rounding does act


def test_prefill_forward_quantises_activations():
    """The prefill layer sees x only through its MXFP8 image: evaluating it on
    bf16 activations off the MXFP8 grid gives exactly what it gives on their
    quantised values, and not what the same products give on x itself."""
    cfg = W.WORKLOADS["tiny"]
    H, I, E, k = cfg["H"], cfg["I"], cfg["E"], 2
    bank = W.fp4_bank(23, 1, E, H, I)
    x = O.bf16_bits_to_f64(W.bf16_normal(23, (2,), (3, H)))
    xc, xs = O.quant_mxfp8(x)
    xq = O.dequant_mxfp8(xc, xs)
    assert not np.array_equal(xq, x)                # bf16 values off the E4M3 grid
    ids, w = O.route(W.router_logits(23, (3,), 3, E), k)
    pre = O.prefill_forward(x, ids, w, lambda e: bank[e], H, I)
    assert np.array_equal(pre, O.prefill_forward(xq, ids, w, lambda e: bank[e], H, I))
    # the same products and h rounding on the unquantised x
    raw = np.zeros_like(pre)
    for t in range(3):
        for r in range(k):
            W1, W3, W2 = O.expert_weights(bank[ids[t, r]], H, I)
            h = O.silu(W1 @ x[t]) * (W3 @ x[t])
            hc, hs = O.quant_mxfp8(h[None, :])
            raw[t] += w[t, r] * (W2 @ O.dequant_mxfp8(hc, hs)[0])
    assert np.linalg.norm(pre - raw) > 1e-3 * np.linalg.norm(raw)
