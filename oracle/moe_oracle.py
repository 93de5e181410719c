"""CPU oracle of the routed MXFP4 mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library (no kernels,
headers, tables or helpers); both sides consume the same seeded input bytes.

Everything is plain NumPy in float64, written to be checked by eye against
the pages it follows:

  [P1] "Running DeepSeek-V4-Flash across four free GPUs"
  [P2] "An elephant through a straw"
  [P3] "DeepSeek V4.1 Flash on 5x 8 GB (PP5 full residency)"

The layer (P1 §What the expert cache actually does; P2 §Not all six experts
matter equally, §43 graphs, 43 syncs):
  1. route: pick each token's top-k experts from the router's scores and
     renormalise their weights;
  2. remap expert ids onto slots of a fixed-size global LRU slot cache,
     classifying each rank against the precision ladder (a, b);
  3. run the SwiGLU expert MLP on MXFP4 weights (or on the 2-bit copy);
  4. combine the expert outputs with the renormalised weights.

Readings where the pages are silent are stated at each function; the list of
them is kept with the design notes.  Functions whose result could not be tied
to anything outside this file would say "parity unpinned" here; every function
below is pinned by a test (closed form, brute force, independent textbook
model or a value printed on the pages).
"""
from __future__ import annotations

import math

import numpy as np

# ============================================================================
# 1. element and scale formats
# ============================================================================

# FP4 E2M1 value of each 4-bit code (sign, 2 exponent bits, 1 mantissa bit,
# exponent bias 1, no infinities or NaN).  The format is the MXFP4 element
# type of the OCP Microscaling spec that P2 cites (References) and that P1
# names for the routed experts (§The model: FP4 packed into I8 with F8_E8M0
# scales alongside).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)


def e8m0_value(e):
    """E8M0 scale byte -> 2^(e-127); 255 is NaN (OCP MX).  P1 §The model."""
    e = np.asarray(e, dtype=np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def _e4m3_table() -> np.ndarray:
    """FP8 E4M3 (OCP 'E4M3FN'): bias 7, exponent field 0 is subnormal
    (m/8 * 2^-6), S.1111.111 is NaN, no infinities, largest finite 448.
    P2 names it as the scale type of the 2-bit copies (opening section;
    §Rig, model & methodology: per-32 fp8-e4m3 scales)."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        ef = (code >> 3) & 0xF
        m = code & 0x7
        if ef == 0xF and m == 0x7:
            t[code] = np.nan
        elif ef == 0:
            t[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            t[code] = s * (1.0 + m / 8.0) * 2.0 ** (ef - 7)
    return t


E4M3_VALUES = _e4m3_table()
E4M3_MAX = 448.0


def e4m3_value(b):
    return E4M3_VALUES[np.asarray(b, dtype=np.int64)]


def int2_level(c):
    """2-bit code -> signed level (c - 1.5): {-1.5, -0.5, +0.5, +1.5}.
    P2 gives only '2-bit codes with one fp8 scale per group of 32 weights'
    (opening section); the symmetric mid-rise codebook is the plain reading."""
    return np.asarray(c, dtype=np.float64) - 1.5


# ============================================================================
# 2. expert record layout and sizes
# ============================================================================
# One expert = three matrices w1 (gate), w3 (up), w2 (down) (P1 §What you
# actually get: 768 expert tensors per shard = 256 experts x w1, w2, w3),
# stored [out][in] with one scale per 32 consecutive weights along the input
# dimension (P1 §Step 2 / Check it divides: FP4 32-element scale blocks).
# Record order: w1 codes, w3 codes, w2 codes, w1 scales, w3 scales, w2 scales.

def fp4_expert_nbytes(H: int, I: int) -> int:
    """Bytes of one MXFP4 expert: 3*H*I weights at 4 bits plus one byte per 32
    weights.  P2 (opening section) prints 13,369,344 bytes for its model."""
    n = 3 * H * I
    return n // 2 + n // 32


def int2_expert_nbytes(H: int, I: int) -> int:
    """Bytes of one 2-bit expert: 2 bits per weight plus one fp8 scale per 32
    (2.25 bits/weight; P2 §Rig, model & methodology: 6.75 MB/expert)."""
    n = 3 * H * I
    return n // 4 + n // 32


def split_record(rec: np.ndarray, H: int, I: int, bits: int) -> dict:
    """Slice a record into (codes, scales) per matrix, each [rows, bytes]."""
    assert bits in (4, 2)
    per = 8 // bits
    shapes = {"w1": (I, H), "w3": (I, H), "w2": (H, I)}
    out, off = {}, 0
    for name in ("w1", "w3", "w2"):
        r, c = shapes[name]
        n = r * c // per
        out[name + "_codes"] = rec[off:off + n].reshape(r, c // per)
        off += n
    for name in ("w1", "w3", "w2"):
        r, c = shapes[name]
        n = r * c // 32
        out[name + "_scales"] = rec[off:off + n].reshape(r, c // 32)
        off += n
    assert off == rec.size, (off, rec.size)
    return out


def unpack_fp4_codes(codes: np.ndarray) -> np.ndarray:
    """[rows, cols/2] bytes -> [rows, cols] 4-bit codes; element 2j is the low
    nibble of byte j (reading: pages silent, the common I8 packing)."""
    c = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    c[:, 0::2] = codes & 0x0F
    c[:, 1::2] = codes >> 4
    return c


def unpack_int2_codes(codes: np.ndarray) -> np.ndarray:
    """[rows, cols/4] bytes -> [rows, cols] 2-bit codes; element 4j+q is bits
    2q..2q+1 of byte j (reading)."""
    c = np.empty((codes.shape[0], codes.shape[1] * 4), dtype=np.uint8)
    for q in range(4):
        c[:, q::4] = (codes >> (2 * q)) & 0x3
    return c


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[o, i] = E2M1(code[o, i]) * 2^(scale[o, i // 32] - 127), float64."""
    c = unpack_fp4_codes(codes)
    s = e8m0_value(scales)
    return E2M1_VALUES[c] * np.repeat(s, 32, axis=1)


def dequant_int2(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[o, i] = (code[o, i] - 1.5) * e4m3(scale[o, i // 32]), float64."""
    c = unpack_int2_codes(codes)
    s = e4m3_value(scales)
    return int2_level(c) * np.repeat(s, 32, axis=1)


def expert_weights(rec: np.ndarray, H: int, I: int, prec: int = 0):
    """(W1 [I,H], W3 [I,H], W2 [H,I]) float64 of one record; prec 0 = FP4,
    1 = the 2-bit copy."""
    if prec == 0:
        p = split_record(rec, H, I, 4)
        dq = dequant_mxfp4
    else:
        p = split_record(rec, H, I, 2)
        dq = dequant_int2
    return (dq(p["w1_codes"], p["w1_scales"]),
            dq(p["w3_codes"], p["w3_scales"]),
            dq(p["w2_codes"], p["w2_scales"]))


# ============================================================================
# 3. routing
# ============================================================================

def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """l[t, e] = x[t] . W_r[e], float64 (tiny configuration computes its
    router scores from the activations)."""
    return np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T


def route(logits: np.ndarray, k: int):
    """Top-k selection with renormalised weights.

    Each token keeps the k experts with the largest router scores and
    renormalises their weights so they sum to one (P1 §What the expert cache
    actually does: the router picks its top_k experts; P2 §Not all six experts
    matter equally: the router emits six weights per token).  Reading: the
    score is a softmax over all E logits; ties in the logit go to the lower
    expert id; experts are emitted in rank order (weight descending).  A NaN
    logit counts as -inf: it ranks with the -inf logits (ties to the lower
    id), never above a real one, and its weight is 0 (when every selected
    logit is -inf the weights are undefined: NaN).

    Returns ids int32 [T, k] and weights float64 [T, k]."""
    lg = np.asarray(logits, dtype=np.float64)
    lg = np.where(np.isnan(lg), -np.inf, lg)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    eid = np.arange(E)
    for t in range(T):
        order = np.lexsort((eid, -lg[t]))        # primary: logit desc; secondary: id asc
        sel = order[:k]
        p = np.exp(lg[t] - lg[t].max())
        p = p / p.sum()                          # softmax over all experts
        ids[t] = sel
        w[t] = p[sel] / p[sel].sum()             # renormalise over the selected
    return ids, w


# ============================================================================
# 4. grouping tokens by expert
# ============================================================================

def group_pairs(ids: np.ndarray, E: int):
    """Stable counting sort of the T*k (token, rank) pairs by expert id.

    P2 §43 graphs, 43 syncs fires grouped expert kernels; grouping each
    expert's tokens lets its weights stream once.  Returns counts [E],
    offsets [E+1] and perm [T*k] (pair index t*k + r, expert-major, ascending
    pair index within an expert)."""
    flat = np.asarray(ids, np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    return counts, offsets, perm


# ============================================================================
# 5. the expert MLP and the combine
# ============================================================================

def silu(g):
    return g / (1.0 + np.exp(-g))


def expert_mlp(x: np.ndarray, W1: np.ndarray, W3: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """SwiGLU expert: y = W2 (silu(W1 x) * (W3 x)), float64.  x is [H] or
    [n, H].  Reading: plain SwiGLU, no clamp and no routed scaling factor."""
    x = np.asarray(x, np.float64)
    g = x @ W1.T
    u = x @ W3.T
    h = silu(g) * u
    return h @ W2.T


def combine(y: np.ndarray, w: np.ndarray, y_shared=None) -> np.ndarray:
    """out = sum over ranks in rank order of w[r] * y[r] (+ the shared expert
    with weight one).  P1 §What the expert cache actually does (_expert_gemm
    takes topk_weights); P2 §Not all six experts matter equally (survivors
    renormalised).  y is [k, H], w is [k] (zero for dropped ranks)."""
    out = np.zeros(y.shape[-1], dtype=np.float64)
    for r in range(y.shape[0]):
        out = out + w[r] * y[r]
    if y_shared is not None:
        out = out + y_shared
    return out


def layer_forward(x, ids, w, get_record, H: int, I: int, shared_rec=None, prec=None):
    """Full layer for T tokens: out[t] = sum_r w[t,r] * expert_{ids[t,r]}(x[t])
    (+ shared expert).  get_record(e) returns the FP4 record of expert e.
    prec (optional [T,k]: 0 FP4, 1 INT2, -1 dropped) with get_record(e, p)
    selecting the precision.  Returns float64 [T, H]."""
    x = np.asarray(x, np.float64)
    T, k = ids.shape
    out = np.zeros((T, H), dtype=np.float64)
    cache = {}

    def weights(e, p):
        key = (int(e), int(p))
        if key not in cache:
            rec = get_record(e) if prec is None else get_record(e, p)
            cache[key] = expert_weights(rec, H, I, p)
        return cache[key]

    shared_w = expert_weights(shared_rec, H, I, 0) if shared_rec is not None else None
    for t in range(T):
        ys = np.zeros((k, H))
        wt = np.array(w[t], dtype=np.float64)
        for r in range(k):
            p = 0 if prec is None else int(prec[t, r])
            if p < 0:
                wt[r] = 0.0
                continue
            ys[r] = expert_mlp(x[t], *weights(ids[t, r], p))
        ysh = expert_mlp(x[t], *shared_w) if shared_w is not None else None
        out[t] = combine(ys, wt, ysh)
    return out


def dense_layer_forward(x, gate: np.ndarray, weights_all, shared_w=None) -> np.ndarray:
    """Brute force: every expert evaluated for every token and mixed by a dense
    gate matrix G[t, e] (the renormalised weight on selected experts, zero
    elsewhere).  Used only to pin the sparse path."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    E = len(weights_all)
    Y = np.stack([expert_mlp(x, *weights_all[e]) for e in range(E)], axis=1)   # [T, E, H]
    out = np.einsum("te,teh->th", gate, Y)
    if shared_w is not None:
        out = out + expert_mlp(x, *shared_w)
    return out


# ============================================================================
# 6. output rounding
# ============================================================================

def round_to_bf16(v) -> np.ndarray:
    """float64 -> nearest bfloat16 (ties to even), returned as float64.
    bf16 = 8 significant bits, exponent range of float32."""
    v = np.asarray(v, np.float64)
    out = np.empty_like(v)
    flat, of = v.reshape(-1), out.reshape(-1)
    for i, a in enumerate(flat):
        if not math.isfinite(a) or a == 0.0:
            of[i] = a
            continue
        e = math.frexp(abs(a))[1] - 1             # |a| in [2^e, 2^(e+1))
        e = max(e, -126)                          # subnormal spacing below 2^-126
        q = 2.0 ** (e - 7)
        r = round(a / q) * q                      # Python round: ties to even, exact
        of[i] = r if abs(r) <= 3.3895313892515355e38 else math.copysign(math.inf, a)
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ============================================================================
# 7. MXFP8 activation quantisation (prefill-sized grouped GEMM)
# ============================================================================
# The prefill workload feeds the FP4 weights and FP8 activations to a scaled
# matrix instruction; activations get one E8M0 scale per 32 consecutive
# elements along the reduction dimension.  Rule (OCP MX): shared exponent =
# floor(log2(amax)) - 8 (8 = exponent of E4M3's largest power of two),
# clamped to the E8M0 range; elements = v / 2^shared rounded to nearest E4M3
# (ties to even) with saturation at +-448; an all-zero group gets scale
# code 0 and zero elements.

_E4M3_POS = E4M3_VALUES[:127]          # codes 0x00..0x7E, ascending, finite


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code, ties to the even code, saturating at +-448."""
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")       # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _E4M3_POS[hi], hi, code).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def quant_mxfp8(v: np.ndarray):
    """[n, K] values -> (E4M3 codes uint8 [n, K], E8M0 scale bytes uint8 [n, K/32])."""
    v = np.asarray(v, np.float64)
    n, K = v.shape
    g = v.reshape(n, K // 32, 32)
    amax = np.abs(g).max(axis=2)
    scales = np.zeros((n, K // 32), dtype=np.uint8)
    codes = np.zeros((n, K // 32, 32), dtype=np.uint8)
    for i in range(n):
        for j in range(K // 32):
            if amax[i, j] == 0.0:
                scales[i, j] = 0
                codes[i, j] = e4m3_encode(g[i, j])            # signed zeros
                continue
            e = math.frexp(amax[i, j])[1] - 1                  # floor(log2(amax))
            sh = min(max(e - 8, -127), 127)
            scales[i, j] = sh + 127
            codes[i, j] = e4m3_encode(g[i, j] / 2.0 ** sh)
    return codes.reshape(n, K), scales


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return e4m3_value(codes) * np.repeat(e8m0_value(scales), 32, axis=1)


def prefill_forward(x, ids, w, get_record, H: int, I: int, shared_rec=None, tokens=None) -> np.ndarray:
    """Prefill layer with MXFP8 activations: x is quantised per 32 along H, the
    SwiGLU output h per 32 along I, each feeding the FP4-weight products.
    tokens (optional) restricts the evaluation to a subset of token indices.
    Each expert is dequantised once and applied to every (token, rank) pair
    that selected it (so memory holds one expert at a time); the outputs are
    then combined per token in rank order.  Returns float64 [len(tokens), H]."""
    x = np.asarray(x, np.float64)
    T, k = ids.shape
    tokens = list(range(T)) if tokens is None else list(tokens)

    def one(xq, W1, W3, W2):
        g = W1 @ xq
        u = W3 @ xq
        h = silu(g) * u
        hc, hs = quant_mxfp8(h[None, :])
        return W2 @ dequant_mxfp8(hc, hs)[0]

    xq = {}
    for t in tokens:
        xc, xs = quant_mxfp8(x[t][None, :])
        xq[t] = dequant_mxfp8(xc, xs)[0]
    ys = np.zeros((len(tokens), k, H))
    pairs = {}
    for j, t in enumerate(tokens):
        for r in range(k):
            pairs.setdefault(int(ids[t, r]), []).append((j, r))
    for e in sorted(pairs):
        We = expert_weights(get_record(e), H, I, 0)
        for j, r in pairs[e]:
            ys[j, r] = one(xq[tokens[j]], *We)
        del We
    ysh = None
    if shared_rec is not None:
        Ws = expert_weights(shared_rec, H, I, 0)
        ysh = np.stack([one(xq[t], *Ws) for t in tokens])
    return np.stack([combine(ys[j], np.asarray(w[t], np.float64), None if ysh is None else ysh[j])
                     for j, t in enumerate(tokens)])


# ============================================================================
# 7b. the 2-bit fallback copy of an MXFP4 expert (offline clip search)
# ============================================================================
# P2 (opening section; §Rig, model & methodology) re-quantises every expert
# to 2-bit codes with one fp8 E4M3 scale per 32 weights, the scale "chosen by
# clip search", and states no more.  Reading: per 32-weight group of the
# dequantised FP4 weights, each clip ratio alpha of CLIP_ALPHAS proposes the
# scale s = E4M3(alpha * amax / 1.5) (nearest, ties to even: the levels
# +-1.5 s then reach alpha * amax), each weight takes the nearest level
# (code = clamp(round_half_even(w / s + 1.5), 0, 3)), and the ratio with the
# least squared error sum(w - w_hat)^2, summed in element order, wins; ties
# go to the larger alpha.  A scale that rounds to 0 gives every weight the
# level 0 (code 2).  All arithmetic is float64, one IEEE operation at a time.

CLIP_ALPHAS = (1.00, 0.95, 0.90, 0.85, 0.80, 0.75, 0.70, 0.65, 0.60, 0.55, 0.50)


def quant_int2_clip(W: np.ndarray):
    """[rows, cols] float64 weights -> (2-bit codes uint8 [rows, cols] (0..3),
    E4M3 scale bytes uint8 [rows, cols/32]) by the clip search above."""
    W = np.asarray(W, np.float64)
    rows, cols = W.shape
    g = W.reshape(rows * (cols // 32), 32)
    amax = np.abs(g).max(axis=1)
    best_err = np.full(g.shape[0], np.inf)
    best_codes = np.full(g.shape, 2, dtype=np.uint8)
    best_scale = np.zeros(g.shape[0], dtype=np.uint8)
    for alpha in CLIP_ALPHAS:
        t = (alpha * amax) / 1.5
        sc = e4m3_encode(t)
        s = e4m3_value(sc)
        ok = s > 0.0
        safe = np.where(ok, s, 1.0)
        c = np.clip(np.rint(g / safe[:, None] + 1.5), 0.0, 3.0)
        c = np.where(ok[:, None], c, 2.0)
        w_hat = (c - 1.5) * s[:, None]
        err = np.zeros(g.shape[0])
        for j in range(32):                 # element order
            d = g[:, j] - w_hat[:, j]
            err = err + d * d
        better = err < best_err              # strict: ties keep the larger alpha
        best_err = np.where(better, err, best_err)
        best_codes = np.where(better[:, None], c.astype(np.uint8), best_codes)
        best_scale = np.where(better, sc, best_scale)
    return best_codes.reshape(rows, cols), best_scale.reshape(rows, cols // 32)


def pack_int2_codes(c: np.ndarray) -> np.ndarray:
    """[rows, cols] 2-bit codes -> [rows, cols/4] bytes, element 4j+q in bits
    2q..2q+1 of byte j (the packing unpack_int2_codes reads)."""
    c = np.asarray(c, np.uint8)
    out = np.zeros((c.shape[0], c.shape[1] // 4), dtype=np.uint8)
    for q in range(4):
        out |= (c[:, q::4] & 0x3) << (2 * q)
    return out


def int2_record_from_fp4(rec: np.ndarray, H: int, I: int, rows=None) -> np.ndarray:
    """The 2-bit record (layout of int2_expert_nbytes) of one MXFP4 record.
    rows (optional): {matrix name: row indices} to compute only those rows;
    the other rows' bytes are left 0."""
    p = split_record(rec, H, I, 4)
    shapes = {"w1": (I, H), "w3": (I, H), "w2": (H, I)}
    codes, scales = {}, {}
    for name in ("w1", "w3", "w2"):
        r, c = shapes[name]
        idx = np.arange(r) if rows is None else np.asarray(rows[name])
        W = dequant_mxfp4(p[name + "_codes"][idx], p[name + "_scales"][idx])
        cq, sq = quant_int2_clip(W)
        codes[name] = np.zeros((r, c // 4), np.uint8)
        scales[name] = np.zeros((r, c // 32), np.uint8)
        codes[name][idx] = pack_int2_codes(cq)
        scales[name][idx] = sq
    return np.concatenate([codes["w1"].ravel(), codes["w3"].ravel(), codes["w2"].ravel(),
                           scales["w1"].ravel(), scales["w3"].ravel(), scales["w2"].ravel()])


# ============================================================================
# 8. the slot cache with the precision ladder
# ============================================================================

FP4, INT2, DROPPED = 0, 1, -1


class SlotCache:
    """Global slot cache over (layer, expert) pairs with the (a, b) ladder.

    P1 §What the expert cache actually does: a fixed number of expert slots
    in device memory ('not layers, not experts, slots'), shared by all layers
    (the cache is global, not per-layer), LRU eviction, expert ids rewritten
    to slots in place, only misses copied from the host banks.
    P2 §Not all six experts matter equally: ranks 1..a always FP4 (fetched on
    a miss); ranks a+1..b FP4 if resident, else the 2-bit copy; ranks > b used
    if resident, dropped otherwise; survivors renormalised.
    P2 §Rig, model & methodology (best configuration): a second, smaller tier
    of device slots for the 2-bit copies, and LFU eviction with frequency
    decay seeded from a routing trace.

    Readings where the pages are silent:
      * residency for a token's classification is read once, before any of
        that token's fetches; only FP4 residency classifies;
      * slots used by any rank of the call are protected from eviction for
        the rest of the call (in each tier);
      * fetches are processed in rank order; each hit or fetch stamps the
        slot with the next value of a global clock shared by both tiers;
      * victim of a fetch: the lowest-index empty slot; else, under LRU, the
        unprotected slot with the oldest stamp; under LFU, the unprotected
        slot whose pair has the lowest use count (ties: oldest stamp);
      * LFU counts belong to pairs (kept while evicted): at the start of every
        call each count is multiplied by the decay, and every use of a pair
        (hit or fetch, either tier) adds one; `seed` gives the initial counts
        (a routing trace's frequencies), zeros otherwise;
      * int2_slots == 0: 2-bit copies are not cached; every use is a fresh
        copy into a staging area, index t*(b-a) + (rank-a-1) within the call;
        int2_slots > 0: the 2-bit copy of a pair is looked up in the tier and
        fetched on a miss;
      * if every rank of a token is dropped, all its weights are zero;
      * prefetch (P2 §Guessing the router two layers ahead: predicted
        experts land in a small round-robin staging ring appended to the slot
        buffers, never evicting a resident expert; a wrong guess is
        overwritten by a later one): each
        predicted expert of the layer that is neither FP4-resident nor in the
        ring is copied, in list order, to the ring entry at the cursor, which
        then advances; entries the last call used are skipped, and so are
        entries this prefetch has filled; ring entries are slots S .. S+R-1;
      * a pair in the ring counts as FP4-resident when a token is classified
        and is used in place (slot S + entry): no copy, no stamp, one use for
        LFU; it is not moved into the cache.
    """

    def __init__(self, L: int, E: int, S: int, k: int, a: int, b: int, int2_slots: int = 0,
                 policy: str = "lru", decay: float = 1.0, seed=None, ring: int = 0):
        assert 0 <= a <= b <= k and S >= 1 and int2_slots >= 0 and policy in ("lru", "lfu")
        self.L, self.E, self.S, self.k, self.a, self.b = L, E, S, k, a, b
        self.S2, self.policy, self.decay = int2_slots, policy, float(decay)
        self.map = np.full(L * E, -1, dtype=np.int64)      # pair -> FP4 slot
        self.owner = np.full(S, -1, dtype=np.int64)        # FP4 slot -> pair
        self.stamp = np.zeros(S, dtype=np.int64)           # 0 = empty
        self.map2 = np.full(L * E, -1, dtype=np.int64)     # pair -> 2-bit slot
        self.owner2 = np.full(max(int2_slots, 1), -1, dtype=np.int64)
        self.stamp2 = np.zeros(max(int2_slots, 1), dtype=np.int64)
        self.count = (np.zeros(L * E) if seed is None else np.asarray(seed, np.float64).reshape(L * E).copy())
        self.R = ring
        self.ring_owner = np.full(max(ring, 1), -1, dtype=np.int64)   # entry -> pair
        self.map_ring = np.full(L * E, -1, dtype=np.int64)            # pair -> entry
        self.cursor = 0
        self.ring_used = set()   # ring entries the last call used (compute may still read them)
        self.clock = 0
        self.hits = self.misses = self.int2 = self.drops = self.int2_hits = 0
        self.prefetches = self.ring_hits = 0
        self.next_buf = 0        # the layer buffer the next stream_layer fills
        self.streamed = 0        # records copied by stream_layer

    def resident(self, layer: int, e: int) -> bool:
        return self.map[layer * self.E + e] >= 0

    def _victim(self, owner, stamp, protected):
        """Lowest-index empty slot, else the unprotected slot to evict."""
        n = len(owner)
        for s in range(n):
            if owner[s] < 0 and s not in protected:
                return s
        cand = [s for s in range(n) if s not in protected]
        assert cand, "every slot is in use by this call"
        if self.policy == "lru":
            return min(cand, key=lambda q: (stamp[q], q))
        return min(cand, key=lambda q: (self.count[owner[q]], stamp[q], q))

    def _use(self, pair: int):
        self.clock += 1
        self.count[pair] += 1.0
        return self.clock

    def step(self, layer: int, ids: np.ndarray, w: np.ndarray):
        """One call for T tokens of one layer.  ids [T,k] expert ids and w
        [T,k] weights in rank order.  Returns (slot int32 [T,k], prec int8
        [T,k], w' float64 [T,k], copies list of (kind, layer, expert, dest))."""
        ids = np.asarray(ids).reshape(-1, self.k)
        w = np.asarray(w, np.float64).reshape(-1, self.k)
        T, k, a, b, E = ids.shape[0], self.k, self.a, self.b, self.E
        assert T * k <= self.S
        assert self.S2 == 0 or T * (b - a) <= self.S2
        if self.policy == "lfu":
            self.count *= self.decay
        slot = np.full((T, k), -1, dtype=np.int32)
        prec = np.full((T, k), DROPPED, dtype=np.int8)
        wout = np.zeros((T, k), dtype=np.float64)
        copies = []
        protected, protected2, ring_used = set(), set(), set()
        for t in range(T):
            res = [self.resident(layer, int(e)) or self.map_ring[layer * E + int(e)] >= 0
                   for e in ids[t]]                                      # snapshot
            cls = []
            for r in range(k):
                rank = r + 1
                if rank <= a:
                    cls.append(FP4)
                elif rank <= b:
                    cls.append(FP4 if res[r] else INT2)
                else:
                    cls.append(FP4 if res[r] else DROPPED)
            for r in range(k):
                if cls[r] == FP4 and res[r] and self.map[layer * E + int(ids[t, r])] >= 0:
                    protected.add(int(self.map[layer * E + int(ids[t, r])]))
            for r in range(k):
                e = int(ids[t, r])
                pair = layer * E + e
                if cls[r] == FP4 and res[r] and self.map[pair] < 0:     # in the staging ring
                    q = int(self.map_ring[pair])
                    self.count[pair] += 1.0
                    ring_used.add(q)
                    slot[t, r], prec[t, r] = self.S + q, FP4
                    self.ring_hits += 1
                elif cls[r] == FP4 and res[r]:
                    s = int(self.map[pair])
                    self.stamp[s] = self._use(pair)
                    slot[t, r], prec[t, r] = s, FP4
                    self.hits += 1
                elif cls[r] == FP4:
                    s = self._victim(self.owner, self.stamp, protected)
                    if self.owner[s] >= 0:
                        self.map[self.owner[s]] = -1
                    self.owner[s] = pair
                    self.map[pair] = s
                    self.stamp[s] = self._use(pair)
                    protected.add(s)
                    slot[t, r], prec[t, r] = s, FP4
                    copies.append(("fp4", layer, e, s))
                    self.misses += 1
                elif cls[r] == INT2 and self.S2 == 0:
                    st = t * (b - a) + (r + 1 - a - 1)
                    self._use(pair)
                    slot[t, r], prec[t, r] = st, INT2
                    copies.append(("int2", layer, e, st))
                    self.int2 += 1
                elif cls[r] == INT2:
                    s = int(self.map2[pair])
                    if s >= 0:
                        self.int2_hits += 1
                    else:
                        s = self._victim(self.owner2, self.stamp2, protected2)
                        if self.owner2[s] >= 0:
                            self.map2[self.owner2[s]] = -1
                        self.owner2[s] = pair
                        self.map2[pair] = s
                        copies.append(("int2", layer, e, s))
                    self.stamp2[s] = self._use(pair)
                    protected2.add(s)
                    slot[t, r], prec[t, r] = s, INT2
                    self.int2 += 1
                else:
                    self.drops += 1
            keep = prec[t] != DROPPED
            tot = w[t][keep].sum()
            if tot > 0:
                wout[t][keep] = w[t][keep] / tot
        self.ring_used = ring_used
        return slot, prec, wout, copies

    def prefetch(self, layer: int, experts):
        """Copy the predicted experts of `layer` that are neither resident nor
        in the ring into the ring.  Returns the copies, as step() does."""
        copies = []
        filled = set()
        for e in experts:
            e = int(e)
            pair = layer * self.E + e
            if self.map[pair] >= 0 or self.map_ring[pair] >= 0:
                continue
            q = None
            for i in range(self.R):
                cand = (self.cursor + i) % self.R
                if cand not in self.ring_used and cand not in filled:
                    q = cand
                    break
            if q is None:
                break
            old = int(self.ring_owner[q])
            if old >= 0:
                self.map_ring[old] = -1
            self.ring_owner[q] = pair
            self.map_ring[pair] = q
            self.cursor = (q + 1) % self.R
            filled.add(q)
            copies.append(("fp4", layer, e, self.S + q))
            self.prefetches += 1
        return copies

    def stream_layer(self, layer: int):
        """Whole-layer streaming for prefill.  P1 §What the expert cache
        actually does: above the crossover (prefill_streams) prefill streams
        whole expert layers instead of fetching slots on demand; P1 §Step 7:
        with prefill overlap the cache lends two full expert-layer buffers,
        so it needs at least 2E slots.

        Readings where the pages are silent: the two buffers are slots [0, E)
        and [E, 2E), filled alternately starting with the first; expert e of
        the layer lands in slot bE + e, whose previous pair is evicted; a pair
        of the layer held elsewhere (another slot or the staging ring) gives
        that place up; a pair already in its buffer slot is not copied again;
        every streamed slot takes the next clock stamp, in expert order, and
        no LFU use; the streamed experts stay resident afterwards.
        Returns (buffer, copies) with copies as step() gives them."""
        E = self.E
        assert self.S >= 2 * E, "layer streaming needs two expert-layer buffers"
        b = self.next_buf
        self.next_buf ^= 1
        copies = []
        for e in range(E):
            s, pair = b * E + e, layer * E + e
            if self.owner[s] != pair:
                if self.owner[s] >= 0:
                    self.map[self.owner[s]] = -1
                old = int(self.map[pair])
                if old >= 0:
                    self.owner[old] = -1
                    self.stamp[old] = 0
                q = int(self.map_ring[pair])
                if q >= 0:
                    self.ring_owner[q] = -1
                    self.map_ring[pair] = -1
                self.owner[s] = pair
                self.map[pair] = s
                copies.append(("fp4", layer, e, s))
                self.streamed += 1
            self.clock += 1
            self.stamp[s] = self.clock
        return b, copies

    def slot_map(self) -> np.ndarray:
        return self.map.astype(np.int32).copy()


def prefill_streams(T: int, k: int, E: int) -> bool:
    """P1 §What the expert cache actually does and §Step 7: a prefill chunk
    of T tokens streams whole expert layers once T * top_k >= num_experts
    (it would touch most of the layer anyway); below that it fetches slots on
    demand."""
    return T * k >= E
