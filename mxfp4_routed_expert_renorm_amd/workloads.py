"""Seeded synthetic inputs for the routed MXFP4 mixture-of-experts layer.

This module is the only code shared by the CPU oracle's tests and the HIP
path's tests and benchmark.  It draws random numbers and places bytes; it
holds none of the layer's arithmetic (no decoding, no routing, no matrix
products).  Every array is a pure function of (seed, stream keys), drawn
with NumPy's PCG64 through a SeedSequence, so any single expert or token can
be regenerated on its own.

Byte layout of one expert record (the format every consumer slices):

    FP4 record  = w1 codes [I][H/2] | w3 codes [I][H/2] | w2 codes [H][I/2]
                | w1 scales [I][H/32] | w3 scales [I][H/32] | w2 scales [H][I/32]
    INT2 record = same order, codes [rows][cols/4], scales [rows][cols/32]

w1 is the gate, w3 the up and w2 the down projection, each stored
[out][in] row-major.  FP4 codes hold two elements per byte (element 2j in
the low nibble); INT2 codes hold four (element 4j+q in bits 2q..2q+1).
FP4 scales are E8M0 bytes, INT2 scales are FP8 E4M3 bytes.

Workload shapes follow the model the pages describe: 256 routed experts with
hidden 4096 and expert intermediate 2048 (Running DeepSeek-V4-Flash across
four free GPUs, §The model; An elephant through a straw, opening section,
13,369,344 bytes per FP4 expert).
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# stream keys (second element of every SeedSequence)
S_BANK, S_SHARED, S_X, S_LOGITS, S_ROUTER_W, S_ZIPF, S_INT2, S_STEP, S_PRED = range(1, 10)

# E8M0 exponent range of the synthetic FP4 scales (2^-8 .. 2^-4)
FP4_EXP_LO, FP4_EXP_HI = 119, 123
# FP8 E4M3 scale bytes of the synthetic INT2 copies: sign 0, exponent field
# uniform in 1..5, mantissa uniform in 0..7
INT2_EXPF_LO, INT2_EXPF_HI = 1, 5


def rng_for(seed: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, keys)])))


def _random_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    """n uniform bytes from the generator's raw 64-bit stream."""
    words = rng.bit_generator.random_raw((n + 7) // 8)
    return words.view(np.uint8)[:n]


def fp4_record_nbytes(H: int, I: int) -> int:
    return 3 * (I * H // 2) + 3 * (I * H // 32)


def int2_record_nbytes(H: int, I: int) -> int:
    return 3 * (I * H // 4) + 3 * (I * H // 32)


def fp4_record(seed: int, stream: int, index: int, H: int, I: int, out: np.ndarray | None = None,
               exp_lo: int = FP4_EXP_LO, exp_hi: int = FP4_EXP_HI) -> np.ndarray:
    """One FP4 expert record: codes uniform over 0..15 per nibble, E8M0 scale
    bytes uniform over exp_lo..exp_hi."""
    n = fp4_record_nbytes(H, I)
    if out is None:
        out = np.empty(n, np.uint8)
    assert out.shape == (n,) and out.dtype == np.uint8
    rng = rng_for(seed, stream, index)
    ncode = 3 * (I * H // 2)
    out[:ncode] = _random_bytes(rng, ncode)
    out[ncode:] = rng.integers(exp_lo, exp_hi + 1, size=n - ncode, dtype=np.uint8)
    return out


def int2_record(seed: int, stream: int, index: int, H: int, I: int, out: np.ndarray | None = None) -> np.ndarray:
    """One 2-bit expert record: codes uniform over 0..3, positive E4M3 scale
    bytes with exponent field INT2_EXPF_LO..INT2_EXPF_HI."""
    n = int2_record_nbytes(H, I)
    if out is None:
        out = np.empty(n, np.uint8)
    assert out.shape == (n,) and out.dtype == np.uint8
    rng = rng_for(seed, stream, index)
    ncode = 3 * (I * H // 4)
    out[:ncode] = _random_bytes(rng, ncode)
    m = n - ncode
    ef = rng.integers(INT2_EXPF_LO, INT2_EXPF_HI + 1, size=m, dtype=np.uint8)
    mant = rng.integers(0, 8, size=m, dtype=np.uint8)
    out[ncode:] = (ef << 3) | mant
    return out


def fp4_bank(seed: int, stream: int, n: int, H: int, I: int, out: np.ndarray | None = None,
             first_index: int = 0) -> np.ndarray:
    """n FP4 records back to back, record i drawn from substream first_index + i."""
    rb = fp4_record_nbytes(H, I)
    if out is None:
        out = np.empty((n, rb), np.uint8)
    for i in range(n):
        fp4_record(seed, stream, first_index + i, H, I, out=out[i])
    return out


def int2_bank(seed: int, stream: int, n: int, H: int, I: int, out: np.ndarray | None = None,
              first_index: int = 0) -> np.ndarray:
    rb = int2_record_nbytes(H, I)
    if out is None:
        out = np.empty((n, rb), np.uint8)
    for i in range(n):
        int2_record(seed, stream, first_index + i, H, I, out=out[i])
    return out


def f32_normal(seed: int, keys: tuple, shape, std: float = 1.0) -> np.ndarray:
    rng = rng_for(seed, *keys)
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def bf16_bits_from_f32(v: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of finite float32 values, round to nearest even.
    Used only to draw bf16 activations; integer bit manipulation."""
    u = np.ascontiguousarray(v, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_normal(seed: int, keys: tuple, shape) -> np.ndarray:
    """N(0,1) activations as bf16 bit patterns (uint16)."""
    return bf16_bits_from_f32(f32_normal(seed, keys, shape))


def zipf_bias(seed: int, keys: tuple, E: int, s: float) -> np.ndarray:
    """Per-expert popularity bias -s*ln(rank), rank a seeded permutation of 1..E."""
    rng = rng_for(seed, *keys)
    rank = rng.permutation(E).astype(np.float64) + 1.0
    return (-s * np.log(rank)).astype(np.float32)


def router_logits(seed: int, keys: tuple, T: int, E: int, bias: np.ndarray | None = None) -> np.ndarray:
    """N(0,1) router logits [T,E] fp32, plus an optional per-expert bias."""
    lg = f32_normal(seed, keys, (T, E))
    if bias is not None:
        lg = (lg + bias[None, :]).astype(np.float32)
    return lg


# ----------------------------------------------------------------------------
# the five workloads

WORKLOADS = {
    "tiny": dict(name="tiny-cpu-checkable", seed=1000, E=8, H=256, I=128, k=2, T=4, shared=False,
                 x_dtype="f32", out_dtype="f32", router="x", router_std=0.02),
    "decode-b1": dict(name="decode-b1-E256-top8-shared", seed=1001, E=256, H=4096, I=2048, k=8, T=1,
                      shared=True, x_dtype="bf16", out_dtype="bf16", router="logits"),
    "decode-b64": dict(name="decode-b64-E256-top6-zipf-shared", seed=1002, E=256, H=4096, I=2048, k=6,
                       T=64, shared=True, x_dtype="bf16", out_dtype="bf16", router="logits", zipf=1.1),
    "prefill": dict(name="prefill-4096-E256-top8-shared", seed=1003, E=256, H=4096, I=2048, k=8, T=4096,
                    shared=True, x_dtype="bf16", out_dtype="bf16", router="logits"),
    "slotcache": dict(name="slotcache-decode-L8-E256-S512-top6-ladder24", seed=1004, L=8, E=256, H=4096,
                      I=2048, k=6, T=512, shared=False, x_dtype="bf16", out_dtype="bf16", router="logits",
                      zipf=1.1, slots=512, ladder=(2, 4)),
}


def make_layer_inputs(cfg: dict, seed: int, step: int = 0, with_bank: bool = True) -> dict:
    """Inputs of one single-layer workload (tiny, decode-b1, decode-b64, prefill).

    step selects fresh activations and logits (bank and router weights are
    fixed per seed)."""
    E, H, I, T = cfg["E"], cfg["H"], cfg["I"], cfg["T"]
    d = dict(cfg=cfg, seed=seed, step=step)
    if with_bank:
        d["bank"] = fp4_bank(seed, S_BANK, E, H, I)
        d["shared_rec"] = fp4_record(seed, S_SHARED, 0, H, I) if cfg["shared"] else None
    if cfg["x_dtype"] == "f32":
        d["x"] = f32_normal(seed, (S_X, step), (T, H))
    else:
        d["x"] = bf16_normal(seed, (S_X, step), (T, H))
    if cfg["router"] == "x":
        d["router_w"] = f32_normal(seed, (S_ROUTER_W,), (E, H), std=cfg["router_std"])
        d["logits"] = None
    else:
        bias = zipf_bias(seed, (S_ZIPF,), E, cfg["zipf"]) if "zipf" in cfg else None
        d["logits"] = router_logits(seed, (S_LOGITS, step), T, E, bias)
    return d


def slotcache_logits(seed: int, L: int, E: int, T: int, s: float) -> np.ndarray:
    """Router logits [T, L, E] of the slot-cache decode workload: per-layer
    Zipf popularity (a separate permutation per layer) plus N(0,1) noise."""
    out = np.empty((T, L, E), np.float32)
    for l in range(L):
        bias = zipf_bias(seed, (S_ZIPF, l), E, s)
        out[:, l, :] = router_logits(seed, (S_LOGITS, l), T, E, bias)
    return out


def slotcache_x(seed: int, t: int, l: int, H: int) -> np.ndarray:
    """Independent bf16 N(0,1) input of token t at layer l, [1, H]."""
    return bf16_normal(seed, (S_X, t, l), (1, H))


def predicted_experts(seed: int, keys: tuple, ranked, k: int, m: int = 12, recall: float = 0.75) -> np.ndarray:
    """A synthetic expert prediction of controlled recall for one (token,
    layer), standing in for the pages' trained router predictor (it needs
    trained weights; out of scope).  ranked: that call's experts in the
    router's rank order, at least k + m long (the caller's top-(k+m) routing).
    The prediction holds round(recall * k) of the first k (a seeded subset),
    filled up to m ids with the experts ranked right after the first k (a
    predictor's false positives are near misses, not uniform draws), in
    ranked order."""
    ranked = np.asarray(ranked, np.int64).reshape(-1)
    n_true = int(round(recall * k))
    assert 0 <= n_true <= min(k, m) and len(ranked) >= k + m - n_true
    rng = rng_for(seed, S_PRED, *keys)
    keep = set(rng.choice(ranked[:k], n_true, replace=False).tolist())
    pred = [e for e in ranked[:k] if e in keep] + ranked[k:k + m - n_true].tolist()
    return np.asarray(pred, np.int32)
