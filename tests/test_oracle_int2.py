"""Pins of the oracle's 2-bit copy of an MXFP4 expert (clip search per 32
weights, "An elephant through a straw", opening section: 2-bit codes with an
fp8 scale per 32 weights, the scale chosen by clip search).

The pins do not retype the oracle's formula: the nearest level is found by
trying all four codes, the clip ratio by trying every candidate scale with
those brute-force levels, and closed forms cover blocks that lie on a
2-bit grid and all-zero blocks."""
import numpy as np

from oracle import moe_oracle as O
from mxfp4_routed_expert_renorm_amd import workloads as W


def _levels_by_brute_force(w, s):
    """For each weight the code 0..3 whose level (c - 1.5) s is nearest; a tie
    goes to the even code (round half to even of w / s + 1.5)."""
    best = np.zeros(w.shape, np.uint8)
    for i, v in np.ndenumerate(w):
        d = [abs(v - (c - 1.5) * s) for c in range(4)]
        m = min(d)
        cands = [c for c in range(4) if d[c] == m]
        best[i] = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return best


def test_block_on_a_two_bit_grid_is_reproduced_exactly():
    """Weights that are levels of an E4M3 scale, with the largest level
    present: alpha = 1 reproduces them with zero error."""
    rng = np.random.default_rng(3)
    for scale_code in (0x28, 0x30, 0x3B, 0x45, 0x04):   # normal and subnormal E4M3 scales
        s0 = float(O.e4m3_value(scale_code))
        c = rng.integers(0, 4, size=(3, 32)).astype(np.uint8)
        c[:, 0] = 3                                      # max |w| = 1.5 s0
        w = (c.astype(np.float64) - 1.5) * s0
        codes, scales = O.quant_int2_clip(w)
        assert np.array_equal(codes, c)
        assert np.all(scales == scale_code)


def test_all_zero_block_takes_scale_zero_and_level_zero():
    codes, scales = O.quant_int2_clip(np.zeros((2, 64)))
    assert np.all(scales == 0)
    assert np.all(codes == 2)                             # level +0.5 * 0 = 0


def test_codes_are_the_nearest_levels_of_the_chosen_scale():
    rec = W.fp4_record(11, 1, 0, 256, 128)
    W1 = O.expert_weights(rec, 256, 128)[0][:4]           # 4 rows x 256 weights
    codes, scales = O.quant_int2_clip(W1)
    for r in range(W1.shape[0]):
        for b in range(W1.shape[1] // 32):
            s = float(O.e4m3_value(scales[r, b]))
            blk = W1[r, 32 * b:32 * b + 32]
            assert np.array_equal(codes[r, 32 * b:32 * b + 32], _levels_by_brute_force(blk, s)), (r, b)


def test_the_chosen_scale_beats_every_other_candidate():
    """Each candidate scale E4M3(alpha * amax / 1.5), with brute-force nearest
    levels: the chosen one has the least squared error, the earliest alpha
    among equals."""
    rec = W.fp4_record(12, 1, 0, 128, 128)
    W2 = O.expert_weights(rec, 128, 128)[2][:3]
    codes, scales = O.quant_int2_clip(W2)
    for r in range(W2.shape[0]):
        for b in range(W2.shape[1] // 32):
            blk = W2[r, 32 * b:32 * b + 32]
            amax = max(abs(v) for v in blk)
            errs, cand = [], []
            for alpha in O.CLIP_ALPHAS:
                sc = int(O.e4m3_encode(alpha * amax / 1.5))
                s = float(O.e4m3_value(sc))
                lv = _levels_by_brute_force(blk, s)
                e = 0.0
                for v, c in zip(blk, lv):
                    e = e + (v - (c - 1.5) * s) ** 2
                errs.append(e)
                cand.append(sc)
            want = cand[int(np.argmin(errs))]                # argmin: first of equals
            assert scales[r, b] == want, (r, b, errs)


def test_record_round_trip_and_row_subsets():
    """The packed record dequantises (through the 2-bit decode) to the levels
    the search chose, and computing a subset of rows gives those rows' bytes."""
    H, I = 256, 128
    rec = W.fp4_record(13, 1, 0, H, I)
    r2 = O.int2_record_from_fp4(rec, H, I)
    assert r2.size == O.int2_expert_nbytes(H, I)
    Wf = O.expert_weights(rec, H, I)
    Wq = O.expert_weights(r2, H, I, prec=1)
    for a, q in zip(Wf, Wq):
        c, sc = O.quant_int2_clip(a)
        assert np.array_equal(q, (c.astype(np.float64) - 1.5) * np.repeat(O.e4m3_value(sc), 32, axis=1))
    rows = {"w1": [0, 5, 127], "w3": [7], "w2": [1, 255]}
    part = O.int2_record_from_fp4(rec, H, I, rows=rows)
    p_full, p_part = O.split_record(r2, H, I, 2), O.split_record(part, H, I, 2)
    for name, idx in rows.items():
        assert np.array_equal(p_full[name + "_codes"][idx], p_part[name + "_codes"][idx])
        assert np.array_equal(p_full[name + "_scales"][idx], p_part[name + "_scales"][idx])
