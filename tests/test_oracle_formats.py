"""Pins of the oracle's formats and sizes against the format definitions and
the numbers printed on the pages (no GPU)."""
import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from tests.conftest import read_golden


def _e2m1_from_bits(code):
    # sign-magnitude with bias-1 exponent; exponent field 0 is subnormal
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    return s * (m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m))


def test_e2m1_table_matches_golden_and_bitfields():
    rows = read_golden("e2m1_values.txt")
    assert len(rows) == 16
    for code_s, val_s in rows:
        code, val = int(code_s, 16), float(val_s)
        got = O.E2M1_VALUES[code]
        assert got == val and math.copysign(1, got) == math.copysign(1, val)
        assert _e2m1_from_bits(code) == val


def test_e4m3_points_golden():
    for code_s, val_s in read_golden("e4m3_points.txt"):
        code, val = int(code_s, 16), float(val_s)
        got = O.e4m3_value(code)
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val)


def test_e4m3_structure():
    v = O.E4M3_VALUES
    assert np.isnan(v).sum() == 2                       # 0x7f and 0xff only
    pos = v[:127]
    assert np.all(np.diff(pos) > 0)                     # monotone in the code
    assert pos.max() == 448.0
    assert np.array_equal(v[128:255], -v[:127])         # sign symmetry
    # consecutive normals within one binade differ by 2^(e-10)
    assert v[0x39] - v[0x38] == 2.0 ** -3


def test_e8m0():
    assert O.e8m0_value(127) == 1.0
    assert O.e8m0_value(0) == 2.0 ** -127
    assert O.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(O.e8m0_value(255))


@pytest.mark.parametrize("expo", [0, 1, 119, 120, 121, 122, 123, 127, 254, 255])
def test_every_fp4_code_times_scale(expo):
    """All 16 codes x chosen E8M0 exponents through the record path, with
    the nibble order fixed by a hand-built row."""
    H, I = 64, 32
    rec = np.zeros(O.fp4_expert_nbytes(H, I), np.uint8)
    parts = O.split_record(rec, H, I, 4)
    # row 0 of w1: codes 0..15 then 15..0 (elements 0..31), then 0..15 again
    seq = np.array(list(range(16)) + list(range(15, -1, -1)) + list(range(16)) * 2, np.uint8)[:H]
    parts["w1_codes"][0] = seq[0::2] | (seq[1::2] << 4)
    parts["w1_scales"][0, :] = expo
    W1, W3, W2 = O.expert_weights(rec, H, I, 0)
    for i in range(H):
        want = _e2m1_from_bits(int(seq[i])) * (math.nan if expo == 255 else 2.0 ** (expo - 127))
        got = W1[0, i]
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want, (i, got, want)
    assert np.all(W1[1:] == 0) and np.all(W3 == 0) and np.all(W2 == 0)


def test_nibble_order_single_byte():
    # byte 0x21: element 0 = low nibble 1 (0.5), element 1 = high nibble 2 (1.0)
    c = O.unpack_fp4_codes(np.array([[0x21]], np.uint8))
    assert c.tolist() == [[1, 2]]


def test_int2_levels_and_order():
    # byte 0xE4 = 0b11_10_01_00: elements 0..3 carry codes 0, 1, 2, 3
    codes = np.zeros((1, 8), np.uint8)
    codes[0, 0] = 0xE4
    scales = np.array([[0x38]], np.uint8)                # e4m3 1.0
    W = O.dequant_int2(codes, scales)
    assert W[0, :4].tolist() == [-1.5, -0.5, 0.5, 1.5]
    assert np.all(W[0, 4:] == -1.5)                      # code 0 elsewhere
    scales2 = np.array([[0x40]], np.uint8)               # e4m3 2.0
    assert O.dequant_int2(codes, scales2)[0, :4].tolist() == [-3.0, -1.0, 1.0, 3.0]


def test_record_split_covers_every_byte():
    H, I = 256, 128
    n = O.fp4_expert_nbytes(H, I)
    rec = np.arange(n, dtype=np.uint64).astype(np.uint8)
    parts = O.split_record(rec, H, I, 4)
    total = sum(p.size for p in parts.values())
    assert total == n
    n2 = O.int2_expert_nbytes(H, I)
    parts2 = O.split_record(np.zeros(n2, np.uint8), H, I, 2)
    assert sum(p.size for p in parts2.values()) == n2


def test_page_constants():
    c = {r[0]: (float(r[1]), float(r[2])) for r in read_golden("page_constants.txt")}
    H, I, E, L = 4096, 2048, 256, 43
    fp4 = O.fp4_expert_nbytes(H, I)
    int2 = O.int2_expert_nbytes(H, I)
    v, tol = c["fp4_expert_bytes"]
    assert fp4 == v
    v, tol = c["int2_expert_megabytes"]
    assert abs(int2 / 2 ** 20 - v) <= tol
    v, tol = c["int2_bits_per_weight"]
    assert int2 * 8 / (3 * H * I) == v
    v, tol = c["int2_all_layers_gb"]
    assert abs(L * E * int2 / 1e9 - v) <= tol
    v, tol = c["per_token_working_set_gb"]
    assert abs(260 * fp4 / 1e9 - v) <= tol
    v, tol = c["per_token_read_ms"]
    assert abs(v / 1e3 * 6.2e9 - 3.4e9) / 3.4e9 < 0.01          # the page's own chain
    assert abs(260 * fp4 / 6.2e9 * 1e3 - v) <= tol
    v, tol = c["codes_per_layer_gb"]
    assert abs(E * 3 * H * I / 2 / 1e9 - v) <= tol                # codes only, no scales
    v, tol = c["bf16_expand_gib"]
    assert abs(268.9 * 16 / (fp4 * 8 / (3 * H * I)) - v) <= tol  # 16 bits over 4.25 bits
    v, tol = c["resident_fraction_pct"]
    assert abs(100 * 4080 / (43 * 256) - v) <= tol
    v, tol = c["slots_per_layer"]
    assert abs(4080 / 43 - v) <= tol
    v, tol = c["prefill_crossover_tokens"]
    assert math.ceil(E / 8) == v
    assert min(T for T in range(1, 300) if O.prefill_streams(T, 8, E)) == v
    v, tol = c["stream_min_slots"]
    O.SlotCache(1, E, int(v), 8, 8, 8).stream_layer(0)
    with pytest.raises(AssertionError):
        O.SlotCache(1, E, int(v) - 1, 8, 8, 8).stream_layer(0)
