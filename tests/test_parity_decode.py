"""GPU parity of the decode path against the CPU oracle, through the C ABI.

Bit-exact: dequantised weights (every FP4 code x every E8M0 byte, every 2-bit
code x every E4M3 byte), routing ids, grouping.  Within tolerance: router
weights, expert outputs and the combined layer output."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from mxfp4_routed_expert_renorm_amd import workloads as W
from tests.gpu_util import (TOL_BF16_MAX_REL, TOL_F32_REL_L2, bf16_dev, dev, log, max_rel, rel_l2, to_f64)

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


# ------------------------------------------------------------------ formats

def _exhaustive_fp4_record(H, I):
    """Record whose w1 covers every (code, E8M0 byte) pair: block b has scale
    b % 256 and codes cycling 0..15 twice."""
    rec = np.zeros(O.fp4_expert_nbytes(H, I), np.uint8)
    p = O.split_record(rec, H, I, 4)
    nblk = I * H // 32
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)
    elems = np.tile(codes, nblk).reshape(I, H)
    p["w1_codes"][:] = elems[:, 0::2] | (elems[:, 1::2] << 4)
    p["w1_scales"][:] = (np.arange(nblk) % 256).reshape(I, H // 32).astype(np.uint8)
    rng = np.random.default_rng(3)
    p["w3_codes"][:] = rng.integers(0, 256, p["w3_codes"].shape, dtype=np.uint8)
    p["w3_scales"][:] = rng.integers(0, 256, p["w3_scales"].shape, dtype=np.uint8)
    p["w2_codes"][:] = rng.integers(0, 256, p["w2_codes"].shape, dtype=np.uint8)
    p["w2_scales"][:] = rng.integers(0, 256, p["w2_scales"].shape, dtype=np.uint8)
    return rec


def _same_bits(got, want):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float64).astype(np.float32)
    nan_ok = np.isnan(got) == np.isnan(want)
    eq = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    return bool(np.all(nan_ok) and np.all(eq))


def test_dequant_fp4_bit_exact_all_codes_all_scales(gpu_lib):
    torch = _torch()
    H, I = 256, 128
    rec = _exhaustive_fp4_record(H, I)
    want = O.expert_weights(rec, H, I, 0)
    d_rec = dev(rec)
    for m in range(3):
        rows, cols = (I, H) if m < 2 else (H, I)
        out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
        gpu_lib.moe_debug_dequant(d_rec, H, I, 0, m, out)
        torch.cuda.synchronize()
        assert _same_bits(out.cpu().numpy(), want[m]), f"matrix {m}"


def test_dequant_int2_bit_exact_all_codes_all_scales(gpu_lib):
    torch = _torch()
    H, I = 256, 128
    rec = np.zeros(O.int2_expert_nbytes(H, I), np.uint8)
    p = O.split_record(rec, H, I, 2)
    nblk = I * H // 32
    p["w1_codes"][:] = 0xE4                        # codes 0,1,2,3 repeating
    p["w1_scales"][:] = (np.arange(nblk) % 256).reshape(I, H // 32).astype(np.uint8)
    rng = np.random.default_rng(5)
    for k in ("w3_codes", "w2_codes", "w3_scales", "w2_scales"):
        p[k][:] = rng.integers(0, 256, p[k].shape, dtype=np.uint8)
    want = O.expert_weights(rec, H, I, 1)
    d_rec = dev(rec)
    for m in range(3):
        rows, cols = (I, H) if m < 2 else (H, I)
        out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
        gpu_lib.moe_debug_dequant(d_rec, H, I, 1, m, out)
        torch.cuda.synchronize()
        assert _same_bits(out.cpu().numpy(), want[m]), f"matrix {m}"


# ------------------------------------------------------------------ routing

def _route_gpu(gpu_lib, logits, k):
    torch = _torch()
    T = logits.shape[0]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    gpu_lib.moe_route(dev(logits.astype(np.float32)), k, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("wl", ["decode-b1", "decode-b64", "prefill"])
def test_route_bit_exact_ids(gpu_lib, wl):
    cfg = W.WORKLOADS[wl]
    d = W.make_layer_inputs(cfg, cfg["seed"], step=0, with_bank=False)
    lg = d["logits"]
    log(f"route parity {wl}: T={lg.shape[0]} E={lg.shape[1]} k={cfg['k']}")
    ids, w = _route_gpu(gpu_lib, lg, cfg["k"])
    oids, ow = O.route(lg, cfg["k"])
    assert np.array_equal(ids, oids)
    assert np.max(np.abs(w - ow)) <= 1e-6
    assert np.max(np.abs(w.sum(axis=1) - 1)) <= 1e-6


def test_route_ties_ragged_and_edges(gpu_lib):
    rng = np.random.default_rng(9)
    cases = []
    lg = np.zeros((3, 8), np.float32)                      # all tied
    cases.append((lg, 3))
    lg = rng.integers(-2, 3, size=(37, 64)).astype(np.float32)   # many ties, ragged T
    cases.append((lg, 6))
    lg = rng.standard_normal((5, 1000)).astype(np.float32)        # E not a multiple of 64
    lg[:, 999] = 50.0
    cases.append((lg, 8))
    lg = rng.standard_normal((2, 17)).astype(np.float32)          # k == E
    cases.append((lg, 17))
    lg = np.full((1, 256), -0.0, np.float32)
    lg[0, ::2] = 0.0                                               # +0 and -0 tie
    cases.append((lg, 5))
    lg = np.full((3, 256), -np.inf, np.float32)                    # NaN counts as -inf
    lg[:, 1::3] = np.nan
    lg[0, [7, 100, 200]] = [1.5, 0.25, 3.0]                        # k-th pick among NaN / -inf
    lg[1, 5] = 0.0
    lg[2, :] = rng.standard_normal(256)
    lg[2, ::5] = np.nan
    cases.append((lg, 6))
    for lg, k in cases:
        ids, w = _route_gpu(gpu_lib, lg, k)
        oids, ow = O.route(lg, k)
        assert np.array_equal(ids, oids), (lg.shape, k)
        assert np.max(np.abs(w - ow)) <= 1e-6


def test_route_T0_is_noop(gpu_lib):
    torch = _torch()
    z = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    gpu_lib.moe_route(z, 2, ids, w)


def test_router_logits_and_decisions_tiny(gpu_lib):
    """Tiny configuration: router scores from x; the GPU decides on its fp32
    logits, the oracle on fp64 ones; decisions must agree wherever the k-th
    and (k+1)-th logits are not within 1e-5 of each other."""
    torch = _torch()
    cfg = W.WORKLOADS["tiny"]
    d = W.make_layer_inputs(cfg, W.WORKLOADS["tiny"]["seed"])
    T, E, H, k = cfg["T"], cfg["E"], cfg["H"], cfg["k"]
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    gpu_lib.moe_router_logits(dev(d["x"]), dev(d["router_w"]), logits)
    torch.cuda.synchronize()
    ol = O.router_logits(d["x"], d["router_w"])
    gl = logits.cpu().numpy()
    assert np.max(np.abs(gl - ol)) <= 1e-5 * np.abs(ol).max()
    ids, w = _route_gpu(gpu_lib, gl, k)
    oids, ow = O.route(ol, k)
    srt = np.sort(ol, axis=1)[:, ::-1]
    clear = (srt[:, k - 1] - srt[:, k]) > 1e-5
    assert clear.all(), "seeded tiny routing has a near-tie; choose another seed"
    assert np.array_equal(ids[clear], oids[clear])


# ------------------------------------------------------------------ grouping

def test_group_bit_exact(gpu_lib):
    torch = _torch()
    rng = np.random.default_rng(17)
    for n, nk in [(384, 257), (32768, 257), (36864, 257), (5, 3), (1000, 4096), (100000, 4096), (70001, 1000),
                  (64, 1), (0, 7)]:
        keys = rng.integers(0, nk, n).astype(np.int32)
        counts = torch.empty(nk, dtype=torch.int32, device="cuda")
        offsets = torch.empty(nk + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(n, dtype=torch.int32, device="cuda")
        gpu_lib.moe_group(dev(keys), nk, counts, offsets, perm)
        torch.cuda.synchronize()
        oc, oo, op = O.group_pairs(keys, nk)
        assert np.array_equal(counts.cpu().numpy(), oc)
        assert np.array_equal(offsets.cpu().numpy(), oo)
        assert np.array_equal(perm.cpu().numpy(), op)


def test_group_skips_out_of_range_keys(gpu_lib):
    torch = _torch()
    rng = np.random.default_rng(18)
    keys = rng.integers(-3, 40, 500).astype(np.int32)
    nk = 32
    counts = torch.empty(nk, dtype=torch.int32, device="cuda")
    offsets = torch.empty(nk + 1, dtype=torch.int32, device="cuda")
    valid = (keys >= 0) & (keys < nk)
    perm = torch.full((int(valid.sum()),), -1, dtype=torch.int32, device="cuda")
    gpu_lib.moe_group(dev(keys), nk, counts, offsets, perm)
    torch.cuda.synchronize()
    pos = np.nonzero(valid)[0]
    oc, oo, op = O.group_pairs(keys[valid], nk)
    assert np.array_equal(counts.cpu().numpy(), oc)
    assert np.array_equal(offsets.cpu().numpy(), oo)
    assert np.array_equal(perm.cpu().numpy(), pos[op])


def test_group_wide_bit_exact(gpu_lib):
    """The many-workgroup grouping (per-chunk histograms in scratch) gives the
    one-workgroup grouping's counts, offsets and permutation bit for bit,
    at prefill sizes, ragged tails and with out-of-range keys skipped."""
    torch = _torch()
    rng = np.random.default_rng(19)
    for n, nk, lo in [(2049, 257, 0), (36864, 257, 0), (100000, 257, 0), (70001, 1000, 0), (5000, 1024, 0),
                      (36864, 257, -5), (4096, 1, 0), (36864, 2000, 0), (1 << 20, 1024, 0)]:
        keys = rng.integers(lo, nk, n).astype(np.int32)
        valid = (keys >= 0) & (keys < nk)
        nv = int(valid.sum())
        sb = gpu_lib.moe_group_scratch_bytes(n, nk)
        assert sb == (0 if nk > 1024 else -(-n // 512) * nk * 4)
        scratch = torch.empty(max(sb // 4, 1), dtype=torch.int32, device="cuda")
        outs = []
        for wide in (True, False):
            counts = torch.full((nk,), -7, dtype=torch.int32, device="cuda")
            offsets = torch.full((nk + 1,), -7, dtype=torch.int32, device="cuda")
            perm = torch.full((nv,), -1, dtype=torch.int32, device="cuda")
            if wide:
                gpu_lib.moe_group_wide(dev(keys), nk, counts, offsets, perm, scratch)
            else:
                gpu_lib.moe_group(dev(keys), nk, counts, offsets, perm)
            torch.cuda.synchronize()
            outs.append([t.cpu().numpy() for t in (counts, offsets, perm)])
        pos = np.nonzero(valid)[0]
        oc, oo, op = O.group_pairs(keys[valid], nk)
        for c, o, pm in outs:
            assert np.array_equal(c, oc), (n, nk)
            assert np.array_equal(o, oo), (n, nk)
            assert np.array_equal(pm, pos[op]), (n, nk)


def test_dequant_fp4_scaled_convert_bit_exact_all_codes_all_scales(gpu_lib):
    """The decode of the batch-1, single-launch and batched-decode kernels:
    the scaled FP4-to-bf16 convert with the E8M0 scale as its operand, for
    every FP4 code times every E8M0 byte, equals the oracle's
    E2M1 value x 2^(e-127) bit for bit (rounded to float32: past the float
    range the product is infinite, as in bf16)."""
    torch = _torch()
    H, I = 256, 128
    rec = _exhaustive_fp4_record(H, I)
    want = O.expert_weights(rec, H, I, 0)
    d_rec = dev(rec)
    for m in range(3):
        rows, cols = (I, H) if m < 2 else (H, I)
        out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
        gpu_lib.moe_debug_dequant(d_rec, H, I, 2, m, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ok = _same_bits(got, want[m])
        if not ok:
            bad = np.nonzero(got.view(np.uint32) != np.asarray(want[m], np.float64).astype(np.float32).view(np.uint32))
            log(f"matrix {m}: {len(bad[0])} mismatches, first {[(got[i, j], want[m][i, j]) for i, j in zip(*bad)][:6]}")
        assert ok, f"matrix {m}"


# ------------------------------------------------------------- layer outputs

class Layer:
    """A fully resident layer on the GPU: bank [E, rec] (+ shared record)."""

    def __init__(self, gpu_lib, bank, shared, H, I, int2_bank=None):
        self.lib = gpu_lib
        self.H, self.I = H, I
        self.bank = dev(bank)
        self.shared = dev(shared) if shared is not None else None
        self.int2 = dev(int2_bank) if int2_bank is not None else None
        self.desc = gpu_lib.make_layer(
            H, I, fp4_base=self.bank, fp4_stride=bank.shape[1], num_slots=bank.shape[0],
            int2_base=self.int2, int2_stride=(int2_bank.shape[1] if int2_bank is not None else 0),
            num_int2=(int2_bank.shape[0] if int2_bank is not None else 0), shared=self.shared)

    def forward(self, x_dev, T, k, slots, prec, w, out):
        torch = _torch()
        ws = self.lib.expert_workspace(self.H, self.I, T, k, self.shared is not None)
        self.lib.moe_expert_forward(self.desc, x_dev, T, k, slots, prec, w, out, ws)
        return out


def _layer_check(gpu_lib, wl, steps=(0,), bank=None):
    torch = _torch()
    cfg = W.WORKLOADS[wl]
    seed = cfg["seed"]
    E, H, I, k, T = cfg["E"], cfg["H"], cfg["I"], cfg["k"], cfg["T"]
    if bank is None:
        d0 = W.make_layer_inputs(cfg, seed, 0)
        bank, shared = d0["bank"], d0["shared_rec"]
    else:
        bank, shared = bank
    layer = Layer(gpu_lib, bank, shared, H, I)
    wcache = {}
    for step in steps:
        d = W.make_layer_inputs(cfg, seed, step, with_bank=False)
        log(f"layer parity {wl} step {step}")
        if cfg["x_dtype"] == "f32":
            x_dev = dev(d["x"])
            x64 = d["x"].astype(np.float64)
        else:
            x_dev = bf16_dev(d["x"])
            x64 = O.bf16_bits_to_f64(d["x"])
        if d["logits"] is None:
            lg_dev = torch.empty((T, E), dtype=torch.float32, device="cuda")
            gpu_lib.moe_router_logits(x_dev, dev(d["router_w"]), lg_dev)
            ol = O.router_logits(d["x"], d["router_w"])
        else:
            lg_dev = dev(d["logits"])
            ol = d["logits"]
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        gpu_lib.moe_route(lg_dev, k, ids, w)
        K1 = k + (1 if shared is not None else 0)
        odt = torch.float32 if cfg["out_dtype"] == "f32" else torch.bfloat16
        out = torch.empty((T, H), dtype=odt, device="cuda")
        layer.forward(x_dev, T, k, ids, None, w, out)
        yr = torch.empty((T, K1, H), dtype=torch.float32, device="cuda")
        layer.forward(x_dev, T, k, ids, None, None, yr)
        torch.cuda.synchronize()
        oids, ow = O.route(ol, k)
        assert np.array_equal(ids.cpu().numpy(), oids)
        # oracle per-rank outputs (each expert dequantised once) and their combine
        yo = np.zeros((T, K1, H))
        for t in range(T):
            for r in range(K1):
                key = int(oids[t, r]) if r < k else -1
                if key not in wcache:
                    wcache[key] = O.expert_weights(bank[key] if r < k else shared, H, I)
                yo[t, r] = O.expert_mlp(x64[t], *wcache[key])
        ref = np.stack([O.combine(yo[t, :k], ow[t], yo[t, k] if K1 > k else None) for t in range(T)])
        got = to_f64(out)
        if cfg["out_dtype"] == "f32":
            err = rel_l2(got, ref)
            log(f"  rel-L2 {err:.3e}")
            assert err <= TOL_F32_REL_L2
        else:
            err = max_rel(got, ref)
            log(f"  max-rel {err:.3e}")
            assert err <= TOL_BF16_MAX_REL
        # per-rank outputs (fp32) against each expert evaluated alone
        yg = yr.cpu().numpy().astype(np.float64)
        for t in range(T):
            for r in range(K1):
                e = rel_l2(yg[t, r], yo[t, r])
                assert e <= TOL_F32_REL_L2, (t, r, e)


def test_layer_tiny_fp32(gpu_lib):
    _layer_check(gpu_lib, "tiny", steps=(0, 1, 2))


def test_layer_decode_b1_full_size(gpu_lib):
    """Batch-1 decode at the full shape (256 experts + shared, H 4096,
    I 2048, top-8), the launch configuration the benchmark times."""
    _layer_check(gpu_lib, "decode-b1", steps=(0, 1))


def _mixed_case(gpu_lib, T, xbf16, with_shared, seed):
    """Mid-size layer (several tiles, 2-bit copies, drops) in both modes."""
    torch = _torch()
    H, I, E, k, NI = 512, 256, 16, 4, 12
    bank = W.fp4_bank(seed, 1, E, H, I)
    int2 = W.int2_bank(seed, 7, NI, H, I)
    shared = W.fp4_record(seed, 2, 0, H, I) if with_shared else None
    layer = Layer(gpu_lib, bank, shared, H, I, int2_bank=int2)
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    prec = rng.choice([0, 0, 1, -1], size=(T, k)).astype(np.int8)
    slots = np.where(prec == 1, rng.integers(0, NI, (T, k)), ids).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    if xbf16:
        xb = W.bf16_normal(seed, (3,), (T, H))
        x_dev, x64 = bf16_dev(xb), O.bf16_bits_to_f64(xb)
    else:
        xf = W.f32_normal(seed, (3,), (T, H))
        x_dev, x64 = dev(xf), xf.astype(np.float64)
    K1 = k + (1 if with_shared else 0)
    yr = torch.empty((T, K1, H), dtype=torch.float32, device="cuda")
    layer.forward(x_dev, T, k, dev(slots), dev(prec), None, yr)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    layer.forward(x_dev, T, k, dev(slots), dev(prec), dev(w), out)
    torch.cuda.synchronize()
    yg = yr.cpu().numpy().astype(np.float64)

    def rec_of(t, r):
        return int2[slots[t, r]] if prec[t, r] == 1 else bank[slots[t, r]]

    ref = np.zeros((T, H))
    for t in range(T):
        for r in range(K1):
            if r < k and prec[t, r] < 0:
                assert np.all(yg[t, r] == 0)
                continue
            rec, pr = (rec_of(t, r), int(prec[t, r])) if r < k else (shared, 0)
            yo = O.expert_mlp(x64[t], *O.expert_weights(rec, H, I, pr))
            assert rel_l2(yg[t, r], yo) <= TOL_F32_REL_L2, (t, r)
            ref[t] += (w[t, r] if r < k else 1.0) * yo
    assert rel_l2(out.cpu().numpy(), ref) <= TOL_F32_REL_L2


@pytest.mark.parametrize("T", [1, 3, 33])
@pytest.mark.parametrize("xbf16", [False, True])
def test_layer_mixed_precision_and_drops(gpu_lib, T, xbf16):
    _mixed_case(gpu_lib, T, xbf16, with_shared=True, seed=100 + T)


def test_layer_no_shared_batched(gpu_lib):
    _mixed_case(gpu_lib, 7, True, with_shared=False, seed=77)


def test_all_dropped_gives_shared_only(gpu_lib):
    torch = _torch()
    H, I, E, k = 256, 128, 8, 2
    bank = W.fp4_bank(5, 1, E, H, I)
    shared = W.fp4_record(5, 2, 0, H, I)
    layer = Layer(gpu_lib, bank, shared, H, I)
    x = W.f32_normal(5, (3,), (2, H))
    prec = np.full((2, k), -1, np.int8)
    slots = np.zeros((2, k), np.int32)
    w = np.zeros((2, k), np.float32)
    out = torch.empty((2, H), dtype=torch.float32, device="cuda")
    layer.forward(dev(x), 2, k, dev(slots), dev(prec), dev(w), out)
    torch.cuda.synchronize()
    ys = O.expert_mlp(x.astype(np.float64), *O.expert_weights(shared, H, I))
    assert rel_l2(out.cpu().numpy(), ys) <= TOL_F32_REL_L2


def test_combine_standalone(gpu_lib):
    torch = _torch()
    rng = np.random.default_rng(1)
    T, k, H = 5, 3, 64
    y = rng.standard_normal((T, k + 1, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    prec = np.array([[0, -1, 0]] * T, np.int8)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    gpu_lib.moe_combine(dev(y), dev(w), dev(prec), T, k, H, True, out)
    torch.cuda.synchronize()
    ref = np.stack([O.combine(y[t, :k].astype(np.float64), np.where(prec[t] < 0, 0, w[t]), y[t, k]) for t in range(T)])
    assert rel_l2(out.cpu().numpy(), ref) <= 1e-6


@pytest.mark.parametrize("xbf16", [True, False])
def test_layer_b1_fused_path_mixed_precision(gpu_lib, xbf16):
    """Batch 1 at H = I = 2048: bf16 activations take the batch-1 streaming
    kernels, fp32 the generic ones; mix FP4, 2-bit copies and drops, with the
    shared expert."""
    torch = _torch()
    H, I, E, k, NI = 2048, 2048, 12, 6, 3
    seed = 31 + int(xbf16)
    bank = W.fp4_bank(seed, 1, E, H, I)
    int2 = W.int2_bank(seed, 7, NI, H, I)
    shared = W.fp4_record(seed, 2, 0, H, I)
    layer = Layer(gpu_lib, bank, shared, H, I, int2_bank=int2)
    ids = np.array([[3, 7, 0, 11, 5, 9]], np.int32)
    prec = np.array([[0, 0, 1, 1, 0, -1]], np.int8)
    slots = np.array([[3, 7, 0, 2, 5, -1]], np.int32)
    w = np.array([[0.3, 0.25, 0.2, 0.1, 0.15, 0.0]], np.float32)
    if xbf16:
        xb = W.bf16_normal(seed, (3,), (1, H))
        x_dev, x64 = bf16_dev(xb), O.bf16_bits_to_f64(xb)
        odt = torch.bfloat16
    else:
        xf = W.f32_normal(seed, (3,), (1, H))
        x_dev, x64 = dev(xf), xf.astype(np.float64)
        odt = torch.float32
    out = torch.empty((1, H), dtype=odt, device="cuda")
    layer.forward(x_dev, 1, k, dev(slots), dev(prec), dev(w), out)
    torch.cuda.synchronize()
    ref = np.zeros(H)
    for r in range(k):
        if prec[0, r] < 0:
            continue
        rec = int2[slots[0, r]] if prec[0, r] == 1 else bank[slots[0, r]]
        ref += w[0, r] * O.expert_mlp(x64[0], *O.expert_weights(rec, H, I, int(prec[0, r])))
    ref += O.expert_mlp(x64[0], *O.expert_weights(shared, H, I))
    got = to_f64(out)[0]
    if xbf16:
        err = max_rel(got, ref)
        log(f"b1 fused path bf16: max-rel {err:.3e}")
        assert err <= TOL_BF16_MAX_REL
    else:
        err = rel_l2(got, ref)
        log(f"b1 fused path fp32: rel-L2 {err:.3e}")
        assert err <= TOL_F32_REL_L2


# ------------------------------------------------------------ moe_layer_decode

def _tiled_bank(seed, E, H, I, distinct=8):
    """E resident experts built from `distinct` seeded records (expert e uses
    record e % distinct): a full-size bank without generating E records."""
    recs = W.fp4_bank(seed, W.S_BANK, distinct, H, I)
    torch = _torch()
    d = dev(recs)
    bank = torch.cat([d] * ((E + distinct - 1) // distinct))[:E].contiguous()
    return recs, bank


def _layer_decode_case(gpu_lib, E, H, I, k, with_shared, seed, out_f32=False):
    torch = _torch()
    recs, bank = _tiled_bank(seed, E, H, I)
    rb = recs.shape[1]
    shared = W.fp4_record(seed, W.S_SHARED, 0, H, I) if with_shared else None
    sh_dev = dev(shared) if with_shared else None
    desc = gpu_lib.make_layer(H, I, fp4_base=bank, fp4_stride=rb, num_slots=E, shared=sh_dev)
    lg = W.router_logits(seed, (W.S_LOGITS,), 1, E)
    xb = W.bf16_normal(seed, (W.S_X,), (1, H))
    x_dev = bf16_dev(xb)
    odt = torch.float32 if out_f32 else torch.bfloat16
    ws = gpu_lib.expert_workspace(H, I, 1, k, with_shared)
    ids = torch.full((k,), -7, dtype=torch.int32, device="cuda")
    w = torch.full((k,), -7.0, dtype=torch.float32, device="cuda")
    out = torch.empty((1, H), dtype=odt, device="cuda")
    gpu_lib.moe_layer_decode(desc, dev(lg[0]), x_dev, k, ids, w, out, ws)
    # the same token through the separate calls
    ids2 = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w2 = torch.empty((1, k), dtype=torch.float32, device="cuda")
    out2 = torch.empty((1, H), dtype=odt, device="cuda")
    gpu_lib.moe_route(dev(lg), k, ids2, w2)
    gpu_lib.moe_expert_forward(desc, x_dev, 1, k, ids2, None, w2, out2, ws)
    torch.cuda.synchronize()
    oids, ow = O.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), oids[0])
    assert np.array_equal(ids2.cpu().numpy()[0], oids[0])
    assert np.array_equal(w.cpu().numpy(), w2.cpu().numpy()[0])          # one routing code path
    assert np.max(np.abs(w.cpu().numpy() - ow[0])) <= 1e-6
    # routing inside the gate/up kernel changes nothing downstream
    assert torch.equal(out, out2)
    ref = O.layer_forward(O.bf16_bits_to_f64(xb), oids, ow, lambda e: recs[int(e) % recs.shape[0]], H, I,
                          shared_rec=shared)
    got = to_f64(out)
    if out_f32:
        err = rel_l2(got, ref)
        log(f"layer_decode E={E} H={H} I={I} k={k} shared={with_shared}: rel-L2 {err:.3e}")
        assert err <= TOL_F32_REL_L2
    else:
        err = max_rel(got, ref)
        log(f"layer_decode E={E} H={H} I={I} k={k} shared={with_shared}: max-rel {err:.3e}")
        assert err <= TOL_BF16_MAX_REL


def test_layer_decode_full_shape(gpu_lib):
    """The decode workload's shape (256 experts + shared, H 4096, I 2048,
    top-8) through the single-call path, routed inside the gate/up kernel."""
    _layer_decode_case(gpu_lib, 256, 4096, 2048, 8, True, seed=81)


@pytest.mark.parametrize("E,k,with_shared,out_f32", [
    (100, 8, True, False),     # E not a multiple of 64: clamped logit loads
    (300, 6, False, False),    # E > 256: 16 logits per lane, no shared expert
    (64, 8, True, True),       # fp32 output: moe_route + the generic kernels
    (64, 1, True, False),      # k = 1
    (64, 11, True, False),     # 12 groups: the largest batch of the down kernel
])
def test_layer_decode_shapes(gpu_lib, E, k, with_shared, out_f32):
    _layer_decode_case(gpu_lib, E, 2048, 2048, k, with_shared, seed=90 + E + k, out_f32=out_f32)


@pytest.mark.parametrize("H,I,E,k,with_shared", [
    (2048, 256, 64, 8, True),      # H 2048, I 256: two wavefronts per gate/up row
    (2048, 512, 100, 6, True),     # one wavefront per row; E not a multiple of 64
    (2048, 1024, 300, 4, False),   # 16 logits per lane, no shared expert
    (4096, 512, 64, 11, True),     # 12 groups: the largest batch of the narrow kernels
    (4096, 1024, 64, 1, True),     # k = 1
])
def test_layer_decode_narrow_experts(gpu_lib, H, I, E, k, with_shared):
    """Tensor-parallel-share widths (the narrow-expert batch-1 kernels):
    routing inside the gate/up launch, each rank's slice requested right after
    the round that picks it, equal bit for bit to moe_route + moe_expert_forward
    from the same ids and within tolerance of the oracle."""
    _layer_decode_case(gpu_lib, E, H, I, k, with_shared, seed=97 + H // 1024 + I // 256 + k)


def test_layer_decode_generic_shape(gpu_lib):
    """A shape outside the batch-1 kernels (H 512) runs moe_route then the
    generic expert kernels; same contract."""
    _layer_decode_case(gpu_lib, 40, 512, 256, 4, True, seed=95)



def test_layer_decode_graph_replays(gpu_lib):
    """moe_layer_decode captured in a HIP graph and replayed, with eager calls
    between the replays: every replay equals the eager result."""
    torch = _torch()
    E, H, I, k, steps, seed = 40, 2048, 2048, 6, 6, 98
    recs, bank = _tiled_bank(seed, E, H, I)
    shared = dev(W.fp4_record(seed, W.S_SHARED, 0, H, I))
    desc = gpu_lib.make_layer(H, I, fp4_base=bank, fp4_stride=recs.shape[1], num_slots=E, shared=shared)
    ws = gpu_lib.expert_workspace(H, I, 1, k, True)
    lg = dev(W.router_logits(seed, (W.S_LOGITS,), steps, E))
    xs = bf16_dev(W.bf16_normal(seed, (W.S_X,), (steps, H)))
    ids = torch.empty((steps, k), dtype=torch.int32, device="cuda")
    w = torch.empty((steps, k), dtype=torch.float32, device="cuda")
    ref = torch.empty((steps, H), dtype=torch.bfloat16, device="cuda")
    for s in range(steps):
        gpu_lib.moe_layer_decode(desc, lg[s], xs[s:s + 1], k, ids[s], w[s], ref[s:s + 1], ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(ref)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for s in range(steps):
                gpu_lib.moe_layer_decode(desc, lg[s], xs[s:s + 1], k, ids[s], w[s], out[s:s + 1], ws)
    torch.cuda.current_stream().wait_stream(stream)
    scratch = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        gpu_lib.moe_layer_decode(desc, lg[rep], xs[rep:rep + 1], k, ids[rep], w[rep], scratch, ws)
        torch.cuda.synchronize()
        assert torch.equal(scratch, ref[rep:rep + 1]), rep


# ------------------------------------------------- batched decode on bf16 MFMA

def _batched_bf16_case(gpu_lib, T, E, k, with_shared, seed, H=512, I=256, bad_slots=0, sample=None):
    """bf16 tokens, all-FP4 ranks, weighted bf16 output: the grouped bf16 MFMA
    path (weights dequantised to bf16 in registers).  Invalid slot ids count
    as dropped ranks.  Compared per token against the oracle's expert MLPs."""
    torch = _torch()
    bank = W.fp4_bank(seed, 1, E, H, I)
    shared = W.fp4_record(seed, 2, 0, H, I) if with_shared else None
    layer = Layer(gpu_lib, bank, shared, H, I)
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    for _ in range(bad_slots):
        ids[rng.integers(T), rng.integers(k)] = rng.choice([-1, E, E + 5])
    w = rng.random((T, k)).astype(np.float32)
    xb = W.bf16_normal(seed, (3,), (T, H))
    x64 = O.bf16_bits_to_f64(xb)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    layer.forward(bf16_dev(xb), T, k, dev(ids), None, dev(w), out)
    torch.cuda.synchronize()
    got = to_f64(out)
    tokens = range(T) if sample is None else sample
    cache = {}

    def ew(key):
        if key not in cache:
            cache[key] = O.expert_weights(shared if key == -2 else bank[key], H, I)
        return cache[key]

    for t in tokens:
        ref = np.zeros(H)
        for r in range(k):
            e = int(ids[t, r])
            if 0 <= e < E:
                ref += w[t, r] * O.expert_mlp(x64[t], *ew(e))
        if with_shared:
            ref += O.expert_mlp(x64[t], *ew(-2))
        err = max_rel(got[t], ref)
        assert err <= TOL_BF16_MAX_REL, (t, err)
    log(f"batched bf16 MFMA T={T} E={E} k={k} shared={with_shared}: ok over {len(list(tokens))} tokens")


@pytest.mark.parametrize("I", [128, 256, 512])   # down K of 1, 2 and 4 stages: within, at and past the LDS ring
@pytest.mark.parametrize("T,E,k,with_shared,bad", [
    (2, 16, 4, True, 0),      # groups of one or two rows
    (37, 16, 4, True, 3),     # ragged groups, dropped ranks
    (70, 4, 3, True, 0),      # groups past 64 rows (two M tiles each), shared 70 rows
    (130, 2, 2, False, 0),    # no shared expert, three M tiles per group
])
def test_batched_bf16_mfma_path(gpu_lib, T, E, k, with_shared, bad, I):
    _batched_bf16_case(gpu_lib, T, E, k, with_shared, seed=300 + T, bad_slots=bad, I=I)


def test_layer_decode_b64_full_size(gpu_lib):
    """The batch-64 decode shape (256 experts + shared, H 4096, I 2048, top-6,
    Zipf-skewed routing) in the launch configuration the benchmark times;
    every token's output compared."""
    torch = _torch()
    cfg = W.WORKLOADS["decode-b64"]
    seed = W.WORKLOADS["decode-b64"]["seed"]
    E, H, I, k, T = cfg["E"], cfg["H"], cfg["I"], cfg["k"], cfg["T"]
    d = W.make_layer_inputs(cfg, seed, 0)
    bank, shared = d["bank"], d["shared_rec"]
    layer = Layer(gpu_lib, bank, shared, H, I)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    gpu_lib.moe_route(dev(d["logits"]), k, ids, w)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    layer.forward(bf16_dev(d["x"]), T, k, ids, None, w, out)
    torch.cuda.synchronize()
    oids, ow = O.route(d["logits"], k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    x64 = O.bf16_bits_to_f64(d["x"])
    got = to_f64(out)
    # every token; each distinct expert dequantised once, its (token, rank)
    # pairs evaluated together
    ys = np.zeros((T, k, H))
    for e in np.unique(oids):
        We = O.expert_weights(bank[int(e)], H, I)
        for t, r in zip(*np.nonzero(oids == e)):
            ys[t, r] = O.expert_mlp(x64[t], *We)
    Ws = O.expert_weights(shared, H, I)
    worst = 0.0
    for t in range(T):
        ref = O.combine(ys[t], ow[t], O.expert_mlp(x64[t], *Ws))
        err = max_rel(got[t], ref)
        worst = max(worst, err)
        assert err <= TOL_BF16_MAX_REL, (t, err)
    log(f"b64: {len(np.unique(oids))} distinct experts, worst token max-rel {worst:.3e} over {T} tokens")
