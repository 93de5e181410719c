"""GPU parity of batch-1 decode at the model shape (256 experts + shared,
H 4096, I 2048), on the decode workload's own bank of 256 distinct records,
through the C ABI.

Both batch-1 steps are covered: the two-launch step (the default) and the
single launch (MOE_LAYER_SINGLE_LAUNCH: routing, gate/up, down and combine in
one kernel, workgroups handing the SwiGLU outputs to each other through the
workspace).  Calls are queued back to back with no synchronisation between
them, as the benchmark runs them, so the per-call tags in the workspace
advance from call to call; every call's routing, weights and output are
checked against the oracle, and the workspace's error word must stay zero."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from mxfp4_routed_expert_renorm_amd import workloads as W
from tests.gpu_util import TOL_BF16_MAX_REL, bf16_dev, dev, log, max_rel, to_f64

pytestmark = pytest.mark.gpu

_STATE = {}


def _torch():
    import torch
    return torch


def _bank(gpu_lib):
    """The decode workload's resident layer on the GPU, built once per module."""
    if "bank" not in _STATE:
        cfg = W.WORKLOADS["decode-b1"]
        seed = cfg["seed"]
        d = W.make_layer_inputs(cfg, seed, 0)
        log(f"fused parity: uploading {d['bank'].shape[0]} distinct records + shared")
        _STATE["bank"] = d["bank"]
        _STATE["shared"] = d["shared_rec"]
        _STATE["bank_dev"] = dev(d["bank"])
        _STATE["shared_dev"] = dev(d["shared_rec"])
        _STATE["weights"] = {}
    return _STATE


def _expert(st, key):
    """Oracle weights of expert key (-1: the shared expert), dequantised once."""
    if key not in st["weights"]:
        rec = st["shared"] if key < 0 else st["bank"][key]
        st["weights"][key] = O.expert_weights(rec, 4096, 2048)
    return st["weights"][key]


def _desc(gpu_lib, st, flags, with_shared=True):
    b = st["bank_dev"]
    return gpu_lib.make_layer(4096, 2048, fp4_base=b, fp4_stride=b.shape[1], num_slots=b.shape[0],
                              shared=st["shared_dev"] if with_shared else None, flags=flags)


def _err_word(gpu_lib, ws, k, with_shared=True):
    off = gpu_lib.moe_expert_workspace_sync_offset(4096, 2048, 1, k, with_shared)
    return int(ws[off + 1024:off + 1028].cpu().numpy().view(np.uint32)[0])


def _decode_tokens(gpu_lib, flags, steps, k=8):
    torch = _torch()
    st = _bank(gpu_lib)
    cfg = W.WORKLOADS["decode-b1"]
    seed, E, H = cfg["seed"], cfg["E"], cfg["H"]
    desc = _desc(gpu_lib, st, flags)
    ws = gpu_lib.expert_workspace(H, 2048, 1, k, True)
    ins = [W.make_layer_inputs(cfg, seed, s, with_bank=False) for s in steps]
    lg = dev(np.concatenate([d["logits"] for d in ins]))
    xs = bf16_dev(np.concatenate([d["x"] for d in ins]))
    n = len(steps)
    ids = torch.full((n, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((n, k), -7.0, dtype=torch.float32, device="cuda")
    out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
    log(f"decode {n} tokens back to back, flags {flags}, k {k}")
    for i in range(n):
        gpu_lib.moe_layer_decode(desc, lg[i], xs[i:i + 1], k, ids[i], w[i], out[i:i + 1], ws)
    torch.cuda.synchronize()
    assert _err_word(gpu_lib, ws, k) == 0
    got_ids, got_w, got = ids.cpu().numpy(), w.cpu().numpy(), to_f64(out)
    for i, d in enumerate(ins):
        oids, ow = O.route(d["logits"], k)
        assert np.array_equal(got_ids[i], oids[0]), i
        assert np.max(np.abs(got_w[i] - ow[0])) <= 1e-6, i
        x64 = O.bf16_bits_to_f64(d["x"])[0]
        ys = np.stack([O.expert_mlp(x64, *_expert(st, int(e))) for e in oids[0]])
        ref = O.combine(ys, ow[0], O.expert_mlp(x64, *_expert(st, -1)))
        err = max_rel(got[i], ref)
        log(f"  token {steps[i]}: max-rel {err:.3e}")
        assert err <= TOL_BF16_MAX_REL, (i, err)
    return out


def test_two_launch_decode_full_shape(gpu_lib):
    """moe_layer_decode on the benchmark's own bank (the benchmark's launch
    configuration): five tokens queued back to back."""
    _decode_tokens(gpu_lib, 0, steps=(0, 1, 2, 3, 4))


def test_single_launch_decode_full_shape(gpu_lib):
    """The same tokens, one launch per token."""
    _decode_tokens(gpu_lib, gpu_lib.MOE_LAYER_SINGLE_LAUNCH, steps=(0, 1, 2, 3, 4))


def test_single_launch_top6(gpu_lib):
    """k = 6 (seven groups: the 7-group batch of the single launch)."""
    _decode_tokens(gpu_lib, gpu_lib.MOE_LAYER_SINGLE_LAUNCH, steps=(5, 6), k=6)


@pytest.mark.parametrize("k", [3, 1])
def test_single_launch_small_k(gpu_lib, k):
    """k = 3 and k = 1 (four and two groups: the 4-group batch of the single
    launch, most of its slots repeating the last group)."""
    _decode_tokens(gpu_lib, gpu_lib.MOE_LAYER_SINGLE_LAUNCH, steps=(7, 8), k=k)


@pytest.mark.parametrize("with_shared", [True, False])
def test_single_launch_given_ids_with_drops(gpu_lib, with_shared):
    """moe_expert_forward at T = 1 from given slot ids and weights: invalid
    slot ids are dropped ranks (their weight is ignored), with and without
    the shared expert."""
    torch = _torch()
    st = _bank(gpu_lib)
    H, I, k = 4096, 2048, 8
    desc = _desc(gpu_lib, st, gpu_lib.MOE_LAYER_SINGLE_LAUNCH, with_shared)
    ws = gpu_lib.expert_workspace(H, I, 1, k, with_shared)
    cases = [
        np.array([17, 3, 250, -1, 96, 256, 5, 201], np.int32),
        np.array([-1, -1, -1, -1, -1, -1, -1, 9], np.int32),
        np.array([255, 0, 128, 64, 32, 16, 8, 4], np.int32),
    ]
    xs = W.bf16_normal(7, (41,), (len(cases), H))
    wts = np.random.default_rng(41).random((len(cases), k)).astype(np.float32)
    outs = torch.empty((len(cases), H), dtype=torch.bfloat16, device="cuda")
    for i, ids in enumerate(cases):
        gpu_lib.moe_expert_forward(desc, bf16_dev(xs[i:i + 1]), 1, k, dev(ids[None]), None, dev(wts[i:i + 1]),
                                   outs[i:i + 1], ws)
    torch.cuda.synchronize()
    assert _err_word(gpu_lib, ws, k, with_shared) == 0
    got = to_f64(outs)
    for i, ids in enumerate(cases):
        x64 = O.bf16_bits_to_f64(xs[i:i + 1])[0]
        ref = np.zeros(H)
        for r in range(k):
            if 0 <= ids[r] < 256:
                ref += float(wts[i, r]) * O.expert_mlp(x64, *_expert(st, int(ids[r])))
        if with_shared:
            ref += O.expert_mlp(x64, *_expert(st, -1))
        err = max_rel(got[i], ref)
        log(f"given ids case {i} shared={with_shared}: max-rel {err:.3e}")
        assert err <= TOL_BF16_MAX_REL, (i, err)


def _x_wide_range():
    """bf16 activations with unusual 32-element blocks: an all-zero block (+0
    and -0), a block whose elements sit 2^-30 below its largest, a block of
    bf16 subnormals, blocks alternating 2^6 and 2^-8 magnitudes, a block near
    the bottom of the normal range, and ordinary N(0,1) blocks elsewhere."""
    x = W.bf16_normal(7, (43,), (1, 4096)).copy()
    rng = np.random.default_rng(43)
    sign = lambda n: np.where(rng.random(n) < 0.5, 0x8000, 0).astype(np.uint16)
    f32_to_bf16 = lambda v: (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x[0, 0:32] = sign(32)                                                   # zeros of both signs
    x[0, 32:64] = f32_to_bf16(rng.standard_normal(32) * 2.0 ** -20)         # tiny against
    x[0, 32] = f32_to_bf16(1024.0)                                          # one large element
    x[0, 64:96] = (rng.integers(1, 0x80, 32).astype(np.uint16) | sign(32))  # subnormal bf16
    alt = np.where(np.arange(64) % 2 == 0, 2.0 ** 6, 2.0 ** -8) * (1.0 + rng.random(64))
    x[0, 96:160] = f32_to_bf16(alt) | sign(64)
    x[0, 4064:4096] = f32_to_bf16(rng.standard_normal(32) * 2.0 ** -126)    # block maximum subnormal or near
    return x


def test_single_launch_x_edge_blocks(gpu_lib):
    """The single launch on activations with zero, subnormal and wide-range
    blocks: within tolerance of the oracle, with no non-finite output."""
    torch = _torch()
    st = _bank(gpu_lib)
    H, I, k = 4096, 2048, 8
    desc = _desc(gpu_lib, st, gpu_lib.MOE_LAYER_SINGLE_LAUNCH)
    ws = gpu_lib.expert_workspace(H, I, 1, k, True)
    ids = np.array([17, 3, 250, 44, 96, 131, 5, 201], np.int32)
    wts = np.random.default_rng(44).random((1, k)).astype(np.float32)
    x = _x_wide_range()
    out = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    log("single launch, edge-case activation blocks")
    gpu_lib.moe_expert_forward(desc, bf16_dev(x), 1, k, dev(ids[None]), None, dev(wts), out, ws)
    torch.cuda.synchronize()
    assert _err_word(gpu_lib, ws, k) == 0
    got = to_f64(out)[0]
    assert np.all(np.isfinite(got))
    x64 = O.bf16_bits_to_f64(x)[0]
    ref = O.expert_mlp(x64, *_expert(st, -1))
    for r in range(k):
        ref = ref + float(wts[0, r]) * O.expert_mlp(x64, *_expert(st, int(ids[r])))
    err = max_rel(got, ref)
    log(f"  edge blocks: max-rel {err:.3e}")
    assert err <= TOL_BF16_MAX_REL, err


def test_single_launch_graph_replays(gpu_lib):
    """The single launch captured in a HIP graph (four tokens) and replayed
    three times, with eager calls on the same workspace between the replays:
    every replay equals the eager result bit for bit."""
    torch = _torch()
    st = _bank(gpu_lib)
    cfg = W.WORKLOADS["decode-b1"]
    seed, H, k, steps = cfg["seed"], 4096, 8, 4
    desc = _desc(gpu_lib, st, gpu_lib.MOE_LAYER_SINGLE_LAUNCH)
    ws = gpu_lib.expert_workspace(H, 2048, 1, k, True)
    ins = [W.make_layer_inputs(cfg, seed, 20 + s, with_bank=False) for s in range(steps)]
    lg = dev(np.concatenate([d["logits"] for d in ins]))
    xs = bf16_dev(np.concatenate([d["x"] for d in ins]))
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
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        gpu_lib.moe_layer_decode(desc, lg[rep], xs[rep:rep + 1], k, ids[rep], w[rep], scratch, ws)
        torch.cuda.synchronize()
        assert torch.equal(scratch, ref[rep:rep + 1]), rep
    assert _err_word(gpu_lib, ws, k) == 0


@pytest.mark.parametrize("single", [True, False])
def test_decode_wide_routing(gpu_lib, single):
    """E = 1000 logits: both batch-1 forms route with 16 logits per lane (the
    other instantiation of their in-kernel top-k).  The bank's 256 records
    are repeated over 1000 slots on the device (13.4 GB), so expert e runs
    record e mod 256; ids and weights are bit-exact against the oracle's
    routing over all 1000 logits, outputs within tolerance."""
    torch = _torch()
    st = _bank(gpu_lib)
    cfg = W.WORKLOADS["decode-b1"]
    H, I, k, E = 4096, 2048, 8, 1000
    base = st["bank_dev"]
    log(f"wide routing ({'single launch' if single else 'two launches'}): {E} slots of {base.shape[0]} records")
    big = base.repeat(-(-E // base.shape[0]), 1)[:E].contiguous()
    desc = gpu_lib.make_layer(H, I, fp4_base=big, fp4_stride=big.shape[1], num_slots=E, shared=st["shared_dev"],
                              flags=gpu_lib.MOE_LAYER_SINGLE_LAUNCH if single else 0)
    ws = gpu_lib.expert_workspace(H, I, 1, k, True)
    n = 3
    lg = W.router_logits(cfg["seed"], (47,), n, E)
    xs = W.bf16_normal(cfg["seed"], (48,), (n, H))
    ids = torch.empty((n, k), dtype=torch.int32, device="cuda")
    w = torch.empty((n, k), dtype=torch.float32, device="cuda")
    out = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
    lgd = dev(lg)
    for i in range(n):
        gpu_lib.moe_layer_decode(desc, lgd[i], bf16_dev(xs[i:i + 1]), k, ids[i], w[i], out[i:i + 1], ws)
    torch.cuda.synchronize()
    if single:
        assert _err_word(gpu_lib, ws, k) == 0
    got_ids, got_w, got = ids.cpu().numpy(), w.cpu().numpy(), to_f64(out)
    del big, desc
    torch.cuda.empty_cache()
    for i in range(n):
        oids, ow = O.route(lg[i:i + 1], k)
        assert np.array_equal(got_ids[i], oids[0]), i
        assert np.max(np.abs(got_w[i] - ow[0])) <= 1e-6, i
        assert np.any(oids[0] >= 256), "the routing reaches past the first 256 experts"
        x64 = O.bf16_bits_to_f64(xs[i:i + 1])[0]
        ys = np.stack([O.expert_mlp(x64, *_expert(st, int(e) % 256)) for e in oids[0]])
        ref = O.combine(ys, ow[0], O.expert_mlp(x64, *_expert(st, -1)))
        err = max_rel(got[i], ref)
        log(f"  token {i}: ids {oids[0].tolist()}, max-rel {err:.3e}")
        assert err <= TOL_BF16_MAX_REL, (i, err)
