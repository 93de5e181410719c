"""One GPU's share of G-way tensor parallelism ("Running DeepSeek-V4-Flash across
four free GPUs", §Step 2): the sliced records dequantise to the oracle's row and
column bands of the full matrices, bit for bit, and the G shares' partial layer
outputs sum to the full layer's output."""
import numpy as np
import pytest

from mxfp4_routed_expert_renorm_amd import workloads as W
from oracle import moe_oracle as O
from tests.gpu_util import TOL_F32_REL_L2, dev, log, rel_l2

pytestmark = pytest.mark.gpu


def _share_bank(gpu_lib, bank_d, H, I, G, g):
    import torch
    rb = O.fp4_expert_nbytes(H, I // G)
    out = torch.empty((bank_d.shape[0], rb), dtype=torch.uint8, device="cuda")
    gpu_lib.moe_tp_slice(bank_d, H, I, G, g, out)
    return out


@pytest.mark.parametrize("G", [2, 4])
def test_tp_slices_are_the_bands_of_the_full_matrices(gpu_lib, G):
    import torch
    H, I, E = 512, 256, 3
    bank = W.fp4_bank(61, 1, E, H, I)
    bank_d = dev(bank)
    Is = I // G
    for g in range(G):
        sl = _share_bank(gpu_lib, bank_d, H, I, G, g)
        torch.cuda.synchronize()
        got = sl.cpu().numpy()
        for e in range(E):
            W1, W3, W2 = O.expert_weights(bank[e], H, I)
            S1, S3, S2 = O.expert_weights(got[e], H, Is)
            assert np.array_equal(S1, W1[g * Is:(g + 1) * Is])
            assert np.array_equal(S3, W3[g * Is:(g + 1) * Is])
            assert np.array_equal(S2, W2[:, g * Is:(g + 1) * Is])


@pytest.mark.parametrize("T,G", [(1, 2), (5, 4), (3, 8)])
def test_tp_partial_outputs_sum_to_the_layer(gpu_lib, T, G):
    """fp32 activations and outputs: each share's expert MLP + combine is a
    partial sum of the layer output; the G partials add up to it."""
    import torch
    H, I, E, k = 512, 128 * G, 8, 3   # each share keeps I/G = 128
    bank = W.fp4_bank(62 + G, 1, E, H, I)
    shared = W.fp4_record(62 + G, 2, 0, H, I)
    rng = np.random.default_rng(G * 10 + T)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    x = W.f32_normal(63, (3,), (T, H))
    bank_d, shared_d = dev(bank), dev(shared[None, :])

    def forward(bk, sh, Ic):
        layer = gpu_lib.make_layer(H, Ic, fp4_base=bk, fp4_stride=bk.shape[1], num_slots=E, shared=sh[0])
        out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ws = gpu_lib.expert_workspace(H, Ic, T, k, True)
        gpu_lib.moe_expert_forward(layer, dev(x), T, k, dev(ids), None, dev(w), out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)

    full = forward(bank_d, shared_d, I)
    parts = sum(forward(_share_bank(gpu_lib, bank_d, H, I, G, g), _share_bank(gpu_lib, shared_d, H, I, G, g), I // G)
                for g in range(G))
    err = rel_l2(parts, full)
    log(f"TP G={G} T={T}: rel-L2 of the summed shares vs the full layer {err:.2e}")
    assert err <= 1e-5
    # and the full layer against the oracle
    ref = np.stack([O.layer_forward(x[t].astype(np.float64)[None, :], ids[t:t + 1], w[t:t + 1],
                                    lambda e: bank[int(e)], H, I, shared_rec=shared)[0] for t in range(T)])
    assert rel_l2(full, ref) <= TOL_F32_REL_L2


# ---------------------------------------------------------------- model width
# One GPU's share at the decode workload's width (H 4096, I 2048 split G ways:
# 256, 512 or 1024 rows per share), run by the batch-1 step the benchmark
# times: routing inside the gate/up launch, then down + combine.

_WIDE = {}


def _wide_bank():
    """24 experts + shared at H 4096, I 2048 (host records and their oracle
    weights, dequantised once)."""
    if not _WIDE:
        H, I, E = 4096, 2048, 24
        _WIDE["bank"] = W.fp4_bank(71, 1, E, H, I)
        _WIDE["shared"] = W.fp4_record(71, 2, 0, H, I)
        _WIDE["w"] = {}
    return _WIDE


def _wide_weights(key):
    st = _wide_bank()
    if key not in st["w"]:
        rec = st["shared"] if key < 0 else st["bank"][key]
        st["w"][key] = O.expert_weights(rec, 4096, 2048)
    return st["w"][key]


def _share_ref(x64, ids, w, G, g, with_shared=True):
    """The oracle's partial layer output of share g: every selected expert's
    SwiGLU over rows [g I/G, (g+1) I/G) of w1 and w3 and the same columns of
    w2, combined with the routing weights (dropped ranks: id outside the bank)."""
    Is = 2048 // G
    band = slice(g * Is, (g + 1) * Is)

    def mlp(key):
        W1, W3, W2 = _wide_weights(key)
        return O.expert_mlp(x64, W1[band], W3[band], W2[:, band])

    ys = np.stack([mlp(int(e)) if 0 <= e < 24 else np.zeros(4096) for e in ids])
    return O.combine(ys, np.where((ids >= 0) & (ids < 24), w, 0.0), mlp(-1) if with_shared else None)


@pytest.mark.parametrize("G,g", [(8, 0), (8, 7), (4, 2), (2, 1)])
def test_tp_share_decode_at_model_width(gpu_lib, G, g):
    """moe_layer_decode on share g of G: ids and weights equal the oracle's
    routing, the output the oracle's partial sum over the share's bands."""
    import torch
    from tests.gpu_util import TOL_BF16_MAX_REL, bf16_dev, max_rel, to_f64
    st = _wide_bank()
    H, I, E, k = 4096, 2048, 24, 8
    bank_d, shared_d = dev(st["bank"]), dev(st["shared"][None, :])
    sb, ss = _share_bank(gpu_lib, bank_d, H, I, G, g), _share_bank(gpu_lib, shared_d, H, I, G, g)
    Is = I // G
    layer = gpu_lib.make_layer(H, Is, fp4_base=sb, fp4_stride=sb.shape[1], num_slots=E, shared=ss[0])
    ws = gpu_lib.expert_workspace(H, Is, 1, k, True)
    ntok = 3
    xs = W.bf16_normal(72, (G, g), (ntok, H))
    lg = W.router_logits(72, (G, g, 1), ntok, E)
    lg_d, x_d = dev(lg), bf16_dev(xs)
    ids = torch.full((ntok, k), -3, dtype=torch.int32, device="cuda")
    w = torch.full((ntok, k), -3.0, dtype=torch.float32, device="cuda")
    out = torch.empty((ntok, H), dtype=torch.bfloat16, device="cuda")
    log(f"TP share {g}/{G} (I = {Is}) at H 4096: {ntok} tokens back to back")
    for t in range(ntok):
        gpu_lib.moe_layer_decode(layer, lg_d[t], x_d[t:t + 1], k, ids[t], w[t], out[t:t + 1], ws)
    torch.cuda.synchronize()
    oids, ow = O.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.max(np.abs(w.cpu().numpy() - ow)) <= 1e-6
    got = to_f64(out)
    for t in range(ntok):
        ref = _share_ref(O.bf16_bits_to_f64(xs[t:t + 1])[0], oids[t], ow[t], G, g)
        err = max_rel(got[t], ref)
        log(f"  token {t}: max-rel {err:.3e}")
        assert err <= TOL_BF16_MAX_REL, (t, err)


@pytest.mark.parametrize("with_shared", [True, False])
def test_tp_share_given_ids_and_the_shares_sum_to_the_layer(gpu_lib, with_shared):
    """moe_expert_forward at T = 1 on every share of an 8-way split, from given
    ids with dropped ranks: each share matches the oracle's partial output,
    and the eight partials add up to the oracle's full layer."""
    import torch
    from tests.gpu_util import TOL_BF16_MAX_REL, bf16_dev, max_rel, to_f64
    st = _wide_bank()
    H, I, E, k, G = 4096, 2048, 24, 8, 8
    bank_d, shared_d = dev(st["bank"]), dev(st["shared"][None, :])
    ids = np.array([[5, 23, -1, 0, 17, 24, 9, 2]], np.int32)
    wts = np.random.default_rng(73).random((1, k)).astype(np.float32)
    xs = W.bf16_normal(73, (1,), (1, H))
    x64 = O.bf16_bits_to_f64(xs)[0]
    total = np.zeros(H)
    for g in range(G):
        sb, ss = _share_bank(gpu_lib, bank_d, H, I, G, g), _share_bank(gpu_lib, shared_d, H, I, G, g)
        layer = gpu_lib.make_layer(H, I // G, fp4_base=sb, fp4_stride=sb.shape[1], num_slots=E,
                                   shared=ss[0] if with_shared else None)
        ws = gpu_lib.expert_workspace(H, I // G, 1, k, with_shared)
        out = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
        gpu_lib.moe_expert_forward(layer, bf16_dev(xs), 1, k, dev(ids), None, dev(wts), out, ws)
        torch.cuda.synchronize()
        got = to_f64(out)[0]
        ref = _share_ref(x64, ids[0], wts[0].astype(np.float64), G, g, with_shared)
        err = max_rel(got, ref)
        log(f"share {g}/8 shared={with_shared}: max-rel {err:.3e}")
        assert err <= TOL_BF16_MAX_REL, (g, err)
        total += got
    full = O.combine(np.stack([O.expert_mlp(x64, *_wide_weights(int(e))) if 0 <= e < 24 else np.zeros(H)
                               for e in ids[0]]),
                     np.where((ids[0] >= 0) & (ids[0] < 24), wts[0].astype(np.float64), 0.0),
                     O.expert_mlp(x64, *_wide_weights(-1)) if with_shared else None)
    err = max_rel(total, full)
    log(f"sum of the 8 shares vs the full layer: max-rel {err:.3e}")
    assert err <= TOL_BF16_MAX_REL


# ------------------------------------------------ single launch of a 1/8 share
# MOE_LAYER_SINGLE_LAUNCH at H 4096, I 256: routing, gate/up, SwiGLU, down and
# combine in one launch, the units handing their SwiGLU outputs to each other
# through the workspace.  Calls go back to back, so the per-call tags advance.

def _err_word(gpu_lib, ws, Is, k, with_shared):
    off = gpu_lib.moe_expert_workspace_sync_offset(4096, Is, 1, k, with_shared)
    return int(ws[off + 1024:off + 1028].cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("g,k", [(0, 8), (5, 8), (3, 6), (7, 3), (2, 1)])
def test_tp_share_single_launch_decode(gpu_lib, g, k):
    """moe_layer_decode on share g of 8 in one launch, k ranks plus the shared
    expert (9, 7, 4 and 2 groups: each batch size of the kernel): routing equal to
    the oracle's, outputs the oracle's partial sums, error word zero."""
    import torch
    from tests.gpu_util import TOL_BF16_MAX_REL, bf16_dev, max_rel, to_f64
    st = _wide_bank()
    H, I, E, G = 4096, 2048, 24, 8
    bank_d, shared_d = dev(st["bank"]), dev(st["shared"][None, :])
    sb, ss = _share_bank(gpu_lib, bank_d, H, I, G, g), _share_bank(gpu_lib, shared_d, H, I, G, g)
    layer = gpu_lib.make_layer(H, I // G, fp4_base=sb, fp4_stride=sb.shape[1], num_slots=E, shared=ss[0],
                               flags=gpu_lib.MOE_LAYER_SINGLE_LAUNCH)
    ws = gpu_lib.expert_workspace(H, I // G, 1, k, True)
    ntok = 4
    xs = W.bf16_normal(74, (g, k), (ntok, H))
    lg = W.router_logits(74, (g, k, 1), ntok, E)
    lg_d, x_d = dev(lg), bf16_dev(xs)
    ids = torch.full((ntok, k), -3, dtype=torch.int32, device="cuda")
    w = torch.full((ntok, k), -3.0, dtype=torch.float32, device="cuda")
    out = torch.empty((ntok, H), dtype=torch.bfloat16, device="cuda")
    log(f"single-launch TP share {g}/8, k {k}: {ntok} tokens back to back")
    for t in range(ntok):
        gpu_lib.moe_layer_decode(layer, lg_d[t], x_d[t:t + 1], k, ids[t], w[t], out[t:t + 1], ws)
    torch.cuda.synchronize()
    assert _err_word(gpu_lib, ws, I // G, k, True) == 0
    oids, ow = O.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.max(np.abs(w.cpu().numpy() - ow)) <= 1e-6
    got = to_f64(out)
    for t in range(ntok):
        ref = _share_ref(O.bf16_bits_to_f64(xs[t:t + 1])[0], oids[t], ow[t], G, g)
        err = max_rel(got[t], ref)
        log(f"  token {t}: max-rel {err:.3e}")
        assert err <= TOL_BF16_MAX_REL, (t, err)


@pytest.mark.parametrize("with_shared", [True, False])
def test_tp_share_single_launch_given_ids_with_drops(gpu_lib, with_shared):
    """moe_expert_forward at T = 1 in one launch on every share of an 8-way
    split, from given ids with dropped ranks (without the shared expert the
    eight ranks fill the 9-group batch but one): each share matches the
    oracle's partial output and the two-launch step's output within the
    tolerance, and the eight partials add up to the full layer."""
    import torch
    from tests.gpu_util import TOL_BF16_MAX_REL, bf16_dev, max_rel, to_f64
    st = _wide_bank()
    H, I, E, k, G = 4096, 2048, 24, 8, 8
    bank_d, shared_d = dev(st["bank"]), dev(st["shared"][None, :])
    cases = [np.array([[5, 23, -1, 0, 17, 24, 9, 2]], np.int32),
             np.array([[-1, -1, -1, -1, -1, -1, -1, -1]], np.int32),
             np.array([[-1, 30, -1, 11, -1, -1, -1, -1]], np.int32)]
    wts = np.random.default_rng(75).random((len(cases), k)).astype(np.float32)
    xs = W.bf16_normal(75, (1,), (len(cases), H))
    total = np.zeros((len(cases), H))
    for g in range(G):
        sb, ss = _share_bank(gpu_lib, bank_d, H, I, G, g), _share_bank(gpu_lib, shared_d, H, I, G, g)
        outs = {}
        for flags in (gpu_lib.MOE_LAYER_SINGLE_LAUNCH, 0):
            layer = gpu_lib.make_layer(H, I // G, fp4_base=sb, fp4_stride=sb.shape[1], num_slots=E,
                                       shared=ss[0] if with_shared else None, flags=flags)
            ws = gpu_lib.expert_workspace(H, I // G, 1, k, with_shared)
            out = torch.empty((len(cases), H), dtype=torch.bfloat16, device="cuda")
            for i, ids in enumerate(cases):
                gpu_lib.moe_expert_forward(layer, bf16_dev(xs[i:i + 1]), 1, k, dev(ids), None, dev(wts[i:i + 1]),
                                           out[i:i + 1], ws)
            torch.cuda.synchronize()
            if flags:
                assert _err_word(gpu_lib, ws, I // G, k, with_shared) == 0
            outs[flags] = to_f64(out)
        got = outs[gpu_lib.MOE_LAYER_SINGLE_LAUNCH]
        for i, ids in enumerate(cases):
            x64 = O.bf16_bits_to_f64(xs[i:i + 1])[0]
            ref = _share_ref(x64, ids[0], wts[i].astype(np.float64), G, g, with_shared)
            if not with_shared and np.all(ids < 0):
                assert np.all(got[i] == 0.0), (g, i)   # nothing to combine: exact zeros
                continue
            err = max_rel(got[i], ref)
            log(f"share {g}/8 case {i} shared={with_shared}: max-rel {err:.3e}")
            assert err <= TOL_BF16_MAX_REL, (g, i, err)
            assert max_rel(got[i], outs[0][i]) <= 2 * TOL_BF16_MAX_REL, (g, i)
        total += got
    for i, ids in enumerate(cases):
        if not with_shared and np.all(ids < 0):
            continue
        x64 = O.bf16_bits_to_f64(xs[i:i + 1])[0]
        full = O.combine(np.stack([O.expert_mlp(x64, *_wide_weights(int(e))) if 0 <= e < 24 else np.zeros(H)
                                   for e in ids[0]]),
                         np.where((ids[0] >= 0) & (ids[0] < 24), wts[i].astype(np.float64), 0.0),
                         O.expert_mlp(x64, *_wide_weights(-1)) if with_shared else None)
        assert max_rel(total[i], full) <= TOL_BF16_MAX_REL, i


def test_tp_share_single_launch_wide_router(gpu_lib):
    """300 experts (more than 256 logits: sixteen per lane in the kernel's
    routing), top-8 + shared, on a bank made at the share's own width: routing
    and outputs equal to the oracle's."""
    import torch
    from tests.gpu_util import TOL_BF16_MAX_REL, bf16_dev, max_rel, to_f64
    H, Is, E, k = 4096, 256, 300, 8
    bank = W.fp4_bank(76, 1, E, H, Is)
    shared = W.fp4_record(76, 2, 0, H, Is)
    bank_d, shared_d = dev(bank), dev(shared[None, :])
    layer = gpu_lib.make_layer(H, Is, fp4_base=bank_d, fp4_stride=bank.shape[1], num_slots=E, shared=shared_d[0],
                               flags=gpu_lib.MOE_LAYER_SINGLE_LAUNCH)
    ws = gpu_lib.expert_workspace(H, Is, 1, k, True)
    ntok = 3
    xs = W.bf16_normal(76, (3,), (ntok, H))
    lg = W.router_logits(76, (4,), ntok, E)
    lg_d, x_d = dev(lg), bf16_dev(xs)
    ids = torch.full((ntok, k), -3, dtype=torch.int32, device="cuda")
    w = torch.full((ntok, k), -3.0, dtype=torch.float32, device="cuda")
    out = torch.empty((ntok, H), dtype=torch.bfloat16, device="cuda")
    for t in range(ntok):
        gpu_lib.moe_layer_decode(layer, lg_d[t], x_d[t:t + 1], k, ids[t], w[t], out[t:t + 1], ws)
    torch.cuda.synchronize()
    assert _err_word(gpu_lib, ws, Is, k, True) == 0
    oids, ow = O.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.max(np.abs(w.cpu().numpy() - ow)) <= 1e-6
    got = to_f64(out)
    for t in range(ntok):
        x64 = O.bf16_bits_to_f64(xs[t:t + 1])[0]
        ys = np.stack([O.expert_mlp(x64, *O.expert_weights(bank[int(e)], H, Is)) for e in oids[t]])
        ref = O.combine(ys, ow[t], O.expert_mlp(x64, *O.expert_weights(shared, H, Is)))
        err = max_rel(got[t], ref)
        log(f"  token {t}: max-rel {err:.3e}")
        assert err <= TOL_BF16_MAX_REL, (t, err)


def test_tp_share_single_launch_graph_replays(gpu_lib):
    """Four single-launch calls of share 2/8 captured in a HIP graph and
    replayed three times with eager calls on the same workspace between the
    replays: every replay equals the eager result bit for bit."""
    import torch
    from tests.gpu_util import bf16_dev
    st = _wide_bank()
    H, I, E, k, G, g = 4096, 2048, 24, 8, 8, 2
    bank_d, shared_d = dev(st["bank"]), dev(st["shared"][None, :])
    sb, ss = _share_bank(gpu_lib, bank_d, H, I, G, g), _share_bank(gpu_lib, shared_d, H, I, G, g)
    layer = gpu_lib.make_layer(H, I // G, fp4_base=sb, fp4_stride=sb.shape[1], num_slots=E, shared=ss[0],
                               flags=gpu_lib.MOE_LAYER_SINGLE_LAUNCH)
    ws = gpu_lib.expert_workspace(H, I // G, 1, k, True)
    steps = 4
    lg_d = dev(W.router_logits(77, (1,), steps, E))
    x_d = bf16_dev(W.bf16_normal(77, (2,), (steps, H)))
    ids = torch.empty((steps, k), dtype=torch.int32, device="cuda")
    w = torch.empty((steps, k), dtype=torch.float32, device="cuda")
    ref = torch.empty((steps, H), dtype=torch.bfloat16, device="cuda")
    for s in range(steps):
        gpu_lib.moe_layer_decode(layer, lg_d[s], x_d[s:s + 1], k, ids[s], w[s], ref[s:s + 1], ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(ref)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(gr, stream=stream):
            for s in range(steps):
                gpu_lib.moe_layer_decode(layer, lg_d[s], x_d[s:s + 1], k, ids[s], w[s], out[s:s + 1], ws)
    torch.cuda.current_stream().wait_stream(stream)
    scratch = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    for rep in range(3):
        out.zero_()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        gpu_lib.moe_layer_decode(layer, lg_d[rep], x_d[rep:rep + 1], k, ids[rep], w[rep], scratch, ws)
        torch.cuda.synchronize()
        assert torch.equal(scratch, ref[rep:rep + 1]), rep
    assert _err_word(gpu_lib, ws, I // G, k, True) == 0
