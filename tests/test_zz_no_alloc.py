"""GPU check of moe_layer_decode_noalloc (batch-1 decode with the library's
static per-device scratch as its workspace) against moe_layer_decode with a
caller's workspace, through the C ABI.

Both entry points run the same kernels in the same order, so the routing ids,
weights and outputs must agree bit for bit.  Calls follow each other with no
synchronisation, as a serving loop makes them: a call at the model shape
(H 4096, I 2048, top-8 + shared), one on a 1/8 tensor-parallel share
(I 256), a smaller one (H 2048, I 1024, top-4, no shared expert) that
rewrites the scratch, the share again, then the model shape again; once with
the two-launch steps and once with the single launches (both the full-width
and the share's kernel), whose tags and arrival counters the scratch keeps
from call to call and from one kernel to the other."""
import numpy as np
import pytest

from mxfp4_routed_expert_renorm_amd import workloads as W
from tests.gpu_util import bf16_dev, dev, log

pytestmark = pytest.mark.gpu

SEED = 4242


def _case(H, I, E, k, shared, key):
    bank = W.fp4_bank(SEED, key, E, H, I)
    sh = W.fp4_record(SEED, key + 1, 0, H, I) if shared else None
    x = W.bf16_normal(SEED, (key, 2), (1, H))
    lg = W.router_logits(SEED, (key, 3), 1, E)
    return dict(H=H, I=I, E=E, k=k, bank=dev(bank), shared=dev(sh) if shared else None, x=bf16_dev(x),
                lg=dev(lg[0]))


def _run(gpu_lib, c, flags, noalloc):
    import torch
    lay = gpu_lib.make_layer(c["H"], c["I"], fp4_base=c["bank"], fp4_stride=c["bank"].shape[1], num_slots=c["E"],
                             shared=c["shared"], flags=flags)
    ids = torch.full((c["k"],), -5, dtype=torch.int32, device="cuda")
    w = torch.full((c["k"],), -5.0, dtype=torch.float32, device="cuda")
    out = torch.full((1, c["H"]), 7.0, dtype=torch.bfloat16, device="cuda")
    if noalloc:
        gpu_lib.moe_layer_decode_noalloc(lay, c["lg"], c["x"], c["k"], ids, w, out)
    else:
        ws = gpu_lib.expert_workspace(c["H"], c["I"], 1, c["k"], c["shared"] is not None)
        gpu_lib.moe_layer_decode(lay, c["lg"], c["x"], c["k"], ids, w, out, ws)
    return ids, w, out, lay


@pytest.mark.parametrize("flags", [0, 1])
def test_noalloc_matches_layer_decode_big_small_big(gpu_lib, flags):
    import torch
    big = _case(4096, 2048, 24, 8, True, 10)
    share = _case(4096, 256, 24, 8, True, 30)
    small = _case(2048, 1024, 16, 4, False, 20)
    seq = [("big", big), ("share", share), ("small", small), ("share", share), ("big", big)]
    got = []
    for name, c in seq:
        log(f"noalloc: {name} H {c['H']} I {c['I']} E {c['E']} k {c['k']} flags {flags}")
        got.append(_run(gpu_lib, c, flags, noalloc=True))
    ref = [_run(gpu_lib, c, flags, noalloc=False) for _, c in seq]
    torch.cuda.synchronize()
    for i, ((gi, gw, go, _), (ri, rw, ro, _)) in enumerate(zip(got, ref)):
        assert torch.equal(gi, ri), i
        assert torch.equal(gw, rw), i
        assert torch.equal(go, ro), i
        assert bool(torch.isfinite(go.float()).all()), i


def test_noalloc_graph_replays(gpu_lib):
    """After one eager call on the device, calls of both shapes captured in a
    graph and replayed three times give the eager results each time."""
    import torch
    big = _case(4096, 2048, 24, 8, True, 30)
    small = _case(2048, 1024, 16, 4, False, 40)
    ref = [_run(gpu_lib, c, 1, noalloc=False) for c in (big, small)]
    torch.cuda.synchronize()
    lays = [gpu_lib.make_layer(c["H"], c["I"], fp4_base=c["bank"], fp4_stride=c["bank"].shape[1], num_slots=c["E"],
                               shared=c["shared"], flags=1) for c in (big, small)]
    outs = [(torch.empty((c["k"],), dtype=torch.int32, device="cuda"),
             torch.empty((c["k"],), dtype=torch.float32, device="cuda"),
             torch.empty((1, c["H"]), dtype=torch.bfloat16, device="cuda")) for c in (big, small)]
    for c, lay, (i_, w_, o_) in zip((big, small), lays, outs):  # eager first call (clears the scratch once)
        gpu_lib.moe_layer_decode_noalloc(lay, c["lg"], c["x"], c["k"], i_, w_, o_)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for c, lay, (i_, w_, o_) in zip((big, small), lays, outs):
                gpu_lib.moe_layer_decode_noalloc(lay, c["lg"], c["x"], c["k"], i_, w_, o_)
    torch.cuda.current_stream().wait_stream(stream)
    for rep in range(3):
        for _, _, o_ in outs:
            o_.zero_()
        g.replay()
        torch.cuda.synchronize()
        for (gi, gw, go), (ri, rw, ro, _) in zip(outs, ref):
            assert torch.equal(gi, ri) and torch.equal(gw, rw) and torch.equal(go, ro), rep
        log(f"noalloc graph replay {rep} ok")


def test_noalloc_rejects_layers_beyond_the_scratch(gpu_lib):
    """A layer whose decode workspace exceeds the static scratch is refused
    before anything is launched."""
    import torch
    H = I = 8192
    k = 64
    need = gpu_lib.moe_expert_workspace_sync_offset(H, I, 1, k, True)
    assert need > gpu_lib.moe_noalloc_scratch_bytes()
    rec = torch.zeros((1, 16), dtype=torch.uint8, device="cuda")
    lay = gpu_lib.make_layer(H, I, fp4_base=rec, fp4_stride=gpu_lib.moe_fp4_expert_bytes(H, I), num_slots=256,
                             shared=rec[0])
    lg = torch.zeros(256, device="cuda")
    x = torch.zeros((1, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty(k, dtype=torch.int32, device="cuda")
    w = torch.empty(k, dtype=torch.float32, device="cuda")
    out = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.MoeError, match="static scratch"):
        gpu_lib.moe_layer_decode_noalloc(lay, lg, x, k, ids, w, out)
