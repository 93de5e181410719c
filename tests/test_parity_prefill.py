"""GPU parity of the prefill path (MXFP8 activations x MXFP4 weights on scaled
MFMA) against the oracle, through the C ABI.  The activation quantisation is
compared bit for bit; the layer output to the bf16 tolerance."""
import numpy as np
import pytest

from mxfp4_routed_expert_renorm_amd import workloads as W
from oracle import moe_oracle as O
from tests.gpu_util import TOL_BF16_MAX_REL, bf16_dev, dev, log, max_rel, to_f64

pytestmark = pytest.mark.gpu


def _bf16_bits(vals):
    return W.bf16_bits_from_f32(np.asarray(vals, np.float32))


def _quant_gpu(gpu_lib, bits):
    import torch
    rows, K = bits.shape
    codes = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
    gpu_lib.moe_quant_mxfp8(bf16_dev(bits), codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_quant_mxfp8_bit_exact_random_and_edges(gpu_lib):
    rng = np.random.default_rng(12)
    rows = [W.bf16_normal(5, (1,), (64, 4096))]
    edge = np.zeros((8, 64), np.float32)
    edge[0, :32] = 0.0                                       # all-zero block
    edge[0, 32:] = -0.0
    edge[1, :32] = np.float32(448.0) * 2.0 ** np.arange(-40, -8)[:32].astype(np.float32)  # wide range, subnormal outputs
    edge[2, :32] = np.linspace(-7.75, 7.75, 32)              # saturation of the largest (7.75 -> 496 -> 448)
    edge[3, :32] = 1.0 + np.arange(32) / 16.0                # many exact ties after scaling
    edge[4, :32] = 3.0e38                                    # top of the exponent range
    edge[5, :32] = 1.0e-38                                   # bottom of the exponent range
    edge[6] = rng.standard_normal(64) * 1e-3
    edge[7, ::2] = 1.0
    rows.append(_bf16_bits(edge))
    for bits in rows:
        codes, scales = _quant_gpu(gpu_lib, bits)
        oc, os_ = O.quant_mxfp8(O.bf16_bits_to_f64(bits))
        assert np.array_equal(scales, os_)
        assert np.array_equal(codes, oc)


def _prefill_case(gpu_lib, E, H, I, k, T, seed, shared=True, sample=None):
    import torch
    bank = W.fp4_bank(seed, W.S_BANK, E, H, I)
    shrec = W.fp4_record(seed, W.S_SHARED, 0, H, I) if shared else None
    xb = W.bf16_normal(seed, (W.S_X,), (T, H))
    lg = W.router_logits(seed, (W.S_LOGITS,), T, E)
    d_bank = dev(bank)
    d_shared = dev(shrec) if shared else None
    layer = gpu_lib.make_layer(H, I, fp4_base=d_bank, fp4_stride=bank.shape[1], num_slots=E, shared=d_shared)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    gpu_lib.moe_route(dev(lg), k, ids, w)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gpu_lib.moe_prefill_workspace_bytes(H, I, T, k, shared), dtype=torch.uint8, device="cuda")
    gpu_lib.moe_prefill_forward(layer, bf16_dev(xb), k, ids, w, out, ws)
    torch.cuda.synchronize()
    oids, ow = O.route(lg, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    tokens = list(range(T)) if sample is None else sample
    ref = O.prefill_forward(O.bf16_bits_to_f64(xb), oids, ow, lambda e: bank[e], H, I, shared_rec=shrec,
                            tokens=tokens)
    got = to_f64(out)[tokens]
    err = max_rel(got, ref)
    log(f"prefill E={E} H={H} I={I} k={k} T={T} shared={shared}: max-rel {err:.3e} over {len(tokens)} tokens")
    assert err <= TOL_BF16_MAX_REL
    # and per token, so one bad row cannot hide behind large ones
    for j in range(len(tokens)):
        assert max_rel(got[j], ref[j]) <= 3 * TOL_BF16_MAX_REL, tokens[j]


def test_prefill_ragged_groups(gpu_lib):
    """300 tokens over 16 experts: groups of ~75 rows (partial 32-row blocks),
    the shared expert's 300 rows span two 256-row tiles; several K steps and
    output tiles."""
    _prefill_case(gpu_lib, E=16, H=512, I=256, k=4, T=300, seed=41)


def test_prefill_no_shared_small(gpu_lib):
    _prefill_case(gpu_lib, E=8, H=256, I=128, k=2, T=37, seed=42, shared=False)


def test_prefill_full_size_sampled(gpu_lib):
    """The prefill workload's shape: 4096 tokens, 256 experts + shared, H 4096,
    I 2048, top-8; outputs compared on 256 seeded tokens (each token's output
    depends only on its own routing; the oracle evaluates expert by expert)."""
    cfg = W.WORKLOADS["prefill"]
    rng = np.random.default_rng(43)
    sample = sorted(rng.choice(cfg["T"], 256, replace=False).tolist())
    _prefill_case(gpu_lib, E=cfg["E"], H=cfg["H"], I=cfg["I"], k=cfg["k"], T=cfg["T"], seed=W.WORKLOADS["prefill"]["seed"],
                  sample=sample)


@pytest.mark.parametrize("T", [1, 5])
def test_prefill_sparse_groups(gpu_lib, T):
    """Few tokens over 64 experts: most groups are empty and the rest hold a
    single row of a 32-row block."""
    _prefill_case(gpu_lib, E=64, H=512, I=256, k=3, T=T, seed=44 + T)


def test_prefill_T0_is_noop(gpu_lib):
    import torch
    H, I, E, k = 256, 128, 8, 2
    layer = gpu_lib.make_layer(H, I, fp4_base=torch.empty(E * O.fp4_expert_nbytes(H, I), dtype=torch.uint8,
                                                           device="cuda"),
                               fp4_stride=O.fp4_expert_nbytes(H, I), num_slots=E)
    x = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, k), dtype=torch.int32, device="cuda")
    w = torch.empty((0, k), dtype=torch.float32, device="cuda")
    out = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    gpu_lib.moe_prefill_forward(layer, x, k, ids, w, out, ws)
    torch.cuda.synchronize()
