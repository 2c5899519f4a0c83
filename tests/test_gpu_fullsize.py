"""GPU parity at the full sizes of the five workloads, in the launch configuration the
bench times (packed expert weights for the bf16 layers): routing and the permutation, every
kept y_perm row, the combine and the layer output, on every token."""
import pytest
import torch

from mixture_experts_layer_37_amd import configs as C
from mixture_experts_layer_37_amd.inputs import make_inputs

import parity as P

pytestmark = pytest.mark.gpu

WORKLOADS = ["tiny", "small", "mixtral", "cap32", "fine", "mixtral_threshold"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_full_size_workload(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = C.get(name)
    if cfg.dtype == C.BF16:
        cfg = cfg.with_(weights="packed")
    print(f"[fullsize] {name}: generating inputs", flush=True)
    inputs = make_inputs(cfg, seed=0, threads=16)
    print(f"[fullsize] {name}: running", flush=True)
    rep, layer = P.full_check(cfg, inputs, tokens_sample=None)
    print(f"[fullsize] {name}: {rep}", flush=True)
    T = cfg.tokens
    # every token is compared except the counted exclusions: near ties of the routing
    # decision, and (capacity only) tokens whose kept/dropped status a flipped near tie
    # shifted
    assert rep["compared_tokens"] == T - rep["excluded"]
    assert rep["excluded"] == rep["excluded_near_tie"] + rep["excluded_keep_shift"]
    assert rep["excluded_near_tie"] <= max(5, T // 500)
    assert rep["ffn_rows"] == rep["kept_rows"]          # every kept y_perm row compared
    if cfg.capacity_factor <= 0:
        assert rep["excluded_keep_shift"] == 0
        if cfg.routing == "topk":
            assert rep["kept_rows"] == T * cfg.top_k
    else:
        assert rep["dropped"] > 0
    del layer
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["mixtral", "cap32", "fine"])
def test_full_size_packed_forward_is_bit_identical(name):
    """Full-size workloads on packed weights, in the bench's launch configuration: the output
    equals the plain-weight forward bit for bit (the packed one is checked against the oracle
    on every token above). cap32 has 32 experts and a binding capacity, fine 128 experts and an odd number
    of n-tiles in GEMM 1 (I = 1408)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_37_amd.layer import MoELayer, to_device
    cfg = C.get(name)
    print(f"[fullsize] {name} packed vs plain: generating inputs", flush=True)
    inputs = make_inputs(cfg, seed=0, threads=16)
    x = to_device(cfg, inputs["x"])
    plain = MoELayer(cfg, inputs)
    a = plain.forward(x).clone()
    del plain
    torch.cuda.empty_cache()
    packed = MoELayer(cfg.with_(weights="packed"), inputs)
    b = packed.forward(x)
    torch.cuda.synchronize()
    same = torch.equal(a.view(torch.int16), b.view(torch.int16))
    print(f"[fullsize] {name} packed vs plain: bit-identical {same}", flush=True)
    assert same
    del packed
    torch.cuda.empty_cache()


def test_full_size_backward_splits_over_tokens():
    """The training step at the bench workload's full size (8192 tokens, H 4096, I 14336, 8
    experts, top-2, no capacity limit, no auxiliary loss), in the launch configuration
    `bench.py --backward` times. With no capacity limit and no auxiliary loss every gradient
    is a sum over tokens of per-token terms: a token's routing and dx depend on that token
    alone, and the weight, router and bias gradients of the batch are the sums of those of
    its two halves. The halves run as batches of their own (the backward at this layer shape
    is checked against the oracle on 1024 tokens)."""
    from mixture_experts_layer_37_amd import _lib as L
    from mixture_experts_layer_37_amd.layer import MoELayer, to_device
    import numpy as np
    from mixture_experts_layer_37_amd.inputs import f32_to_bf16_bits

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = C.MIXTRAL.with_(weights="plain")
    assert cfg.capacity_factor == 0 and cfg.aux_loss_coeff == 0
    T, half = cfg.tokens, cfg.tokens // 2
    print("[fullsize] backward: generating inputs", flush=True)
    inputs = make_inputs(cfg, seed=3, threads=16)
    x = to_device(cfg, inputs["x"])
    dout = to_device(cfg, f32_to_bf16_bits(
        np.random.default_rng(13).standard_normal((T, cfg.hidden)).astype(np.float32)))

    def run(tokens, xs, ds):
        layer = MoELayer(cfg, inputs, tokens=tokens)
        layer.forward_train(xs)
        g = {k: v.clone() for k, v in layer.backward(xs, ds).items() if v is not None}
        g["idx"] = layer.view(L.MOE_WS_TOPK_IDX).clone()
        torch.cuda.synchronize()
        del layer
        torch.cuda.empty_cache()
        return g

    print("[fullsize] backward: whole batch", flush=True)
    gf = run(T, x, dout)
    print("[fullsize] backward: two halves", flush=True)
    g0 = run(half, x[:half].contiguous(), dout[:half].contiguous())
    g1 = run(T - half, x[half:].contiguous(), dout[half:].contiguous())

    # routing is per token: the same experts in the same slot order
    assert torch.equal(gf["idx"], torch.cat([g0["idx"], g1["idx"]]))
    # dx: per token; rows may differ only by the summation order of the split-K tail of the
    # dx product (float32) before their bf16 rounding
    dxf = gf["dx"].float()
    dxh = torch.cat([g0["dx"], g1["dx"]]).float()
    scale = dxf.abs().max().item()
    assert (dxf - dxh).abs().max().item() <= 2.0 ** -8 * scale
    assert ((dxf - dxh).abs().mean() / dxf.abs().mean()).item() <= 2.0 ** -10
    # sums over tokens: the whole batch's gradient against the sum of the halves', each a
    # float32 accumulation rounded once (bf16 weight gradients) or not (float32 router)
    for k in ("dw_gate", "dw_up", "dw_down", "dw_router", "dbias"):
        a, b0, b1 = gf[k].float(), g0[k].float(), g1[k].float()
        err = (a - (b0 + b1)).abs()
        bound = 2.0 ** -7 * (b0.abs() + b1.abs()) + 2.0 ** -12 * a.abs().max()
        worst = (err - bound).max().item()
        print(f"[fullsize] backward {k}: max err {err.max().item():.3e}, "
              f"max|g| {a.abs().max().item():.3e}", flush=True)
        assert worst <= 0, k
