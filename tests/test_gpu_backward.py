"""GPU parity of the backward pass: moe_backward through the C ABI against the float64
oracle's gradients on the same inputs, with the oracle routed on the GPU's own logits (so
both take the same experts)."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_37_amd import _lib as L
from mixture_experts_layer_37_amd import configs as C
from mixture_experts_layer_37_amd.inputs import ExpertView, as_float, f32_to_bf16_bits, make_inputs
from mixture_experts_layer_37_amd.layer import MoELayer, to_device

import parity as P

pytestmark = pytest.mark.gpu

# Gradient bars: bf16 storage with float32 accumulation; a gradient passes through up to
# four bf16 roundings (dy, the saved pre-activations, dg/du, the output), each ~2^-9 ln 2 in
# mean relative error, so mean <= 8e-3 and max <= 3e-2 of max|ref|.
GRAD_MAX_REL = 3e-2
GRAD_MEAN_REL = 8e-3

CASES = {
    "swiglu": C.SMALL.with_(name="bwd_swiglu", tokens=700, hidden=512, inter=512, experts=8,
                            top_k=2),
    "gelu_raw": C.SMALL.with_(name="bwd_gelu_raw", tokens=500, hidden=256, inter=512,
                              experts=6, top_k=3, activation=C.GELU, renormalize=False,
                              bias=None),
    "capacity": C.SMALL.with_(name="bwd_capacity", tokens=900, hidden=256, inter=256,
                              experts=16, top_k=2, capacity_factor=0.7),
    "threshold": C.SMALL.with_(name="bwd_threshold", tokens=600, hidden=512, inter=256,
                               experts=8, top_k=8, routing="threshold", bias=None),
    "many_experts": C.FINE.with_(name="bwd_many_experts", tokens=400, hidden=256, inter=256,
                                 experts=64, top_k=8),
    "one_expert": C.SMALL.with_(name="bwd_one_expert", tokens=333, hidden=256, inter=256,
                                experts=1, top_k=1, bias=None),
    # the bench workload's layer shape (H 4096, I 14336, 8 experts, top-2) on 1024 tokens
    "mixtral_shape": C.MIXTRAL.with_(name="bwd_mixtral_shape", tokens=1024),
    # the largest gate the library takes (256 experts, top-16); one token; experts left
    # without rows (their weight gradients must be exactly zero)
    "max_experts": C.FINE.with_(name="bwd_max_experts", tokens=300, hidden=256, inter=256,
                                experts=256, top_k=16, bias=("normal", 4.0)),
    "single_token": C.MIXTRAL.with_(name="bwd_single_token", tokens=1, hidden=256, inter=256),
    "empty_experts": C.SMALL.with_(name="bwd_empty_experts", tokens=20, hidden=256, inter=256,
                                   experts=16, top_k=1, bias=None),
    # with the auxiliary load-balancing loss at MindSpeed's largest advised coefficient
    "aux_loss": C.SMALL.with_(name="bwd_aux_loss", tokens=700, hidden=512, inter=512,
                              experts=8, top_k=2, aux_loss_coeff=0.1),
}


def _close(got, ref, what):
    err = np.abs(got - ref)
    mx = err.max() / max(np.abs(ref).max(), 1e-30)
    mean = err.sum() / max(np.abs(ref).sum(), 1e-30)
    assert np.isfinite(got).all(), what
    assert mx <= GRAD_MAX_REL and mean <= GRAD_MEAN_REL, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return float(mx), float(mean)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    _check_backward(CASES[name], name)


def _random_backward_config(seed):
    """A seeded random bf16 layer within the backward's limits (I a multiple of 256, plain
    weights): tokens, sizes, experts, k, routing, capacity, gate bias, activation,
    renormalisation and the auxiliary-loss coefficient all drawn."""
    rng = np.random.default_rng(9100 + seed)
    E = int(rng.choice([1, 4, 8, 12, 16, 24, 48]))
    return C.SMALL.with_(
        name=f"bwd_random_{seed}", tokens=int(rng.integers(1, 1500)),
        hidden=int(rng.choice([256, 512, 1024])), inter=256 * int(rng.integers(1, 5)),
        experts=E, top_k=int(rng.integers(1, min(E, 6) + 1)),
        activation=C.GELU if rng.random() < 0.3 else C.SWIGLU,
        routing="threshold" if rng.random() < 0.3 else "topk",
        bias=[None, ("normal", 1.0), ("zipf", 1.1)][int(rng.integers(0, 3))],
        capacity_factor=float(rng.choice([0.0, 0.0, 0.7, 1.2])),
        renormalize=bool(rng.random() < 0.8),
        aux_loss_coeff=float(rng.choice([0.0, 0.0, 0.01])))


# Seeded random layers through moe_forward_train and moe_backward against the oracle's
# gradients, for combinations the named cases do not fix.
@pytest.mark.parametrize("seed", range(4))
def test_random_backward_matches_oracle(seed):
    _check_backward(_random_backward_config(seed), f"random {seed}")


def _check_backward(cfg, name):
    print(f"[case] {name} {cfg}", flush=True)
    inp = make_inputs(cfg, seed=8)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    layer.forward(x)
    rng = np.random.default_rng(99)
    dout_np = f32_to_bf16_bits(rng.standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32))
    dout = to_device(cfg, dout_np)
    g = layer.backward(x, dout)
    torch.cuda.synchronize()
    gl = layer.view(L.MOE_WS_LOGITS).cpu().numpy().astype(np.float64)
    wg = ExpertView(cfg, inp["w_gate"]) if cfg.activation == C.SWIGLU else None
    ref = O.backward(as_float(cfg, inp["x"]), as_float(cfg, inp["w_router"]), inp["bias"], wg,
                     ExpertView(cfg, inp["w_up"]), ExpertView(cfg, inp["w_down"]),
                     as_float(cfg, dout_np).astype(np.float64), top_k=cfg.top_k,
                     activation=cfg.activation, capacity_factor=cfg.capacity_factor,
                     renormalize=cfg.renormalize, routing=cfg.routing,
                     threshold=cfg.threshold, logits=gl, aux_loss_coeff=cfg.aux_loss_coeff)
    if cfg.aux_loss_coeff > 0:
        assert float(g["aux_loss"].item()) == pytest.approx(ref["aux_loss"], rel=1e-9)
    rep = {"dx": _close(P.decode(cfg, g["dx"]), ref["dx"], "dx"),
           "dw_router": _close(g["dw_router"].cpu().numpy().astype(np.float64), ref["dw_router"],
                               "dw_router"),
           "dbias": _close(g["dbias"].cpu().numpy().astype(np.float64), ref["dbias"], "dbias")}
    offs = layer.view(L.MOE_WS_OFFSETS).cpu().numpy()
    empty = np.nonzero(np.diff(offs) == 0)[0]
    for key in ("dw_gate", "dw_up", "dw_down"):
        if g[key] is None:
            continue
        want = np.stack(ref[key])
        got = P.decode(cfg, g[key]).reshape(want.shape)
        rep[key] = _close(got, want, key)
        assert (got[empty] == 0).all(), f"{key}: experts without rows must get zero gradients"
    rep["experts_without_rows"] = int(len(empty))
    print(f"[backward] {name}: {rep}", flush=True)


def test_backward_is_deterministic():
    cfg = CASES["capacity"]
    inp = make_inputs(cfg, seed=9)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    dout = to_device(cfg, f32_to_bf16_bits(
        np.random.default_rng(5).standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32)))
    outs = []
    for _ in range(2):
        layer.forward(x)
        g = layer.backward(x, dout)
        torch.cuda.synchronize()
        outs.append({k: v.clone() for k, v in g.items() if v is not None})
    for k in outs[0]:
        assert torch.equal(outs[0][k].view(torch.uint8), outs[1][k].view(torch.uint8)), k


@pytest.mark.parametrize("name", ["swiglu", "gelu_raw", "capacity", "threshold"])
def test_saved_preactivations_match_recompute(name):
    """moe_forward_train gives moe_forward's output bit for bit, and the backward that uses
    its kept pre-activations gives the recomputing backward's gradients bit for bit (same
    products, same order)."""
    cfg = CASES[name]
    inp = make_inputs(cfg, seed=10)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    dout = to_device(cfg, f32_to_bf16_bits(
        np.random.default_rng(6).standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32)))
    out_a = layer.forward(x).clone()
    ga = {k: v.clone() for k, v in layer.backward(x, dout).items() if v is not None}
    out_b = layer.forward_train(x).clone()
    gb = {k: v.clone() for k, v in layer.backward(x, dout).items() if v is not None}
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    for k in ga:
        assert torch.equal(ga[k].view(torch.uint8), gb[k].view(torch.uint8)), k


def test_stale_saved_preactivations_are_flagged():
    """moe_backward(saved = 1) after another permutation was built in the workspace (here a
    plain moe_forward between moe_forward_train and the backward) raises
    MOE_FLAG_STALE_SAVED; the regular order raises nothing, and the flag is re-evaluated by
    every backward."""
    cfg = CASES["swiglu"]
    inp = make_inputs(cfg, seed=11)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    dout = to_device(cfg, f32_to_bf16_bits(
        np.random.default_rng(7).standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32)))
    layer.forward_train(x)
    layer.backward(x, dout)
    assert layer.device_status(4) == 0
    layer.forward_train(x)
    out = torch.empty_like(x)
    L.moe_forward(layer.c, x, layer.fw_router, layer.bias, layer.fw_gate, layer.fw_up,
                  layer.fw_down, out, layer.ws, None)
    layer._saved = True            # the caller still believes the saved pre-activations hold
    layer.backward(x, dout)
    assert layer.device_status(4) == L.MOE_FLAG_STALE_SAVED
    assert layer.device_status(3) == 0
    layer.forward_train(x)
    layer.backward(x, dout)
    assert layer.device_status(4) == 0


AUX_CASES = {
    "topk": C.SMALL.with_(name="aux_topk", tokens=700, hidden=512, inter=256, experts=8,
                          top_k=2, aux_loss_coeff=0.1),
    "capacity": C.SMALL.with_(name="aux_capacity", tokens=900, hidden=256, inter=256,
                              experts=16, top_k=2, capacity_factor=0.7, aux_loss_coeff=0.01),
    "threshold_raw": C.SMALL.with_(name="aux_threshold_raw", tokens=600, hidden=512, inter=256,
                                   experts=8, top_k=8, routing="threshold", renormalize=False,
                                   bias=None, aux_loss_coeff=0.05),
    "many_experts": C.FINE.with_(name="aux_many_experts", tokens=513, hidden=256, inter=256,
                                 experts=64, top_k=8, aux_loss_coeff=0.02),
}


@pytest.mark.parametrize("name", list(AUX_CASES))
def test_aux_loss_alone(name):
    """dout = 0 leaves the auxiliary load-balancing loss as the only objective: its value
    against the oracle's (both in float64 from the same float32 logits and counts), the
    router-side gradients (dx, dW_router, dbias) against the oracle's at float32 accuracy,
    and expert-weight gradients exactly zero."""
    cfg = AUX_CASES[name]
    print(f"[case] aux {name} {cfg}", flush=True)
    inp = make_inputs(cfg, seed=12)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    layer.forward(x)
    dout = torch.zeros_like(x)
    g = layer.backward(x, dout)
    torch.cuda.synchronize()
    gl = layer.view(L.MOE_WS_LOGITS).cpu().numpy().astype(np.float64)
    wg = ExpertView(cfg, inp["w_gate"]) if cfg.activation == C.SWIGLU else None
    ref = O.backward(as_float(cfg, inp["x"]), as_float(cfg, inp["w_router"]), inp["bias"], wg,
                     ExpertView(cfg, inp["w_up"]), ExpertView(cfg, inp["w_down"]),
                     np.zeros((cfg.tokens, cfg.hidden)), top_k=cfg.top_k,
                     activation=cfg.activation, capacity_factor=cfg.capacity_factor,
                     renormalize=cfg.renormalize, routing=cfg.routing,
                     threshold=cfg.threshold, logits=gl, aux_loss_coeff=cfg.aux_loss_coeff)
    assert float(g["aux_loss"].item()) == pytest.approx(ref["aux_loss"], rel=1e-9)
    for key in ("dw_router", "dbias"):
        got = g[key].cpu().numpy().astype(np.float64)
        err = np.abs(got - ref[key]).max() / np.abs(ref[key]).max()
        assert err <= 1e-4, f"{key}: {err:.3e}"
    dx = P.decode(cfg, g["dx"])   # bf16 output: one rounding
    err = np.abs(dx - ref["dx"]).max() / np.abs(ref["dx"]).max()
    assert err <= 8e-3, f"dx: {err:.3e}"
    for key in ("dw_gate", "dw_up", "dw_down"):
        if g[key] is not None:
            assert not g[key].view(torch.int16).any(), f"{key} must be zero"
