"""GPU parity: the HIP path through the C ABI against the CPU oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle as O
from mixture_experts_layer_37_amd import _lib as L
from mixture_experts_layer_37_amd import configs as C
from mixture_experts_layer_37_amd.inputs import ExpertView, as_float, f32_to_bf16_bits, make_inputs
from mixture_experts_layer_37_amd.layer import MoELayer, from_device, to_device

import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _report(name, rep):
    print(f"[parity] {name}: {rep}", flush=True)


# Small shapes that still span several tiles in every dimension and end in ragged tiles.
CASES = {
    "tiny_fp32": C.TINY,
    "bf16_ragged": C.SMALL.with_(name="bf16_ragged", tokens=2000, hidden=512, inter=768),
    "bf16_capacity": C.CAP32.with_(name="bf16_capacity", tokens=1500, hidden=256, inter=384,
                                   experts=16, capacity_factor=0.9),
    "bf16_many_experts": C.FINE.with_(name="bf16_many_experts", tokens=700, hidden=256, inter=256,
                                      experts=128, top_k=8),
    "bf16_gelu": C.SMALL.with_(name="bf16_gelu", tokens=600, hidden=256, inter=512,
                               activation=C.GELU, bias=None),
    "bf16_raw_weights": C.SMALL.with_(name="bf16_raw_weights", tokens=300, hidden=256, inter=256,
                                      renormalize=False, experts=12, top_k=3),
    "bf16_single_token": C.MIXTRAL.with_(name="bf16_single_token", tokens=1, hidden=256, inter=256),
    "bf16_max_experts": C.FINE.with_(name="bf16_max_experts", tokens=512, hidden=256, inter=128,
                                     experts=256, top_k=16, bias=("normal", 4.0)),
    "bf16_one_expert": C.SMALL.with_(name="bf16_one_expert", tokens=333, hidden=256, inter=256,
                                     experts=1, top_k=1, bias=None),
    # the streaming router (E <= 16, H a multiple of 1024): ragged token blocks, E not a
    # multiple of 8 (lanes for experts >= E carry zeros), both staging buffers in use
    "bf16_stream_router": C.SMALL.with_(name="bf16_stream_router", tokens=1000, hidden=1024,
                                        inter=256, experts=12, top_k=3),
    "bf16_stream_router_e16": C.SMALL.with_(name="bf16_stream_router_e16", tokens=777,
                                            hidden=2048, inter=256, experts=16, top_k=4,
                                            bias=("normal", 1.0)),
    "fp32_swiglu_capacity": C.TINY.with_(name="fp32_swiglu_capacity", tokens=257, hidden=40,
                                         inter=24, experts=5, top_k=2, activation=C.SWIGLU,
                                         capacity_factor=0.6, bias=("zipf", 1.1)),
    # threshold routing (experts with softmax score > delta): delta = 1/E with no cap (the
    # streaming router), a cap of 3 slots that binds, an explicit delta with capacity, the
    # MFMA router with 64 experts, and the fp32 layer
    "thr_uncapped": C.SMALL.with_(name="thr_uncapped", tokens=1200, hidden=1024, inter=384,
                                  experts=8, top_k=8, routing="threshold", bias=None),
    "thr_capped": C.SMALL.with_(name="thr_capped", tokens=900, hidden=512, inter=256,
                                experts=12, top_k=3, routing="threshold",
                                router_std=0.3 / 512 ** 0.5),
    "thr_delta_capacity": C.SMALL.with_(name="thr_delta_capacity", tokens=1000, hidden=256,
                                        inter=256, experts=16, top_k=6, routing="threshold",
                                        threshold=0.08, capacity_factor=0.8, renormalize=False),
    "thr_many_experts": C.FINE.with_(name="thr_many_experts", tokens=600, hidden=256,
                                     inter=256, experts=64, top_k=16, routing="threshold"),
    "thr_fp32": C.TINY.with_(name="thr_fp32", tokens=200, hidden=48, inter=32, experts=6,
                             top_k=6, routing="threshold"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_matches_oracle(name):
    cfg = CASES[name]
    print(f"[case] {name} {cfg}", flush=True)
    rep, _ = P.full_check(cfg, make_inputs(cfg, seed=0))
    _report(name, rep)
    if cfg.capacity_factor > 0 and name == "bf16_capacity":
        assert rep["dropped"] > 0


def _random_config(seed):
    """A seeded random bf16 layer within the boundary's limits: token count, hidden and
    intermediate sizes, expert count, k, routing rule, capacity, gate bias, activation and
    weight renormalisation all drawn."""
    rng = np.random.default_rng(7000 + seed)
    act = C.GELU if rng.random() < 0.3 else C.SWIGLU
    E = int(rng.choice([1, 3, 6, 8, 12, 16, 24, 40, 96]))
    k = int(rng.integers(1, min(E, 8) + 1))
    routing = "threshold" if rng.random() < 0.3 else "topk"
    bias = [None, ("normal", 1.0), ("zipf", 1.1)][int(rng.integers(0, 3))]
    return C.SMALL.with_(
        name=f"random_{seed}", tokens=int(rng.integers(1, 2500)),
        hidden=int(rng.choice([256, 512, 1024, 2048])),
        inter=int(rng.integers(1, 10)) * (256 if act == C.GELU else 128),
        experts=E, top_k=k, activation=act, routing=routing, bias=bias,
        capacity_factor=float(rng.choice([0.0, 0.0, 0.6, 1.0, 1.4])),
        renormalize=bool(rng.random() < 0.8))


# Seeded random layers through moe_forward against the oracle, for combinations the named
# cases above do not fix (each prints its configuration first).
@pytest.mark.parametrize("seed", range(6))
def test_random_layers_match_oracle(seed):
    cfg = _random_config(seed)
    print(f"[case] random layer {seed}: {cfg}", flush=True)
    rep, _ = P.full_check(cfg, make_inputs(cfg, seed=seed))
    _report(cfg.name, rep)


def test_deterministic_bytes():
    cfg = CASES["bf16_many_experts"]
    inp = make_inputs(cfg, seed=3)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    a = layer.forward(x).clone()
    ya = layer.view(L.MOE_WS_Y_PERM).clone()
    b = layer.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(ya.view(torch.int16), layer.view(L.MOE_WS_Y_PERM).view(torch.int16))


def test_empty_batch_is_a_noop():
    cfg = C.SMALL.with_(tokens=0, hidden=256, inter=256)
    inp = make_inputs(cfg.with_(tokens=4), seed=0)
    layer = MoELayer(cfg, inp, tokens=0)
    out = torch.empty((0, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((0, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    layer.forward(x, out)
    torch.cuda.synchronize()
    assert layer.device_status() == 0


def _route_only(cfg, logits_np):
    """moe_route with x = NULL: top-k straight from the given fp32 logits."""
    T, E, k = logits_np.shape[0], cfg.experts, cfg.top_k
    c = L.cconfig(cfg, T)
    ws = torch.empty(L.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    lg = torch.from_numpy(logits_np.astype(np.float32)).cuda()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    L.moe_route(c, None, None, None, lg, idx, w, ws)
    flags = L.moe_read_device_status(c, ws, 1)
    return idx.cpu().numpy(), w.cpu().numpy(), flags


@pytest.mark.parametrize("E,k", [(8, 2), (9, 3), (32, 4), (128, 8), (256, 16), (5, 5), (64, 1)])
def test_topk_tie_suite(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 300
    pool = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 2.0], dtype=np.float32)
    L_np = pool[rng.integers(0, len(pool), (T, E))]
    L_np[:100] = rng.standard_normal((100, E)).astype(np.float32)       # distinct values
    L_np[100:110] = 0.0                                                  # all tied
    L_np[110, 0] = np.nan
    L_np[111, E - 1] = np.inf
    L_np[112, :] = -np.inf
    L_np[113, ::2] = np.nan
    cfg = C.SMALL.with_(tokens=T, hidden=256, inter=256, experts=E, top_k=k)
    idx, w, flags = _route_only(cfg, L_np)
    P.check_route_from_logits(L_np, idx, w, cfg)
    assert flags == L.MOE_FLAG_NONFINITE_LOGIT
    np.testing.assert_array_equal(idx[100:110], np.tile(np.arange(k), (10, 1)))
    idx2, w2, flags2 = _route_only(cfg, L_np[:100])
    assert flags2 == 0
    np.testing.assert_array_equal(idx2, idx[:100])


@pytest.mark.parametrize("E,k,H,routing,renorm", [
    (8, 2, 1024, "topk", True),        # streaming router (small gate)
    (32, 4, 256, "topk", True),        # general router, 32-expert layout
    (64, 8, 512, "topk", False),       # 64-expert layout, raw softmax weights
    (128, 8, 1024, "topk", True),      # 128-expert layout
    (256, 16, 256, "topk", True),      # 256-expert layout
    (128, 8, 512, "threshold", True),  # threshold routing through the general router
])
def test_router_gemm_ties_and_nonfinite_logits(E, k, H, routing, renorm):
    """Tied, infinite and NaN logits made by the gate GEMM itself: one-hot token rows of value
    1 copy router rows of small integers (exact ties), rows of value +inf / -inf give +-inf
    (NaN where the router entry is 0), an all-NaN row gives NaN logits; the rest are random.
    Selection from the exported logits is bit-exact to the oracle's rank rule (NaN lowest,
    lower index first), the weights agree, and the non-finite flag is raised."""
    T = 300
    cfg = C.SMALL.with_(tokens=T, hidden=H, inter=256, experts=E, top_k=k, bias=None,
                        routing=routing, renormalize=renorm)
    print(f"[case] router E={E} k={k} H={H} {routing} renorm={renorm}", flush=True)
    rng = np.random.default_rng(E + 7 * k + H)
    x = np.zeros((T, H), dtype=np.float32)
    hot = np.arange(T) % H
    x[np.arange(150), hot[:150]] = 1.0
    x[np.arange(150, 200), hot[150:200]] = np.inf
    x[np.arange(200, 210), hot[200:210]] = -np.inf
    x[210] = np.nan
    x[211:] = rng.standard_normal((T - 211, H)).astype(np.float32)
    wr = rng.integers(-2, 3, (H, E)).astype(np.float32)
    c = L.cconfig(cfg)
    ws = torch.empty(L.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    xd = to_device(cfg, f32_to_bf16_bits(x))
    wd = to_device(cfg, f32_to_bf16_bits(wr))
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    L.moe_route(c, xd, wd, None, lg, idx, w, ws)
    flags = L.moe_read_device_status(c, ws, 1)
    gl = lg.cpu().numpy()
    np.testing.assert_array_equal(gl[:150], wr[hot[:150]])
    with np.errstate(invalid="ignore"):
        np.testing.assert_array_equal(gl[150:200], np.inf * wr[hot[150:200]])
        np.testing.assert_array_equal(gl[200:210], -np.inf * wr[hot[200:210]])
    assert np.isnan(gl[210]).all()
    P.check_route_from_logits(gl, idx.cpu().numpy(), w.cpu().numpy(), cfg)
    assert flags == L.MOE_FLAG_NONFINITE_LOGIT


@pytest.mark.parametrize("T,H,E,k", [
    (333, 768, 40, 3),     # 64-expert layout, 6 pieces of 128 k: two-deep ring
    (129, 1280, 20, 5),    # 32-expert layout, 10 pieces of 128 k: one k-step per k-share
    (200, 2560, 17, 4),    # 32-expert layout, 10 pieces of 256 k
    (64, 768, 100, 7),     # 128-expert layout, one block of 128 tokens, half past the end
    (97, 1536, 200, 9),    # 256-expert layout, 12 pieces: four-deep ring
])
def test_general_router_shapes(T, H, E, k):
    """The general router at hidden sizes whose piece counts take the two-deep ring or
    narrower pieces, expert counts between the layouts' multiples of 16, and token counts
    that end inside a block: logits against the fp64 gate GEMM, routing bit-exact from the
    exported logits, no flags."""
    cfg = C.SMALL.with_(tokens=T, hidden=H, inter=256, experts=E, top_k=k,
                        bias=("normal", 0.5))
    print(f"[case] general router T={T} H={H} E={E} k={k}", flush=True)
    inp = make_inputs(cfg, seed=T + E)
    c = L.cconfig(cfg)
    ws = torch.empty(L.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    xd = to_device(cfg, inp["x"])
    wd = to_device(cfg, inp["w_router"])
    bd = torch.from_numpy(np.asarray(inp["bias"], dtype=np.float32)).cuda()
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    L.moe_route(c, xd, wd, bd, lg, idx, w, ws)
    flags = L.moe_read_device_status(c, ws, 1)
    gl = lg.cpu().numpy()
    ref = O.gate_logits(as_float(cfg, inp["x"]), as_float(cfg, inp["w_router"]), inp["bias"])
    assert np.all(np.abs(gl - ref) <= P.LOGIT_RTOL * (1.0 + np.abs(ref)))
    P.check_route_from_logits(gl, idx.cpu().numpy(), w.cpu().numpy(), cfg)
    assert flags == 0


def test_route_entry_point_with_crafted_ties():
    """Logits made exactly equal through the gate GEMM itself: one-hot x rows pick router rows."""
    T, E, k, H = 200, 16, 4, 256
    cfg = C.SMALL.with_(tokens=T, hidden=H, inter=256, experts=E, top_k=k, bias=None)
    rng = np.random.default_rng(7)
    x = np.zeros((T, H), dtype=np.float32)
    x[np.arange(T), np.arange(T) % H] = 1.0
    wr = rng.integers(-2, 3, (H, E)).astype(np.float32)
    c = L.cconfig(cfg)
    ws = torch.empty(L.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    xd = to_device(cfg, f32_to_bf16_bits(x))
    wd = to_device(cfg, f32_to_bf16_bits(wr))
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    L.moe_route(c, xd, wd, None, lg, idx, w, ws)
    gl = lg.cpu().numpy()
    np.testing.assert_array_equal(gl, wr[np.arange(T) % H])
    P.check_route_from_logits(gl, idx.cpu().numpy(), w.cpu().numpy(), cfg)


def test_permute_entry_point_flags_invalid_ids():
    T, E, k, H = 1100, 6, 3, 256
    cfg = C.SMALL.with_(tokens=T, hidden=H, inter=256, experts=E, top_k=k, capacity_factor=0.7)
    rng = np.random.default_rng(11)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    idx[5, 1] = E          # out of range
    idx[17, 0] = -3        # negative
    idx[1030, 2] = idx[1030, 0]   # repeated within the token
    x = make_inputs(cfg, seed=1, weights=False)["x"]
    c = L.cconfig(cfg)
    ws = torch.empty(L.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    xd = to_device(cfg, x)
    xp = torch.full((T * k, H), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    rt = torch.empty(T * k, dtype=torch.int32, device="cuda")
    sr = torch.empty((T, k), dtype=torch.int32, device="cuda")
    L.moe_permute(c, xd, torch.from_numpy(idx).cuda(), xp, counts, offs, rt, sr, ws)
    assert L.moe_read_device_status(c, ws, 2) == L.MOE_FLAG_BAD_INDEX
    cap = O.capacity(0.7, T, k, E)
    P.check_permute(cfg, x, idx, cap, counts.cpu().numpy(), offs.cpu().numpy(), sr.cpu().numpy(),
                    rt.cpu().numpy(), from_device(xp))
    s = sr.cpu().numpy()
    assert s[5, 1] == -1 and s[17, 0] == -1 and s[1030, 2] == -1
    # rows past the kept total are left untouched
    n = int(offs[-1].item())
    assert (from_device(xp)[n:] == 7).all()


def test_stage_entry_points_compose_to_forward():
    cfg = CASES["bf16_capacity"]
    inp = make_inputs(cfg, seed=2)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    ref = layer.forward(x).clone()
    c, T, k, E, H, I = layer.c, cfg.tokens, cfg.top_k, cfg.experts, cfg.hidden, cfg.inter
    ws = torch.empty_like(layer.ws)
    dev = "cuda"
    lg = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    L.moe_route(c, x, layer.w_router, layer.bias, lg, idx, w, ws)
    xp = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    rt = torch.empty(T * k, dtype=torch.int32, device=dev)
    sr = torch.empty((T, k), dtype=torch.int32, device=dev)
    L.moe_permute(c, x, idx, xp, counts, offs, rt, sr, ws)
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    L.moe_expert_up(c, xp, offs, layer.w_gate, layer.w_up, h)
    L.moe_expert_down(c, h, offs, layer.w_down, y, ws)
    y2 = torch.empty_like(y)
    L.moe_grouped_ffn(c, xp, offs, layer.w_gate, layer.w_up, layer.w_down, y2, ws)
    out = torch.empty_like(x)
    L.moe_combine(c, y, sr, w, out)
    torch.cuda.synchronize()
    n = int(offs[-1].item())
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(y[:n].view(torch.int16), y2[:n].view(torch.int16))
    assert torch.equal(h[:n].view(torch.int16), layer.view(L.MOE_WS_H)[:n].view(torch.int16))


def test_single_expert_gemm_matches_torch_matmul():
    """All tokens on one expert: GEMM 2 against torch's own matmul of the same bf16 inputs."""
    cfg = C.MIXTRAL.with_(tokens=1000, hidden=512, inter=1024, experts=1, top_k=1)
    inp = make_inputs(cfg, seed=5)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    layer.forward(x)
    h = layer.view(L.MOE_WS_H)
    y = layer.view(L.MOE_WS_Y_PERM)
    ref = (h.float() @ layer.w_down[0].float())
    torch.cuda.synchronize()
    rel = ((y.float() - ref).abs().max() / ref.abs().max()).item()
    assert rel < 1e-2, rel


@pytest.mark.parametrize("name", ["bf16_capacity", "bf16_many_experts", "fp32_swiglu_capacity",
                                  "bf16_gelu"])
def test_expert_up_rows_equals_gather_then_expert_up(name):
    """GEMM 1 reading token rows in place through row_token gives bit-identical h to GEMM 1 on
    the x_perm that moe_permute materialises; the row-maps-only permute (x_perm = NULL) writes
    the same maps as the materialising one."""
    cfg = CASES[name]
    inp = make_inputs(cfg, seed=4)
    layer = MoELayer(cfg, inp)
    c, T, k, E, H, I = layer.c, cfg.tokens, cfg.top_k, cfg.experts, cfg.hidden, cfg.inter
    dev = "cuda"
    x = to_device(cfg, inp["x"])
    edt = x.dtype
    ws = torch.empty_like(layer.ws)
    lg = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    L.moe_route(c, x, layer.w_router, layer.bias, lg, idx, w, ws)
    maps = []
    for materialise in (True, False):
        xp = torch.empty((T * k, H), dtype=edt, device=dev) if materialise else None
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
        rt = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
        sr = torch.empty((T, k), dtype=torch.int32, device=dev)
        L.moe_permute(c, x, idx, xp, counts, offs, rt, sr, ws)
        maps.append((xp, counts, offs, rt, sr))
    (xp, counts, offs, rt, sr), (_, counts2, offs2, rt2, sr2) = maps
    torch.cuda.synchronize()
    n = int(offs[-1].item())
    assert torch.equal(counts, counts2) and torch.equal(offs, offs2) and torch.equal(sr, sr2)
    assert torch.equal(rt[:n], rt2[:n])
    h1 = torch.zeros((T * k, I), dtype=edt, device=dev)
    h2 = torch.ones((T * k, I), dtype=edt, device=dev)
    L.moe_expert_up(c, xp, offs, layer.w_gate, layer.w_up, h1)
    L.moe_expert_up_rows(c, x, rt, offs, layer.w_gate, layer.w_up, h2)
    torch.cuda.synchronize()
    bits = torch.int16 if edt == torch.bfloat16 else torch.int32
    assert torch.equal(h1[:n].view(bits), h2[:n].view(bits))


# Expert row counts around the 256-row m-tile and the 128-row half tile that takes an
# expert's last 1 .. 128 rows: none, one, 127, exactly 128, 129 (a whole ragged tile), 255,
# 256, 257 (a whole tile and a one-row half tile), 384 (a whole tile and a full half tile),
# 600 (two whole tiles and 88 rows), 700 (two whole tiles and a whole tile of 188 rows).
RAGGED_ROWS = [0, 1, 127, 128, 129, 255, 256, 257, 384, 600, 700]


@pytest.mark.parametrize("activation", [C.SWIGLU, C.GELU])
def test_expert_up_ragged_rows(activation):
    """GEMM 1 on x_perm with crafted expert offsets: every row of h against the float64
    activation of the products of the same bf16 inputs."""
    E, T = len(RAGGED_ROWS), sum(RAGGED_ROWS)
    cfg = C.SMALL.with_(name=f"ragged_{activation}", tokens=T, hidden=512, inter=512,
                        experts=E, top_k=1, activation=activation, bias=None)
    print(f"[case] ragged rows {activation} {RAGGED_ROWS}", flush=True)
    inp = make_inputs(cfg, seed=8)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    o = np.concatenate([[0], np.cumsum(RAGGED_ROWS)]).astype(np.int32)
    offs = torch.from_numpy(o).to("cuda")
    h = torch.full((T, cfg.inter), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    L.moe_expert_up(layer.c, x, offs, layer.w_gate, layer.w_up, h)
    torch.cuda.synchronize()
    hf = P.decode(cfg, h)
    xf = as_float(cfg, inp["x"]).astype(np.float64)
    wu = ExpertView(cfg, inp["w_up"])
    wg = ExpertView(cfg, inp["w_gate"]) if activation == C.SWIGLU else None
    ref = np.empty_like(hf)
    for e in range(E):
        xr = xf[o[e]:o[e + 1]]
        u = xr @ wu[e].astype(np.float64)
        ref[o[e]:o[e + 1]] = (O.silu(xr @ wg[e].astype(np.float64)) * u
                              if activation == C.SWIGLU else O.gelu(u))
    _report(f"ragged_{activation}", P.assert_layer_close(hf, ref, "h"))
    for e in range(E):   # every expert's rows, checked on their own
        if o[e + 1] > o[e]:
            P.assert_layer_close(hf[o[e]:o[e + 1]], ref[o[e]:o[e + 1]], f"h of expert {e}")


# GEMM 2's split-K tail: shapes whose tile list leaves a partial round of the grid and whose
# K is long enough to be sliced: two slices over an odd number of k-step pairs, four slices,
# and whole rounds followed by a sliced tail.
SPLIT_CASES = {
    "split2_uneven": C.SMALL.with_(name="split2_uneven", tokens=1500, hidden=512, inter=2176,
                                   bias=None),
    "split4": C.SMALL.with_(name="split4", tokens=1500, hidden=512, inter=4096, bias=None),
    "rounds_plus_tail": C.SMALL.with_(name="rounds_plus_tail", tokens=4000, hidden=2048,
                                      inter=2048, bias=None),
}


def _expected_split(offsets, hidden, inter):
    """(whole tiles, sliced tiles, slices) that the launch should use, for the coverage check."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = max(8, cus // 8 * 8)
    m = np.diff(offsets)
    total = int(((m + 255) // 256).sum()) * (hidden // 256)
    full, tail, kt, s = total // grid * grid, total % grid, inter // 64, 1
    while tail > 0 and s < 8 and tail * s * 2 <= min(grid, 256) and kt >= 32 * s:
        s *= 2
    return (full, tail, s) if s > 1 else (total, 0, 1)


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_down_split_tail(name):
    """GEMM 2 with the workspace (split-K tail) and without (every tile whole), each against
    the float64 product of the GPU's own h and W_down on every row; the two launches differ
    only in float32 summation order, so they agree to within one bf16 ulp."""
    cfg = SPLIT_CASES[name]
    print(f"[case] {name} {cfg}", flush=True)
    inp = make_inputs(cfg, seed=6)
    layer = MoELayer(cfg, inp)
    x = to_device(cfg, inp["x"])
    layer.forward(x)
    h, offs = layer.view(L.MOE_WS_H), layer.view(L.MOE_WS_OFFSETS)
    y = layer.view(L.MOE_WS_Y_PERM).clone()
    y2 = torch.empty_like(y)
    L.moe_expert_down(layer.c, h, offs, layer.w_down, y2)
    torch.cuda.synchronize()
    o = offs.cpu().numpy().astype(np.int64)
    full, tail, s = _expected_split(o, cfg.hidden, cfg.inter)
    print(f"[split] {name}: whole tiles {full}, sliced tiles {tail} x {s}", flush=True)
    assert s > 1, "the case no longer exercises the split"
    n = int(o[-1])
    hf, yf, y2f = P.decode(cfg, h[:n]), P.decode(cfg, y[:n]), P.decode(cfg, y2[:n])
    wd = ExpertView(cfg, inp["w_down"])
    ref = np.empty_like(yf)
    for e in range(cfg.experts):
        ref[o[e]:o[e + 1]] = hf[o[e]:o[e + 1]] @ wd[e].astype(np.float64)
    _report(name, {"split": P.assert_layer_close(yf, ref, "split"),
                   "whole": P.assert_layer_close(y2f, ref, "whole")})
    mag = np.maximum(np.abs(yf), np.abs(y2f))
    ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-30))) - 7)
    assert (np.abs(yf - y2f) <= ulp + 1e-5 * np.abs(ref).max()).all()


def test_threshold_route_entry_point_edges():
    """Threshold routing from given logits: rows whose scores sit exactly on delta = 1/E
    (all equal: nothing kept), two-level rows (exactly one group kept), a cap that binds,
    and non-finite rows (nothing kept, flagged); everything else on random logits."""
    T, E, k = 400, 8, 8
    cfg = C.SMALL.with_(tokens=T, hidden=256, inter=256, experts=E, top_k=k,
                        routing="threshold")
    rng = np.random.default_rng(21)
    L_np = (rng.standard_normal((T, E)) * 1.5).astype(np.float32)
    L_np[:10] = 0.25                                   # uniform: p = 1/E exactly
    for i in range(10, 30):                            # a experts at u, the rest at 0
        a, u = 1 + i % (E - 1), (0.5 if i % 2 else -0.5)
        L_np[i] = 0.0
        L_np[i, :a] = u
    L_np[30, 2] = np.nan
    L_np[31, 5] = np.inf
    L_np[32, :4] = -np.inf
    idx, w, flags = _route_only(cfg, L_np)
    assert flags == L.MOE_FLAG_NONFINITE_LOGIT
    assert P.check_route_from_logits(L_np, idx, w, cfg) == 10   # the uniform rows
    assert (idx[:10] == -1).all() and (w[:10] == 0).all()
    for i in range(10, 30):
        a = 1 + i % (E - 1)
        want = list(range(a)) if i % 2 else list(range(a, E))
        assert [int(e) for e in idx[i] if e >= 0] == want
    assert (idx[30:32] == -1).all()
    # a cap of 2 slots keeps the two best of the experts above delta
    cfg2 = cfg.with_(top_k=2)
    idx2, w2, _ = _route_only(cfg2, L_np)
    P.check_route_from_logits(L_np, idx2, w2, cfg2)
    full = [[int(e) for e in r if e >= 0] for r in idx]
    assert all([int(e) for e in r2 if e >= 0] == f[:2] for r2, f in zip(idx2, full))


def test_threshold_rows_flow_through_permute_without_flags():
    """-1 slots from threshold routing are empty, not invalid: no bad-index flag, and the
    permutation of the GPU's ids matches the oracle's."""
    cfg = CASES["thr_uncapped"]
    inp = make_inputs(cfg, seed=3)
    layer = MoELayer(cfg, inp)
    layer.forward(to_device(cfg, inp["x"]))
    torch.cuda.synchronize()
    idx = layer.view(L.MOE_WS_TOPK_IDX).cpu().numpy()
    assert (idx == -1).any() and layer.device_status() == 0
    kept = (idx >= 0).sum(1)
    print(f"[threshold] experts per token: mean {kept.mean():.2f}, min {kept.min()}, "
          f"max {kept.max()}", flush=True)
    assert kept.min() >= 1 and kept.max() <= cfg.experts - 1


# The row maps come from the count and one scan-and-rows launch on batches of up to 65536
# tokens (64 count blocks), and from the three-launch count / scan / rows path above that;
# with an x_perm destination the three-launch path (its third launch the gather) always
# runs. Both against the oracle's permutation, and the two paths against each other, on
# batches on both sides of the boundary, with capacity drops, empty (-1) slots and invalid
# ids.
@pytest.mark.parametrize("T,E,k,cf", [(1100, 6, 3, 0.7), (9000, 16, 2, 0.0),
                                      (65536, 8, 2, 1.1), (65537, 64, 4, 0.9),
                                      (70000, 16, 2, 0.0), (40000, 128, 8, 0.0),
                                      (5000, 256, 16, 1.0)])
def test_row_map_paths_agree(T, E, k, cf):
    cfg = C.SMALL.with_(tokens=T, hidden=256, inter=256, experts=E, top_k=k,
                        capacity_factor=cf)
    rng = np.random.default_rng(T + E)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    idx[rng.random((T, k)) < 0.02] = -1                 # empty slots
    idx[3, 0] = E                                       # out of range
    idx[T - 1, k - 1] = idx[T - 1, 0] if k > 1 else -2  # repeated (or negative)
    c = L.cconfig(cfg)
    ws = torch.empty(L.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
    xd = torch.zeros((T, 256), dtype=torch.bfloat16, device="cuda")
    idd = torch.from_numpy(idx).cuda()
    out = {}
    for tag, xp in (("maps", None),
                    ("gather", torch.empty((T * k, 256), dtype=torch.bfloat16, device="cuda"))):
        counts = torch.full((E,), -9, dtype=torch.int32, device="cuda")
        offs = torch.full((E + 1,), -9, dtype=torch.int32, device="cuda")
        rt = torch.full((T * k,), -9, dtype=torch.int32, device="cuda")
        sr = torch.full((T, k), -9, dtype=torch.int32, device="cuda")
        print(f"[permute] T={T} E={E} k={k} cf={cf} path={tag}", flush=True)
        L.moe_permute(c, xd, idd, xp, counts, offs, rt, sr, ws)
        flag = L.moe_read_device_status(c, ws, 2)
        out[tag] = [a.cpu().numpy() for a in (counts, offs, rt, sr)] + [flag]
    cap = O.capacity(cf, T, k, E) if cf > 0 else T
    counts, offs, rt, sr, flag = out["maps"]
    P.check_permute(cfg, None, idx, cap, counts, offs, sr, rt)
    assert flag == L.MOE_FLAG_BAD_INDEX
    n = int(offs[-1])
    for a, b in zip(out["maps"][:3], out["gather"][:3]):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(out["maps"][3], out["gather"][3])
    np.testing.assert_array_equal(out["maps"][2][:n], out["gather"][2][:n])
    assert out["gather"][4] == flag


# moe_route_permute (the count step inside the streaming router, two launches) against
# moe_route then moe_permute on the same inputs: every output bit for bit, and the flags.
# The streaming router's cases: a whole Mixtral gate, ragged token blocks, capacity drops,
# threshold routing with empty slots, 16 experts, T beyond one 65536-token map batch, a
# single token; then a 32-expert gate, which takes the two calls inside it.
@pytest.mark.parametrize("T,H,E,k,routing,cf", [(8192, 4096, 8, 2, "topk", 0.0),
                                                (1000, 1024, 12, 3, "topk", 0.7),
                                                (5000, 2048, 16, 4, "threshold", 0.0),
                                                (777, 4096, 8, 8, "threshold", 0.9),
                                                (33, 1024, 5, 1, "topk", 0.0),
                                                (70000, 1024, 8, 2, "topk", 1.1),
                                                (1, 1024, 8, 2, "topk", 0.0),
                                                (600, 512, 32, 4, "topk", 0.8)])
def test_route_permute_matches_route_then_permute(T, H, E, k, routing, cf):
    cfg = C.SMALL.with_(tokens=T, hidden=H, inter=256, experts=E, top_k=k, routing=routing,
                        capacity_factor=cf, bias=("normal", 1.0))
    inp = make_inputs(cfg, seed=T + 3 * E, weights=False)
    x = to_device(cfg, inp["x"])
    w = to_device(cfg, inp["w_router"])
    bias = to_device(cfg, inp["bias"])
    c = L.cconfig(cfg)
    out = {}
    for tag in ("separate", "fused"):
        ws = torch.empty(L.moe_workspace_size(c), dtype=torch.uint8, device="cuda")
        lg = torch.full((T, E), -9.0, dtype=torch.float32, device="cuda")
        idx = torch.full((T, k), -9, dtype=torch.int32, device="cuda")
        tw = torch.full((T, k), -9.0, dtype=torch.float32, device="cuda")
        counts = torch.full((E,), -9, dtype=torch.int32, device="cuda")
        offs = torch.full((E + 1,), -9, dtype=torch.int32, device="cuda")
        rt = torch.full((T * k,), -9, dtype=torch.int32, device="cuda")
        sr = torch.full((T, k), -9, dtype=torch.int32, device="cuda")
        # raise the permutation's bad-id flag in this workspace first: the call under test
        # must leave its own flags, not this one
        bad = torch.full((T, k), E, dtype=torch.int32, device="cuda")
        L.moe_permute(c, None, bad, None, counts, offs, rt, sr, ws)
        assert L.moe_read_device_status(c, ws, 2) == L.MOE_FLAG_BAD_INDEX
        print(f"[route_permute] T={T} H={H} E={E} k={k} {routing} cf={cf} {tag}", flush=True)
        if tag == "separate":
            L.moe_route(c, x, w, bias, lg, idx, tw, ws)
            L.moe_permute(c, None, idx, None, counts, offs, rt, sr, ws)
        else:
            L.moe_route_permute(c, x, w, bias, lg, idx, tw, counts, offs, rt, sr, ws)
        torch.cuda.synchronize()
        out[tag] = ([a.cpu() for a in (lg, idx, tw, counts, offs, rt, sr)],
                    L.moe_read_device_status(c, ws, 1), L.moe_read_device_status(c, ws, 2))
    (a, fa1, fa2), (b, fb1, fb2) = out["separate"], out["fused"]
    for u, v, what in zip(a, b, ("logits", "idx", "weights", "counts", "offsets", "row_token",
                                 "slot_row")):
        if u.dtype == torch.float32:
            u, v = u.view(torch.int32), v.view(torch.int32)
        assert torch.equal(u, v), what
    assert fa1 == fb1 and fa2 == fb2 == 0
    assert int(a[4][-1]) > 0 and int(a[4][-1]) == int((a[6] >= 0).sum())
