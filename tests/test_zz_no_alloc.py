"""moe_permute_noalloc (fixed library scratch, no workspace) against moe_permute (workspace
scratch) through the C ABI: bit-identical row maps, counts, offsets and x_perm, on two calls
in a row on one device, the second with a smaller input (so the second call runs on what
the first left in the shared scratch); and the bad-index flag it reports itself."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_37_amd import _lib as L
from mixture_experts_layer_37_amd import configs as C
from mixture_experts_layer_37_amd.inputs import make_inputs
from mixture_experts_layer_37_amd.layer import to_device

pytestmark = pytest.mark.gpu


def _routing(T, E, k, seed):
    """Distinct expert ids per token, skewed towards low experts (a capacity binds)."""
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
    return idx.astype(np.int32)


def _run(cfg, x, idx_np, noalloc):
    dev = x.device
    T, k, E, H = cfg.tokens, cfg.top_k, cfg.experts, cfg.hidden
    idx = torch.from_numpy(idx_np).to(dev)
    out = dict(x_perm=torch.zeros((T * k, H), dtype=x.dtype, device=dev),
               counts=torch.full((E,), -7, dtype=torch.int32, device=dev),
               offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
               row_token=torch.full((T * k,), -7, dtype=torch.int32, device=dev),
               slot_row=torch.full((T, k), -7, dtype=torch.int32, device=dev))
    c = L.cconfig(cfg, T)
    if noalloc:
        flags = torch.full((1,), -1, dtype=torch.int32, device=dev)
        L.moe_permute_noalloc(c, x, idx, out["x_perm"], out["counts"], out["offsets"],
                              out["row_token"], out["slot_row"], flags)
        torch.cuda.synchronize()
        return out, int(flags.item())
    ws = torch.empty(L.moe_workspace_size(c), dtype=torch.uint8, device=dev)
    L.moe_permute(c, x, idx, out["x_perm"], out["counts"], out["offsets"], out["row_token"],
                  out["slot_row"], ws)
    torch.cuda.synchronize()
    return out, L.moe_read_device_status(c, ws, 2)


def _same(a, b):
    n = int(a["offsets"][-1].item())
    assert torch.equal(a["counts"], b["counts"])
    assert torch.equal(a["offsets"], b["offsets"])
    assert torch.equal(a["slot_row"], b["slot_row"])
    assert torch.equal(a["row_token"][:n], b["row_token"][:n])
    assert torch.equal(a["x_perm"][:n].view(torch.int16), b["x_perm"][:n].view(torch.int16))


def test_noalloc_permute_matches_workspace_permute():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = C.CAP32.with_(tokens=5000, hidden=512, experts=32, top_k=4, capacity_factor=1.1)
    small = C.SMALL.with_(tokens=1500, hidden=256, experts=8, top_k=2)
    for cfg, seed in ((big, 1), (small, 2)):            # the second call is the smaller one
        x = to_device(cfg, make_inputs(cfg, seed=seed, weights=False)["x"])
        idx = _routing(cfg.tokens, cfg.experts, cfg.top_k, seed)
        ref, ref_flags = _run(cfg, x, idx, noalloc=False)
        got, got_flags = _run(cfg, x, idx, noalloc=True)
        _same(ref, got)
        assert ref_flags == 0 and got_flags == 0
        if cfg.capacity_factor > 0:
            assert (got["slot_row"] < 0).any()           # the capacity bound: drops happen
        # row maps only (x_perm = NULL), as moe_forward's path uses them
        c = L.cconfig(cfg, cfg.tokens)
        rt = torch.full_like(got["row_token"], -7)
        sr = torch.full_like(got["slot_row"], -7)
        cnt = torch.empty_like(got["counts"])
        off = torch.empty_like(got["offsets"])
        L.moe_permute_noalloc(c, x, torch.from_numpy(idx).to(x.device), None, cnt, off, rt, sr)
        torch.cuda.synchronize()
        n = int(off[-1].item())
        assert torch.equal(sr, ref["slot_row"]) and torch.equal(rt[:n], ref["row_token"][:n])
        assert torch.equal(cnt, ref["counts"]) and torch.equal(off, ref["offsets"])


def test_noalloc_permute_reports_bad_indices():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = C.SMALL.with_(tokens=3000, hidden=256, experts=8, top_k=2)
    x = to_device(cfg, make_inputs(cfg, seed=3, weights=False)["x"])
    idx = _routing(cfg.tokens, cfg.experts, cfg.top_k, 3)
    idx[2500, 1] = 8            # out of range: dropped and flagged, in the third count block
    idx[17, 1] = idx[17, 0]     # a repeat within a token: dropped and flagged
    ref, ref_flags = _run(cfg, x, idx, noalloc=False)
    got, got_flags = _run(cfg, x, idx, noalloc=True)
    _same(ref, got)
    assert ref_flags == L.MOE_FLAG_BAD_INDEX and got_flags == L.MOE_FLAG_BAD_INDEX
    # the next clean call reports no flag (nothing is left over from the shared scratch)
    idx2 = _routing(cfg.tokens, cfg.experts, cfg.top_k, 4)
    got2, got2_flags = _run(cfg, x, idx2, noalloc=True)
    ref2, _ = _run(cfg, x, idx2, noalloc=False)
    _same(ref2, got2)
    assert got2_flags == 0
