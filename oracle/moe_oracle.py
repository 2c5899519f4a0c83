"""CPU oracle for one Mixture-of-Experts FFN layer forward -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy. Only the tests, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg may import it; the HIP library never does, and this module imports
nothing from it.

What is computed, and where the pages state it
----------------------------------------------
* The layer: gate scores are a softmax of ``x @ W_gate``, the k best experts are kept, and
  the output is the gate-weighted sum of those experts' outputs (intelliparadigm.com,
  "MoE模型高效推理：CANN算子库优化实践", section 2.1, the ``moe_layer`` pseudo-code).
* The order of steps: routing scores -> top-k expert ids -> per-expert gather of its tokens
  -> expert forward -> scatter-add into the dense output (gitcode.csdn.net,
  "ops-transformer 仓库 - MoE 算子优化实战", section "核心代码解析", ``MoEOperator::Forward``).
* Expert FFN: an up-projection hidden -> intermediate with weights [E, hidden, inter],
  then the activation, then the down-projection (lshu.cn/news/82007, section 3, the fused
  ``npu_moe_final_optimizer_mm`` example).
* Renormalised top-k weights: the threshold router renormalises the kept scores
  (intelliparadigm.com page, section 3.2.1) and ``moe_router`` defaults to
  ``normalize_scores=True`` (mhpn.cn/news/871594, chapter 8).
* Capacity: a capacity factor bounds each expert's load (hnwysp.cn/news/132341, section 3.2
  and section 4.2); imbalance overflows per-expert buffers (lshu.cn page, section 5.3).
* Expert ids are int32 in [0, E) (lshu.cn page, section 5.2).
* Threshold routing: compute every expert's gate score, keep only the experts whose score
  exceeds a threshold delta (1/E by default), renormalise over the kept ones
  (intelliparadigm.com page, section 3.2.1, the sparse gate; gitcode page, "路由算法": a
  threshold router activates only the experts scoring above the threshold).

Readings where the pages are silent or conflict (each is listed with its reason in the
project's design notes):
  R1 selection is done on the logits (same set and order as on the softmax in exact
     arithmetic); lower expert index wins ties; -0.0 equals +0.0; NaN ranks below -inf.
  R2 weights are renormalised over the k selected experts unless ``renormalize`` is off.
  R3 capacity C = ceil(cf * (T*k) / E) in IEEE double; cf <= 0 means no limit (C = T).
  R4 each expert keeps its assignments in ascending token order up to C; a dropped slot
     contributes zero, is not re-routed and the other weights are not renormalised.
  R5 SwiGLU is silu(x Wg) * (x Wu) then Wd; GELU is the exact erf form; no expert biases.
  R6 a user-supplied expert id outside [0, E) other than -1, or one repeated within a
     token's slots (the later slot), is invalid: the slot is dropped and flagged. -1 marks
     an empty slot (threshold routing): dropped, not flagged.
  R14 threshold routing: the score is the softmax probability p (float64); an expert is
     kept when p > delta strictly; delta <= 0 or absent means 1/E. The kept experts are
     listed best first (the order of R1) in at most k slots (k caps the experts per token;
     with k = E nothing is capped); the remaining slots hold -1 and weight 0. A token with
     no expert above delta (all scores equal to 1/E, or a NaN or +inf logit) contributes
     zero. Renormalisation (R2) is over the kept experts.
  R15 backward: the gradient of sum(out * dout); the expert choice (top-k, threshold,
     capacity) is piecewise constant in the logits and contributes no gradient; the gate
     weights' dependence on the logits is differentiated exactly.
  R16 auxiliary load-balancing loss. The pages describe an extra loss term that penalises
     uneven expert load and pushes the router to spread tokens evenly (mhpn.cn/news/871594,
     the routing chapter), scaled by MindSpeed's moe-aux-loss-coeff (0.01, at most 0.1:
     lshu.cn/news/82007, section 5.3), but give no formula. Read as the published
     switch-style form coeff * E * sum_e f_e P_e: f_e is the fraction of the routed
     assignments (the valid selected slots, before any capacity drop; T*k under top-k)
     that chose expert e, P_e the mean over the T tokens of expert e's softmax probability.
     The counts are piecewise constant in the logits (no gradient, as R15); the gradient
     flows through P. Off (coefficient 0) unless asked for.

Every function here is pinned by tests/test_oracle_*.py against hand-worked cases, closed
forms, brute force and invariants that do not reuse this code.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

FLAG_BAD_INDEX = 1
FLAG_NONFINITE_LOGIT = 2


# ---------------------------------------------------------------- step 1: gate GEMM
def gate_logits(x, w_router, bias=None) -> np.ndarray:
    """L[t, e] = sum_h x[t, h] * W_router[h, e] + bias[e], in float64.

    intelliparadigm.com page, section 2.1: the gate is ``x @ W_gate``."""
    L = np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64)
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float64)[None, :]
    return L


# ---------------------------------------------------------- step 2: top-k selection
def select_experts(logits, k: int):
    """Indices of the k best experts per token, best first (reading R1).

    Sort key per token: (is NaN, -logit, expert index), ascending. Returns
    (idx int32 [T, k], flags) where flags has FLAG_NONFINITE_LOGIT if any logit is not
    finite. gitcode page, "核心代码解析": ``TopKRouting(routing_scores, top_k)``."""
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    nan = np.isnan(L)
    neg = np.where(nan, 0.0, -L)
    ids = np.broadcast_to(np.arange(E), L.shape)
    order = np.lexsort((ids, neg, nan), axis=-1)   # last key is the primary one
    flags = FLAG_NONFINITE_LOGIT if (~np.isfinite(L)).any() else 0
    return order[:, :k].astype(np.int32), flags


def selection_margin(logits, k: int) -> np.ndarray:
    """L_(k) - L_(k+1) per token on the sorted logits (+inf when k == E)."""
    L = np.sort(np.asarray(logits, dtype=np.float64), axis=1)[:, ::-1]
    if k >= L.shape[1]:
        return np.full(L.shape[0], np.inf)
    with np.errstate(invalid="ignore"):   # inf - inf on rows of infinities: NaN, no warning
        return L[:, k - 1] - L[:, k]


# ---------------------------------------------------------------- step 3: weights
def softmax(logits) -> np.ndarray:
    """p[t, e] = exp(L - max) / sum exp(L - max); NaN anywhere in a row gives NaN."""
    L = np.asarray(logits, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m = L.max(axis=1, keepdims=True)
        z = np.exp(L - m)
        return z / z.sum(axis=1, keepdims=True)


def topk_weights(logits, idx, renormalize: bool = True) -> np.ndarray:
    """Gate weights of the selected experts (reading R2), float64 [T, k]."""
    p = softmax(logits)
    sel = np.take_along_axis(p, np.asarray(idx, dtype=np.int64), axis=1)
    if renormalize:
        with np.errstate(invalid="ignore"):
            sel = sel / sel.sum(axis=1, keepdims=True)
    return sel


# ------------------------------------------------- steps 2-3, threshold routing (R14)
def threshold_delta(experts: int, delta=None) -> float:
    """The threshold: delta if given and > 0, else 1/E (intelliparadigm.com page, 3.2.1)."""
    return 1.0 / experts if delta is None or delta <= 0 else float(delta)


def threshold_select(logits, k: int, delta=None):
    """Experts whose gate score p = softmax(L) exceeds delta, best first, at most k per
    token; empty slots are -1 (reading R14). Returns (idx int32 [T, k], flags)."""
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    d = threshold_delta(E, delta)
    order, flags = select_experts(L, E)                        # every expert, best first
    p = np.take_along_axis(softmax(L), order.astype(np.int64), axis=1)
    with np.errstate(invalid="ignore"):
        keep = p > d                                           # NaN scores are never kept
    idx = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        kept = order[t][keep[t]][:k]
        idx[t, :len(kept)] = kept
    return idx, flags


def threshold_weights(logits, idx, renormalize: bool = True) -> np.ndarray:
    """Gate weights of the kept experts (0 in empty slots), float64 [T, k]; renormalised
    over the kept experts when asked (intelliparadigm.com page, 3.2.1)."""
    idx = np.asarray(idx, dtype=np.int64)
    p = softmax(logits)
    sel = np.where(idx >= 0, np.take_along_axis(p, np.maximum(idx, 0), axis=1), 0.0)
    if renormalize:
        s = sel.sum(axis=1, keepdims=True)
        sel = np.divide(sel, s, out=np.zeros_like(sel), where=s > 0)
    return sel


def threshold_margin(logits, delta=None) -> np.ndarray:
    """min over experts of |p - delta| / delta per token (how near a decision is)."""
    L = np.asarray(logits, dtype=np.float64)
    d = threshold_delta(L.shape[1], delta)
    with np.errstate(invalid="ignore"):
        m = np.abs(softmax(L) - d).min(axis=1) / d
    return np.where(np.isnan(m), np.inf, m)


# ------------------------------------------------------------ step 4: capacity rule
def capacity(capacity_factor: float, tokens: int, top_k: int, experts: int) -> int:
    """C = ceil(cf * (T*k) / E) in IEEE double; no limit (C = T) when cf <= 0 (R3)."""
    if capacity_factor <= 0:
        return int(tokens)
    return int(math.ceil((float(capacity_factor) * float(tokens * top_k)) / float(experts)))


def valid_slots(idx, experts: int) -> np.ndarray:
    """True where an expert id is in range and not a repeat of an earlier slot (R6)."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    ok = (idx >= 0) & (idx < experts)
    for j in range(1, k):
        ok[:, j] &= ~(idx[:, :j] == idx[:, j:j + 1]).any(axis=1)
    return ok


def flagged_slots(idx, experts: int) -> np.ndarray:
    """Invalid slots that raise the bad-index flag: every invalid slot except the empty
    marker -1 (R6)."""
    return ~valid_slots(idx, experts) & (np.asarray(idx) != -1)


# ------------------------------------------------------------ steps 4-5: permutation
def permute_indices(idx, experts: int, cap: int) -> dict:
    """Group assignments by expert, in token order, under the capacity rule (R4, R6).

    gitcode page, "核心代码解析": per expert a mask ``expert_ids == i`` selects the tokens
    that ``SparseGather`` packs; gitcode page, "MoE 算子核心原理" section 2: CSR-compressed
    storage (here ``offsets`` + ``row_token``).

    Returns counts (pre-capacity, int32 [E]), kept (int32 [E]), offsets (int32 [E+1]),
    slot_row (int32 [T, k], -1 = dropped/invalid), row_token (int32 [sum kept]), flags."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    ok = valid_slots(idx, experts)
    flags = FLAG_BAD_INDEX if flagged_slots(idx, experts).any() else 0
    flat = np.where(ok, idx, experts).reshape(-1)            # invalid slots sort last
    order = np.argsort(flat, kind="stable")                  # expert-major, then (t, j)
    counts = np.bincount(flat[flat < experts], minlength=experts).astype(np.int64)
    start = np.concatenate([[0], np.cumsum(counts)])
    kept = np.minimum(counts, cap)
    offsets = np.concatenate([[0], np.cumsum(kept)])
    slot_row = np.full(T * k, -1, dtype=np.int64)
    row_token = np.empty(int(offsets[-1]), dtype=np.int64)
    n_valid = int(start[-1])
    sorted_e = flat[order[:n_valid]]
    pos = np.arange(n_valid) - start[sorted_e]               # position inside its expert
    keep = pos < cap
    rows = offsets[sorted_e] + pos
    slot_row[order[:n_valid][keep]] = rows[keep]
    row_token[rows[keep]] = order[:n_valid][keep] // k
    return dict(counts=counts.astype(np.int32), kept=kept.astype(np.int32),
                offsets=offsets.astype(np.int32), slot_row=slot_row.reshape(T, k).astype(np.int32),
                row_token=row_token.astype(np.int32), flags=flags)


def gather_rows(x, row_token) -> np.ndarray:
    """x_perm[row] = x[row_token[row]] (``SparseGather``)."""
    return np.asarray(x)[np.asarray(row_token, dtype=np.int64)]


# ------------------------------------------------------------ steps 6-7: expert FFN
def silu(z):
    return z / (1.0 + np.exp(-z))


def gelu(z):
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def expert_ffn(xr, w_gate_e, w_up_e, w_down_e, activation: str) -> np.ndarray:
    """One expert on a block of rows (reading R5), float64.

    lshu.cn page, section 3: up-projection [hidden -> inter], activation, down-projection."""
    xr = np.asarray(xr, dtype=np.float64)
    wu = np.asarray(w_up_e, dtype=np.float64)
    wd = np.asarray(w_down_e, dtype=np.float64)
    with np.errstate(over="ignore"):
        if activation == "swiglu":
            wg = np.asarray(w_gate_e, dtype=np.float64)
            h = silu(xr @ wg) * (xr @ wu)
        elif activation == "gelu":
            h = gelu(xr @ wu)
        else:
            raise ValueError(activation)
    return h @ wd


def grouped_ffn(x_perm_rows, offsets, w_gate, w_up, w_down, activation: str,
                rows=None) -> np.ndarray:
    """y[row] = FFN_e(x_perm[row]) for the expert e owning each row.

    ``x_perm_rows(rows) -> array`` or an array; weights are indexable per expert.
    ``rows`` restricts the rows computed (others are left as NaN)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    E = len(offsets) - 1
    N = int(offsets[-1])
    want = np.arange(N) if rows is None else np.unique(np.asarray(rows, dtype=np.int64))
    y = None
    for e in range(E):
        r = want[(want >= offsets[e]) & (want < offsets[e + 1])]
        if r.size == 0:
            continue
        xr = x_perm_rows(r) if callable(x_perm_rows) else np.asarray(x_perm_rows)[r]
        ye = expert_ffn(xr, None if w_gate is None else w_gate[e], w_up[e], w_down[e], activation)
        if y is None:
            y = np.full((N, ye.shape[1]), np.nan)
        y[r] = ye
    if y is None:
        y = np.zeros((N, 0))
    return y


# ---------------------------------------------------------------- step 8: combine
def combine(y, slot_row, weights, hidden: int, tokens=None) -> np.ndarray:
    """out[t] = sum_j [slot kept] w[t, j] * y[slot_row[t, j]], j in slot order.

    intelliparadigm.com page, section 2.1 (``sum(results)``); gitcode page,
    ``SparseScatterAdd`` accumulates expert outputs into the dense output."""
    slot_row = np.asarray(slot_row, dtype=np.int64)
    T, k = slot_row.shape
    ts = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = np.zeros((len(ts), hidden))
    for j in range(k):
        r = slot_row[ts, j]
        m = r >= 0
        if m.any():
            out[m] += np.asarray(weights, dtype=np.float64)[ts[m], j][:, None] * y[r[m]]
    return out


# ---------------------------------------------------------------- whole layer
def forward(x, w_router, bias, w_gate, w_up, w_down, *, top_k: int, activation: str,
            capacity_factor: float = 0.0, renormalize: bool = True, tokens=None,
            logits=None, routing: str = "topk", threshold=None) -> dict:
    """The whole layer. ``tokens`` restricts the expert FFN and combine to those tokens
    (routing and the capacity rule always see every token). ``logits`` replaces step 1.
    ``routing`` is "topk" or "threshold" (then ``top_k`` caps the experts per token and
    ``threshold`` is delta, default 1/E)."""
    x = np.asarray(x)
    T, H = x.shape
    L = gate_logits(x, w_router, bias) if logits is None else np.asarray(logits, np.float64)
    E = L.shape[1]
    if routing == "threshold":
        idx, f1 = threshold_select(L, top_k, threshold)
        w = threshold_weights(L, idx, renormalize)
        margin = threshold_margin(L, threshold)
    elif routing == "topk":
        idx, f1 = select_experts(L, top_k)
        w = topk_weights(L, idx, renormalize)
        margin = selection_margin(L, top_k)
    else:
        raise ValueError(routing)
    cap = capacity(capacity_factor, T, top_k, E)
    perm = permute_indices(idx, E, cap)
    ts = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    rows = perm["slot_row"][ts].reshape(-1)
    rows = rows[rows >= 0]
    rt = perm["row_token"]
    y = grouped_ffn(lambda r: x[rt[r]].astype(np.float64), perm["offsets"], w_gate, w_up,
                    w_down, activation, rows=rows)
    if y.shape[1] == 0:
        y = np.zeros((int(perm["offsets"][-1]), H))
    out = combine(y, perm["slot_row"], w, H, tokens=ts)
    return dict(logits=L, topk_idx=idx, topk_w=w, capacity=cap, y=y, out=out, tokens=ts,
                flags=f1 | perm["flags"], margin=margin, **{
                    k_: v for k_, v in perm.items() if k_ != "flags"})


# ---------------------------------------------------------------- backward pass
def silu_grad(z):
    """d/dz of z * logistic(z) = s (1 + z (1 - s)), s = logistic(z)."""
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def gelu_grad(z):
    """d/dz of z * Phi(z) = Phi(z) + z * phi(z)."""
    return 0.5 * (1.0 + _erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def aux_loss(logits, idx, coeff: float) -> dict:
    """Auxiliary load-balancing loss of reading R16 and its gradient with respect to the
    logits, float64: loss = coeff * E * sum_e f_e P_e with f_e = count_e / sum(count) over
    the valid selected slots of ``idx`` (ids in [0, E); -1 and invalid ids do not count) and
    P_e = mean_t softmax(logits)[t, e]. With the counts fixed, dloss/dP_e = coeff E f_e and
    P_e = (1/T) sum_t p[t, e], so dloss/dlogits[t, :] = p[t] (g - <p[t], g>) with
    g = coeff E f / T (the softmax Jacobian)."""
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    ids = np.asarray(idx, dtype=np.int64).ravel()
    ids = ids[(ids >= 0) & (ids < E)]
    counts = np.bincount(ids, minlength=E).astype(np.float64)
    n = counts.sum()
    f = counts / n if n > 0 else np.zeros(E)
    p = softmax(L)
    P = p.sum(axis=0) / T if T > 0 else np.zeros(E)
    loss = float(coeff) * E * float((f * P).sum())
    g = float(coeff) * E * f / T if T > 0 else np.zeros(E)
    dlogits = p * (g[None, :] - (p * g[None, :]).sum(axis=1, keepdims=True))
    return dict(loss=loss, f=f, P=P, counts=counts, dlogits=dlogits)


def backward(x, w_router, bias, w_gate, w_up, w_down, dout, *, top_k: int, activation: str,
             capacity_factor: float = 0.0, renormalize: bool = True, routing: str = "topk",
             threshold=None, logits=None, aux_loss_coeff: float = 0.0) -> dict:
    """Gradients of sum(out * dout) with respect to x, W_router, the gate bias and the expert
    weights, in float64, for the layer of ``forward`` (reading R15: the expert choice is a
    fixed function of the logits, so no gradient flows through the selection itself; the
    weights' dependence on the logits is differentiated exactly).

    The pages compute the backward only for the selected experts' parameters (gitcode
    page, "MoE 算子核心原理": sparse computation runs forward and backward on the chosen
    experts only); every step below is the chain rule of one forward step:
      combine          dy_j = w_j dout,  dw_j = <dout, y_j>
      down-projection  dh = dy Wd^T,     dWd += h^T dy
      activation       SwiGLU: dg = dh u silu'(g), du = dh silu(g); GELU: da = dh gelu'(a)
      up-projection    dWg += x^T dg, dWu += x^T du (da), dx += dg Wg^T + du Wu^T
      weights          renormalised: dp_i = (dw_i - sum_j w_j dw_j) / sum_S p; raw: dp = dw
      softmax          dL = p (dp - sum_e p_e dp_e)
      gate GEMM        dW_router = x^T dL, dbias = sum_t dL, dx += dL W_router^T
    Slots dropped by the capacity rule contribute dw = 0 but stay in the weights' sum.
    ``logits`` replaces the gate GEMM's output (as in ``forward``); the gate GEMM's own
    gradients still use ``x`` and ``w_router``. With ``aux_loss_coeff`` > 0 the objective is
    sum(out * dout) + aux_loss(logits, topk_idx, aux_loss_coeff) (reading R16): its logit
    gradient is added to dL before the gate GEMM's gradients, and its value is returned."""
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    wr = np.asarray(w_router, dtype=np.float64)
    T, H = x.shape
    fwd = forward(x, wr, bias, w_gate, w_up, w_down, top_k=top_k, activation=activation,
                  capacity_factor=capacity_factor, renormalize=renormalize, routing=routing,
                  threshold=threshold, logits=logits)
    L, idx, w = fwd["logits"], np.asarray(fwd["topk_idx"], np.int64), fwd["topk_w"]
    slot_row, offsets, row_token = fwd["slot_row"], fwd["offsets"], fwd["row_token"]
    E = L.shape[1]
    dx = np.zeros_like(x)
    dWg = None if w_gate is None else [None] * E
    dWu, dWd = [None] * E, [None] * E
    dw = np.zeros_like(w)
    row_t = np.full(int(offsets[-1]), -1, dtype=np.int64)    # row -> (token, slot)
    row_j = np.full(int(offsets[-1]), -1, dtype=np.int64)
    t_k, j_k = np.nonzero(slot_row >= 0)
    row_t[slot_row[t_k, j_k]] = t_k
    row_j[slot_row[t_k, j_k]] = j_k
    for e in range(E):
        wu = np.asarray(w_up[e], dtype=np.float64)
        wd = np.asarray(w_down[e], dtype=np.float64)
        wg = None if w_gate is None else np.asarray(w_gate[e], dtype=np.float64)
        rows = np.arange(offsets[e], offsets[e + 1])
        toks = row_token[rows].astype(np.int64)
        t_of, j_of = row_t[rows], row_j[rows]
        xe = x[toks]
        if activation == "swiglu":
            g, u = xe @ wg, xe @ wu
            h = silu(g) * u
        else:
            a = xe @ wu
            h = gelu(a)
        y = h @ wd
        de = dout[toks]
        dw[t_of, j_of] = (de * y).sum(axis=1)
        dy = w[t_of, j_of][:, None] * de
        dh = dy @ wd.T
        dWd[e] = h.T @ dy
        if activation == "swiglu":
            dg = dh * u * silu_grad(g)
            du = dh * silu(g)
            dWg[e] = xe.T @ dg
            dWu[e] = xe.T @ du
            dxe = dg @ wg.T + du @ wu.T
        else:
            da = dh * gelu_grad(a)
            dWu[e] = xe.T @ da
            dxe = da @ wu.T
        np.add.at(dx, toks, dxe)
    # gate weights -> scores -> logits
    p = softmax(L)
    kept = idx >= 0
    psel = np.where(kept, np.take_along_axis(p, np.maximum(idx, 0), axis=1), 0.0)
    if renormalize:
        s = psel.sum(axis=1, keepdims=True)
        dps = np.divide(dw - (w * dw).sum(axis=1, keepdims=True), s,
                        out=np.zeros_like(dw), where=s > 0)
    else:
        dps = dw
    dp = np.zeros_like(p)
    for j in range(idx.shape[1]):
        m = kept[:, j]
        dp[np.nonzero(m)[0], idx[m, j]] += dps[m, j]
    dL = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    aux = None
    if aux_loss_coeff > 0:
        aux = aux_loss(L, idx, aux_loss_coeff)
        dL = dL + aux["dlogits"]
    dx += dL @ wr.T
    return dict(dx=dx, dw_router=x.T @ dL, dbias=dL.sum(axis=0), dw_gate=dWg, dw_up=dWu,
                dw_down=dWd, dlogits=dL, dw=dw, forward=fwd,
                aux_loss=None if aux is None else aux["loss"])
